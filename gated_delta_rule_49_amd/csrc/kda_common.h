// kda_common.h -- device helpers shared by the KDA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace kda {

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float lo_bf16_of(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float hi_bf16_of(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ uint16_t bf16_raw(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_hl(float x, __bf16 &hi, __bf16 &lo) {
    hi = to_bf16(x);
    lo = to_bf16(x - bf16_to_f32(hi));
}

typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (round to nearest even) packed in one word, a at the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){a, b}, bf16x2v_t));
}
// hi/lo split of a pair, packed: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_hl2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Load one input element of type T (float or raw bf16 bits) as fp32.
template <typename T> __device__ __forceinline__ float load_in(const T *p);
template <> __device__ __forceinline__ float load_in<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p) {
    return bf16_bits_to_f32(*p);
}

// Widen one input element (raw bf16 bits or fp32) already held in a register.
__device__ __forceinline__ float widen(uint16_t b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ float widen(float x) { return x; }

// ---- register-pressure control -------------------------------------------------
// Return x unchanged while hiding its value from the optimizer.  Values derived
// from the result are recomputed inside a loop body instead of being hoisted
// out of the loop and kept live in registers for its whole duration (per-lane
// LDS offsets are cheap to recompute and expensive to hold).  The asm emits no
// instruction.
__device__ __forceinline__ int opaque_v(int x) { __asm__ volatile("" : "+v"(x)); return x; }
__device__ __forceinline__ int opaque_s(int x) { __asm__ volatile("" : "+s"(x)); return x; }
// Lane index 0..63, recomputed where it is called (v_mbcnt): unlike threadIdx.x & 63 it needs no
// register kept live across a loop, and the opaque mask keeps it from being hoisted.
__device__ __forceinline__ int lane_id() {
    const unsigned m = (unsigned)opaque_s(-1);
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

// ---- wave-level helpers ---------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
// v from another lane of the same 16-lane row, by a DPP control (e.g. 0x121..0x12F: row_ror:1..15)
template <int CTRL> __device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Fused prologue of the chunked prefill (bits of ChunkParams::flags).
constexpr int KDA_PRO_GATE = 1;   // g holds bf16 pre-activations a (g = -5 sigmoid(a)), beta fp32 b (sigmoid(b))
constexpr int KDA_PRO_NORM = 2;   // q and k are L2-normalised per (token, head) over d_k
// Internal (the backward's recompute of the chunk-start states): o is neither formed nor written,
// and q is not read.
constexpr int KDA_STATES_ONLY = 4;
// (KDA_BWD_STATES_GIVEN = 8 and KDA_BWD_ONE_WG_SCAN = 32, the backward's own launch flags, are in
// kda_bwd_flags.h.)
// Internal (the forward cut into segments; one workgroup per run): the grid covers twice the
// launch's (segment, head) chains, and each chain runs twice, on one XCD.  "Kind 0" runs with its
// v from the initial state that s0_idx names (a sequence's first segment: its slot, -1 zeros;
// later segments: -2, zeros): outputs to o, checkpoints as usual, final state N.  "Kind 1" runs
// with v taken as zero from the identity (d_k = d_v), for later segments only (s0_idx -2): its
// final state is the segment's transition matrix M = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t),
// its outputs scale M_t^T q_t go to o_tr and its checkpoints (the partial products) to ckpt_tr.
// Final states go to sf[(kind * nseq + n) * H + h].  s0_idx is always set.
constexpr int KDA_TRANSITION = 16;

// ---- MFMA ------------------------------------------------------------------
// 16x16 output tiles: lane l holds D[4*(l/16) + e][l % 16], e = 0..3.
// A operand: lane l supplies row l % 16; B operand: lane l supplies column l % 16.
// Both use the same k for the same (lane group q = l/16, element slot), so any
// fixed assignment of k-indices to (q, slot) pairs is a valid contraction order.
__device__ __forceinline__ f32x4_t mfma_bf16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace kda

// Compute units of the current device (host side; queried once per device).
inline int kda_cu_count() {
    // per device, filled on first use; concurrent first calls store the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (!cus) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}
