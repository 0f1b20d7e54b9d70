// kda_common.h -- device helpers shared by the KDA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
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

// Load one input element of type T (float or raw bf16 bits) as fp32.
template <typename T> __device__ __forceinline__ float load_in(const T *p);
template <> __device__ __forceinline__ float load_in<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p) {
    return bf16_bits_to_f32(*p);
}

// ---- wave-level helpers ---------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

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
