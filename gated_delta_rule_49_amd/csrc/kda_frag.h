// kda_frag.h -- MFMA operand layout and precision policies shared by the chunk kernels.
#pragma once
#include "kda_common.h"

namespace kda {

constexpr int SUB = 16;   // sub-chunk size (rows of one MFMA tile)
constexpr int TP = 20;    // row pitch (floats) of the fp32 16x16 tiles used by the inverse
constexpr int TSZ = 16 * TP;

// ---- fragment-major LDS operand layout ---------------------------------------
// A matrix with R rows and K contraction columns is stored in blocks of 16 rows
// x 32 columns; inside a block, the 8 values lane l feeds to one MFMA K-step
// are contiguous (16 B as bf16, 32 B as fp32) so a fragment is one wide read.
// Column k of a block maps to (lane group q, slot e):
//     k%32 <  16 : q = (k%16)/4, e = k%4          k%32 >= 16 : q = (k%16)/4, e = 4 + k%4
// which is also the row order of a pair of 16x16 MFMA output tiles, so an
// output pair can be fed back as an operand straight from registers.
// Inside a block, the 16 fragments of lane group q are permuted by XOR with
// (q + 4 kb + rb): any such permutation keeps the 16-byte fragment reads
// conflict-free, and this one spreads the 4-byte writes of one row across all
// 32 banks, and the writes of one column across 8 fragment slots.
__device__ __forceinline__ int frag_slot(int rr, int q, int kb, int rb) {
    return 16 * q + (rr ^ ((q + 4 * kb + rb) & 15));
}

template <int KB>
__device__ __forceinline__ int fofs(int r, int k) {
    const int rb = r >> 4, rr = r & 15, kb = k >> 5, kk = k & 31;
    const int q = (kk & 15) >> 2, e = (kk & 3) | ((kk >> 4) << 2);
    return ((rb * KB + kb) * 64 + frag_slot(rr, q, kb, rb)) * 8 + e;
}
template <int KB>
__device__ __forceinline__ int fbase(int rb, int kb, int lane) {
    return ((rb * KB + kb) * 64 + frag_slot(lane & 15, lane >> 4, kb, rb)) * 8;
}
// 64x64 lower-block-triangular matrices (T, A_qk): only blocks (rb, kb <= rb/2) exist.
__device__ __forceinline__ int tri_block(int rb, int kb) { return rb < 2 ? rb : 2 + 2 * (rb - 2) + kb; }
__device__ __forceinline__ int tofs(int r, int k) {
    const int rb = r >> 4, rr = r & 15, kb = k >> 5, kk = k & 31;
    const int q = (kk & 15) >> 2, e = (kk & 3) | ((kk >> 4) << 2);
    return (tri_block(rb, kb) * 64 + frag_slot(rr, q, kb, rb)) * 8 + e;
}
__device__ __forceinline__ int tbase(int rb, int kb, int lane) {
    return (tri_block(rb, kb) * 64 + frag_slot(lane & 15, lane >> 4, kb, rb)) * 8;
}

// ---- precision policies -------------------------------------------------------
template <bool F32P> struct Frag;
template <> struct Frag<false> { bf16x8_t hi, lo; };
template <> struct Frag<true> { float v[8]; };

// Matrix storage: "HL" = value carried at ~16 bits (bf16 hi + lo planes, or fp32),
// "H" = single precision carrier (one bf16 plane, or fp32).
template <bool F32P> struct Mat;
template <> struct Mat<false> {
    static constexpr int ES = 2;  // element bytes per plane
    template <int N> __device__ static void put_hl(char *base, int plane_bytes, int off, const float (&x)[N]) {
        // the lo plane's address is taken from the hi one, so that a constant plane distance
        // folds into the LDS instruction's offset field instead of costing an address add
        __bf16 *hi = reinterpret_cast<__bf16 *>(base) + off;
        __bf16 *lo = reinterpret_cast<__bf16 *>(reinterpret_cast<char *>(hi) + plane_bytes);
        if constexpr (N == 2) {
            uint32_t H, Lw;
            split_hl2(x[0], x[1], H, Lw);
            *reinterpret_cast<uint32_t *>(hi) = H;
            *reinterpret_cast<uint32_t *>(lo) = Lw;
        } else if constexpr (N == 4) {
            uint2 H, Lw;
            split_hl2(x[0], x[1], H.x, Lw.x);
            split_hl2(x[2], x[3], H.y, Lw.y);
            *reinterpret_cast<uint2 *>(hi) = H;
            *reinterpret_cast<uint2 *>(lo) = Lw;
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) split_hl(x[i], hi[i], lo[i]);
        }
    }
    __device__ static void put_hl1(char *base, int plane_bytes, int off, float x) {
        __bf16 h, l;
        split_hl(x, h, l);
        reinterpret_cast<__bf16 *>(base)[off] = h;
        reinterpret_cast<__bf16 *>(base + plane_bytes)[off] = l;
    }
    __device__ static void put_h2(char *base, int off, float x0, float x1) {
        *reinterpret_cast<uint32_t *>(reinterpret_cast<__bf16 *>(base) + off) = pack_bf16x2(x0, x1);
    }
    template <bool LO> __device__ static Frag<false> get(const char *base, int plane_bytes, int off) {
        Frag<false> f;
        const __bf16 *hp = reinterpret_cast<const __bf16 *>(base) + off;
        f.hi = *reinterpret_cast<const bf16x8_t *>(hp);
        if constexpr (LO) f.lo = *reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const char *>(hp) + plane_bytes);
        return f;
    }
    // Operand fragment from two 16x16 output tiles covering contraction rows
    // [32s, 32s+16) and [32s+16, 32s+32) (hi only, or hi+lo).
    template <bool LO> __device__ static Frag<false> from_tiles(const f32x4_t &t0, const f32x4_t &t1) {
        uint32_t h[4], l[4];
        if constexpr (LO) {
            split_hl2(t0[0], t0[1], h[0], l[0]);
            split_hl2(t0[2], t0[3], h[1], l[1]);
            split_hl2(t1[0], t1[1], h[2], l[2]);
            split_hl2(t1[2], t1[3], h[3], l[3]);
        } else {
            h[0] = pack_bf16x2(t0[0], t0[1]);
            h[1] = pack_bf16x2(t0[2], t0[3]);
            h[2] = pack_bf16x2(t1[0], t1[1]);
            h[3] = pack_bf16x2(t1[2], t1[3]);
        }
        Frag<false> f;
        f.hi = __builtin_bit_cast(bf16x8_t, (uint4){h[0], h[1], h[2], h[3]});
        if constexpr (LO) f.lo = __builtin_bit_cast(bf16x8_t, (uint4){l[0], l[1], l[2], l[3]});
        return f;
    }
    // Fragment from two tiles with a per-element scale (one factor per slot).
    template <bool LO> __device__ static Frag<false> from_tiles_scaled(const f32x4_t &t0, const f32x4_t &t1,
                                                                     const float (&sc)[8]) {
        f32x4_t a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = t0[e] * sc[e]; b[e] = t1[e] * sc[4 + e]; }
        return from_tiles<LO>(a, b);
    }
};
template <> struct Mat<true> {
    static constexpr int ES = 4;
    template <int N> __device__ static void put_hl(char *base, int, int off, const float (&x)[N]) {
        float *p = reinterpret_cast<float *>(base) + off;
        if constexpr (N == 2) *reinterpret_cast<float2 *>(p) = make_float2(x[0], x[1]);
        else if constexpr (N == 4) *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
        else {
#pragma unroll
            for (int i = 0; i < N; ++i) p[i] = x[i];
        }
    }
    __device__ static void put_hl1(char *base, int, int off, float x) { reinterpret_cast<float *>(base)[off] = x; }
    __device__ static void put_h2(char *base, int off, float x0, float x1) {
        *reinterpret_cast<float2 *>(reinterpret_cast<float *>(base) + off) = make_float2(x0, x1);
    }
    template <bool LO> __device__ static Frag<true> get(const char *base, int, int off) {
        Frag<true> f;
        const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off);
        const float4 b = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off + 4);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
        return f;
    }
    template <bool LO> __device__ static Frag<true> from_tiles(const f32x4_t &t0, const f32x4_t &t1) {
        Frag<true> f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f.v[e] = t0[e]; f.v[4 + e] = t1[e]; }
        return f;
    }
    template <bool LO> __device__ static Frag<true> from_tiles_scaled(const f32x4_t &t0, const f32x4_t &t1,
                                                                    const float (&sc)[8]) {
        Frag<true> f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f.v[e] = t0[e] * sc[e]; f.v[4 + e] = t1[e] * sc[4 + e]; }
        return f;
    }
};

// acc += A * B over one 32-wide K-step.  bf16: hi*hi (+ lo*hi) (+ hi*lo).
template <bool ALO, bool BLO>
__device__ __forceinline__ void mma(f32x4_t &acc, const Frag<false> &a, const Frag<false> &b) {
    if constexpr (ALO) acc = mfma_bf16(a.lo, b.hi, acc);
    if constexpr (BLO) acc = mfma_bf16(a.hi, b.lo, acc);
    acc = mfma_bf16(a.hi, b.hi, acc);
}
template <bool ALO, bool BLO>
__device__ __forceinline__ void mma(f32x4_t &acc, const Frag<true> &a, const Frag<true> &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = mfma_f32(a.v[e], b.v[e], acc);
}

// ---- fp32 16x16 tile products for the triangular inverse ------------------------
// Tiles are row-major [16][TP] fp32 in LDS.  In instruction kk lane l feeds
// k = 4*(l/16) + kk, which matches the row order of an output tile held in
// registers (element kk of lane l is row 4*(l/16) + kk).
__device__ __forceinline__ void tmm_ll(f32x4_t &acc, const float *A, const float *B, int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(A[r * TP + 4 * q + kk], B[(4 * q + kk) * TP + r], acc);
}
__device__ __forceinline__ void tmm_lr(f32x4_t &acc, const float *A, const f32x4_t &R, int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(A[r * TP + 4 * q + kk], R[kk], acc);
}
__device__ __forceinline__ void tile_store(float *Tl, const f32x4_t &v, int lane) {
    const int c = lane & 15, q = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Tl[(4 * q + e) * TP + c] = v[e];
}

__host__ __device__ constexpr int vidx(int a, int b) { return a * (a + 1) / 2 + b; }


// Arguments of the chunked-prefill kernels (device pointers; see include/kda.h).
struct ChunkParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    const int32_t *order;          // sequences, longest first
    const int64_t *ckpt_base;      // per sequence: index of its first checkpoint
    const float *s0;
    float *sf;
    float *ckpt;
    float *o;
    const int32_t *s0_idx;         // NULL, or the pool slot of each sequence's initial state (-1: zeros)
    const int32_t *ck_idx;         // NULL, or the pool slot of each checkpoint (-1: not written)
    int nslots;                    // slots of the checkpoint pool (ck_idx set)
    int s0_slots;                  // slots of the initial-state pool (s0_idx set)
    int flags;                     // KDA_PRO_GATE: g, beta are pre-activations; KDA_PRO_NORM: normalise q, k
    int H;
    int every;
    float scale;
    int nseq;                      // sequences of this launch (the paired segment pass indexes its states by it)
    float *o_tr;                   // the paired segment pass: outputs of the transition runs, [T, H, dk]
    float *ckpt_tr;                // the paired segment pass: their checkpoints, dense [M, H, dk, dk]
    // states-only runs: when set, R = V - (Gamma K) S of every chunk, [32][dv] fp32 (zero rows past
    // a sequence's end), at rres + ((rbase[n] + chunk) H + h) rstride
    float *rres = nullptr;
    const int32_t *rbase = nullptr;
    long long rstride = 0;
};

// Element offset of the initial state of (n, h) in p.s0, or -1 for a zero state (no initial
// state, or a pool index of -1 or out of range).
__device__ __forceinline__ long long s0_offset(const ChunkParams &p, int n, int h, int dkdv) {
    if (!p.s0) return -1;
    long long slot = n;
    if (p.s0_idx) {
        const int s = p.s0_idx[n];
        if (s < 0 || s >= p.s0_slots) return -1;
        slot = s;
    }
    return (slot * p.H + h) * dkdv;
}
// Destination of checkpoint m of head h, or NULL when it is not written (pool index -1 or out of
// range).
__device__ __forceinline__ float *ckpt_dst(const ChunkParams &p, int64_t m, int h, int dkdv) {
    int64_t slot = m;
    if (p.ck_idx) {
        const int s = p.ck_idx[m];
        if (s < 0 || s >= p.nslots) return nullptr;
        slot = s;
    }
    return p.ckpt + (slot * p.H + h) * dkdv;
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads
// (prefetches into registers) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order a wave's own LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

}  // namespace kda
