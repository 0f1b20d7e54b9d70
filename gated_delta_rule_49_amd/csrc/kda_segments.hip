// kda_segments.hip -- the chunked forward of few, long (sequence, head) chains, each cut into
// segments that run side by side (context parallelism inside one GPU).
//
// Over a segment the recurrence is affine in the state it starts from: S_t = M_t S_in + N_t, where
// M_t is the product of the tokens' (I - beta k k^T) Diag(alpha) up to t and N_t the state reached
// from a zero start, and so o_t = scale S_t^T q_t = o0_t + S_in^T (scale M_t^T q_t).  Only the
// fixed-size state has to cross a segment boundary (the t.iss.one DNSPODT digest of the K3 report,
// infrastructure paragraph: KDA's context parallelism exchanges only the fixed-size recurrent
// state).  Four launches:
//   1. plan: the segment list (cut every `seg` tokens from each sequence's start);
//   2. every segment runs twice at once (kda_chunk32.hip, KDA_TRANSITION): from zero with its v
//      (o0 into o, N_t into the checkpoints, N as final state) and, for every segment but a
//      sequence's first, with v = 0 from the identity (scale M_t^T q_t, M_t, M).  A first segment
//      starts from the sequence's initial state instead, so its outputs are final at once;
//   3. chain, per (sequence, head, 16 value columns): S_in(1) = N_0, S_in(p + 1) = M_p S_in(p) + N_p,
//      each later segment's checkpoints corrected by M_t S_in(p), and the final state written;
//   4. correction of the outputs of every later segment: o_t += S_in^T (scale M_t^T q_t).
// Segments are cut at multiples of `seg` tokens, seg a multiple of the chunk (32) and of
// checkpoint_every, so that chunks and checkpoints fall where they fall without the cut.
#include "kda_frag.h"

namespace kda {

// Segment list.  Sequence n has P_n = max(1, ceil(L_n / seg)) segments b_n .. b_n + P_n - 1 (an
// empty sequence keeps one empty segment).  Segment s = b_n + p: cuB[s] = cu[n] + p seg (cuB[NB] =
// cu[N]), order[s] = s, ckb[s] its first checkpoint's index, s0map[s] the initial-state slot of a
// first segment (-1: zeros) or -2 (a later segment).  info[2 n] = b_n, info[2 n + 1] = P_n.  NB, the
// host's count from its copy of the offsets, bounds every write (offsets that disagree with that
// copy give wrong results, never a write outside the arrays).  One workgroup of 1024.
__global__ void __launch_bounds__(1024)
segment_plan_kernel(const int32_t *__restrict__ cu, int N, int seg, int every, int NB, const float *s0,
                    const int32_t *__restrict__ s0_idx, int s0_slots, int32_t *__restrict__ cuB,
                    int32_t *__restrict__ info, int32_t *__restrict__ order, int64_t *__restrict__ ckb,
                    int32_t *__restrict__ s0map) {
    __shared__ int32_t partP[1024];
    __shared__ int64_t partC[1024];
    __shared__ int32_t carryP;
    __shared__ int64_t carryC;
    const int tid = (int)threadIdx.x;
    for (int s = tid; s < NB; s += blockDim.x) {   // defaults: empty first segments
        cuB[s] = cu[N];
        order[s] = s;
        ckb[s] = 0;
        s0map[s] = -1;
    }
    if (tid == 0) {
        carryP = 0;
        carryC = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += blockDim.x) {
        const int n = base + tid;
        int P = 0, start = 0, L = 0;
        int64_t C = 0;
        if (n < N) {
            start = cu[n];
            L = cu[n + 1] - start;
            P = L > 0 ? (L + seg - 1) / seg : 1;
            C = every > 0 ? L / every : 0;
        }
        partP[tid] = P;
        partC[tid] = C;
        __syncthreads();
        for (int off = 1; off < (int)blockDim.x; off <<= 1) {   // inclusive scans of P and C
            const int xp = tid >= off ? partP[tid - off] : 0;
            const int64_t xc = tid >= off ? partC[tid - off] : 0;
            __syncthreads();
            partP[tid] += xp;
            partC[tid] += xc;
            __syncthreads();
        }
        if (n < N) {
            const int b = min(carryP + partP[tid] - P, NB);
            const int Pc = min(P, NB - b);
            const int64_t cb = carryC + partC[tid] - C;
            int slot = -1;
            if (s0) {
                slot = n;
                if (s0_idx) {
                    slot = s0_idx[n];
                    if (slot < 0 || slot >= s0_slots) slot = -1;
                }
            }
            info[2 * n] = b;
            info[2 * n + 1] = Pc;
            for (int p = 0; p < Pc; ++p) {
                cuB[b + p] = start + p * seg;
                ckb[b + p] = cb + (every > 0 ? (int64_t)p * (seg / every) : 0);
                s0map[b + p] = p == 0 ? slot : -2;
            }
        }
        __syncthreads();
        if (tid == (int)blockDim.x - 1) {
            carryP += partP[tid];
            carryC += partC[tid];
        }
        __syncthreads();
    }
    if (tid == 0) cuB[NB] = cu[N];
}

// The chain's products on one 16-row x 16-column tile (wave w: rows 16 w .., the workgroup's 16
// columns): A[16 w .. 16 w + 15, :] S[:, cols] + c, with A's row slice already in registers, S in
// LDS.  fp32 MFMA 16x16x4; lane (lr, lq) holds k = KQ lq + kk (KQ = d / 4): KQ adjacent floats of
// A's row 16 w + lr.  S row k sits at LDS row 4 (k % KQ) + k / KQ, which puts the four lane groups
// of each B read on distinct banks.
template <int D>
__device__ __forceinline__ void chain_load_a(const float *__restrict__ A, int w, int lr, int lq, float (&a)[D / 4]) {
    const float4 *ar = reinterpret_cast<const float4 *>(A + (size_t)(16 * w + lr) * D + (D / 4) * lq);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
        const float4 x = ar[i];
        a[4 * i] = x.x; a[4 * i + 1] = x.y; a[4 * i + 2] = x.z; a[4 * i + 3] = x.w;
    }
}
template <int D>
__device__ __forceinline__ f32x4_t chain_mma(const float (&a)[D / 4], const float *S, f32x4_t c, int lr, int lq) {
    f32x4_t d = {0.f, 0.f, 0.f, 0.f};   // two accumulation chains: half the dependent latency
#pragma unroll
    for (int kk = 0; kk < D / 4; kk += 2) {
        c = mfma_f32(a[kk], S[(4 * kk + lq) * 16 + lr], c);
        d = mfma_f32(a[kk + 1], S[(4 * kk + 4 + lq) * 16 + lr], d);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] += d[e];
    return c;
}
// S_in as the correction reads it: S^T split into bf16 hi and lo planes, [column][k] with rows
// padded to D + 8 (per segment and head: [2][D][D + 8] bf16, as many bytes as fp32 S plus the pad).
template <int D> constexpr int sin_pitch() { return D + 8; }
template <int D> constexpr size_t sin_elems() { return (size_t)2 * D * sin_pitch<D>(); }

template <int D>
__device__ __forceinline__ int chain_lds_row(int r) {
    return 4 * (r % (D / 4)) + r / (D / 4);
}

// The chain along each sequence's segments, for one (sequence, head) and 16 value columns per
// workgroup (D / 16 waves, one 16-row tile each).  st: [2][NB][H][D][D] (kind 0: N, kind 1: M).
// Writes S_in of every later segment to sin_ ([NB][H] x sin_elems, the correction's layout), corrects its checkpoints
// (ckpt[m] += M_m S_in, M_m from ckI, dense [M][H][D][D]) and writes the final state.  The next
// step's M and N are loaded while the current step's products run.
template <int D>
__global__ void __launch_bounds__(512)
segment_chain_kernel(const int32_t *__restrict__ info, const int32_t *__restrict__ cuB,
                     const int64_t *__restrict__ ckb, int H, int NB, int every, const float *__restrict__ st,
                     __bf16 *__restrict__ sin_, float *sf, float *ckpt, const int32_t *__restrict__ ck_idx,
                     int nslots, const float *__restrict__ ckI) {
    __shared__ __attribute__((aligned(16))) float S[D * 16];
    constexpr int CB = D / 16;
    const int c0 = 16 * ((int)blockIdx.x % CB), nh = (int)blockIdx.x / CB;
    const int n = nh / H, h = nh % H;
    const int b = info[2 * n], P = info[2 * n + 1];
    if (P == 0) return;   // only when the offsets disagree with the host's copy
    const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const bool act = w < D / 16;
    const size_t per = (size_t)D * D;
    const size_t tile = (size_t)(16 * w + 4 * lq) * D + c0 + lr;   // element (row 16 w + 4 lq + e: + e D)
    auto mat = [&](int kind, int sg) { return st + ((size_t)(kind * NB + sg) * H + h) * per; };
    f32x4_t s = {0.f, 0.f, 0.f, 0.f}, nx = s;
    float a[D / 4];
    if (act) {
        const float *n0 = mat(0, b) + tile;   // N of the first segment (from the sequence's initial state)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = n0[e * D];
        if (P > 1) {
            chain_load_a<D>(mat(1, b + 1), w, lr, lq, a);
#pragma unroll
            for (int e = 0; e < 4; ++e) nx[e] = mat(0, b + 1)[tile + e * D];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) S[chain_lds_row<D>(16 * w + 4 * lq + e) * 16 + lr] = s[e];
    }
    __syncthreads();
    for (int p = 1; p < P; ++p) {
        const int sg = b + p;
        f32x4_t next = s;
        if (act) {
            {   // rows 16 w + 4 lq .. + 3 of column c0 + lr: 4 adjacent k of S^T, hi and lo
                __bf16 *si = sin_ + ((size_t)sg * H + h) * sin_elems<D>() + (size_t)(c0 + lr) * sin_pitch<D>() +
                             16 * w + 4 * lq;
                __attribute__((ext_vector_type(4))) __bf16 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = (__bf16)s[e];
                    lo[e] = (__bf16)(s[e] - (float)hi[e]);
                }
                *reinterpret_cast<decltype(hi) *>(si) = hi;
                *reinterpret_cast<decltype(lo) *>(si + (size_t)D * sin_pitch<D>()) = lo;
            }
            if (every > 0) {
                const int nck = (cuB[sg + 1] - cuB[sg]) / every;
                for (int j = 0; j < nck; ++j) {
                    const int64_t m = ckb[sg] + j;
                    float *dst = nullptr;
                    if (ck_idx) {
                        const int slot = ck_idx[m];
                        if (slot >= 0 && slot < nslots) dst = ckpt + ((size_t)slot * H + h) * per;
                    } else {
                        dst = ckpt + ((size_t)m * H + h) * per;
                    }
                    if (!dst) continue;
                    float am[D / 4];
                    chain_load_a<D>(ckI + ((size_t)m * H + h) * per, w, lr, lq, am);
                    f32x4_t c;
#pragma unroll
                    for (int e = 0; e < 4; ++e) c[e] = dst[tile + e * D];
                    c = chain_mma<D>(am, S, c, lr, lq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[tile + e * D] = c[e];
                }
            }
            float an[D / 4];
            f32x4_t nn = nx;
            if (p + 1 < P) {   // the next step's operands, in flight during this step's products
                chain_load_a<D>(mat(1, sg + 1), w, lr, lq, an);
#pragma unroll
                for (int e = 0; e < 4; ++e) nn[e] = mat(0, sg + 1)[tile + e * D];
            }
            next = chain_mma<D>(a, S, nx, lr, lq);
            if (p + 1 < P) {
#pragma unroll
                for (int i = 0; i < D / 4; ++i) a[i] = an[i];
                nx = nn;
            }
        }
        __syncthreads();   // every wave has read S
        if (act) {
            s = next;
#pragma unroll
            for (int e = 0; e < 4; ++e) S[chain_lds_row<D>(16 * w + 4 * lq + e) * 16 + lr] = s[e];
        }
        __syncthreads();
    }
    if (sf && act) {
        float *d = sf + ((size_t)n * H + h) * per + tile;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e * D] = s[e];
    }
}

// Output correction of the later segments: o_t += S_in^T r_t, r_t = scale M_t^T q_t (the transition
// runs' outputs, oI [T][H][D]).  Workgroup (segment s, tile group jg, head h): TPW consecutive tiles
// of 16 NW tokens from cuB[s] + 16 NW TPW jg, wave w of NW taking 16 tokens of each tile.  S_in is
// staged once per workgroup; each tile's rows of oI (and, with PO, of o) load while the previous
// tile's products run.  The product is formed transposed, out[c][t] = sum_k S[k][c] r_t[k]
// (S_in^T from LDS as the A operand, r_t as the B operand), so that each lane ends up with 4
// adjacent columns of one token: o moves as 16-byte vectors.  bf16 MFMA 16x16x32 in three terms
// (hi hi + hi lo + lo hi, each operand split as x = hi + lo): about 16 significant bits, the fp32
// bar's precision.  S_in sits in LDS transposed, [column][k], hi and lo planes, rows padded to
// D + 8 (the 16 lanes of an operand read then start 4 banks apart).
constexpr int CORR_WAVES = 8;   // waves (16 tokens each) of a correction workgroup
template <int D, int NW, int TPW, bool PO>
__global__ void __launch_bounds__(64 * NW)
segment_correct_kernel(const int32_t *__restrict__ cuB, const int32_t *__restrict__ s0map, int H, int groups,
                       const __bf16 *__restrict__ sin_, const float *__restrict__ oI, float *__restrict__ o) {
    constexpr int KP = D + 8, KS = D / 32, CT = D / 16, TT = 16 * NW;
    static_assert(KP == sin_pitch<D>(), "LDS rows as stored");
    constexpr int NV = (int)(sin_elems<D>() * 2 / 16);   // 16-byte vectors of S_in
    constexpr int VEC = (NV + 64 * NW - 1) / (64 * NW);
    __shared__ __attribute__((aligned(16))) __bf16 SH[2 * D * KP];   // hi plane, then lo plane
    __bf16 *const SL = SH + D * KP;
    const int s = (int)blockIdx.x / groups, jg = (int)blockIdx.x % groups, h = (int)blockIdx.y;
    if (s0map[s] != -2) return;   // a first segment: its outputs are final
    const int seg_end = cuB[s + 1], t_first = cuB[s] + TT * TPW * jg;
    if (t_first >= seg_end) return;
    const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    // this lane's token of tile i, and its rows: r_t as B operands (k = 32 ks + 8 lq .. + 7),
    // o_t[16 ct + 4 lq .. + 3] as the addends
    auto token = [&](int i) { return t_first + TT * i + 16 * w + lr; };
    auto load_r = [&](int i, float (&x)[KS][8]) {
        const int t = token(i);
        const size_t row = ((size_t)t * H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float4 u = make_float4(0.f, 0.f, 0.f, 0.f), v = u;
            if (t < seg_end) {
                const float4 *src = reinterpret_cast<const float4 *>(oI + row + 32 * ks + 8 * lq);
                u = src[0];
                v = src[1];
            }
            x[ks][0] = u.x; x[ks][1] = u.y; x[ks][2] = u.z; x[ks][3] = u.w;
            x[ks][4] = v.x; x[ks][5] = v.y; x[ks][6] = v.z; x[ks][7] = v.w;
        }
    };
    auto load_o = [&](int i, f32x4_t (&a)[CT]) {
        const int t = token(i);
        const size_t row = ((size_t)t * H + h) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < seg_end) y = *reinterpret_cast<const float4 *>(o + row + 16 * ct + 4 * lq);
            a[ct][0] = y.x; a[ct][1] = y.y; a[ct][2] = y.z; a[ct][3] = y.w;
        }
    };
    float x[KS][8], xn[KS][8];
    f32x4_t acc[CT], accn[CT];
    load_r(0, x);
    load_o(0, acc);
    {   // S_in (already split and transposed) -> LDS: a straight copy of 16-byte vectors
        const uint4 *src = reinterpret_cast<const uint4 *>(sin_ + ((size_t)s * H + h) * sin_elems<D>());
        uint4 *dst = reinterpret_cast<uint4 *>(SH);
        uint4 y[VEC];
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
            const int i = (int)threadIdx.x + 64 * NW * q;
            y[q] = i < NV ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
            const int i = (int)threadIdx.x + 64 * NW * q;
            if (i < NV) dst[i] = y[q];
        }
    }
    __syncthreads();
    for (int i = 0; i < TPW; ++i) {
        if (t_first + TT * i >= seg_end) break;   // (uniform)
        const bool more = i + 1 < TPW && t_first + TT * (i + 1) < seg_end;
        if (more) {
            load_r(i + 1, xn);
            if constexpr (PO) load_o(i + 1, accn);
        }
        bf16x8_t bh[KS], bl[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bh[ks][e] = (__bf16)x[ks][e];
                bl[ks][e] = (__bf16)(x[ks][e] - (float)bh[ks][e]);
            }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = (16 * ct + lr) * KP + 32 * ks + 8 * lq;
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&SH[off]);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(&SL[off]);
                acc[ct] = mfma_bf16(al, bh[ks], acc[ct]);
                acc[ct] = mfma_bf16(ah, bl[ks], acc[ct]);
                acc[ct] = mfma_bf16(ah, bh[ks], acc[ct]);
            }
        }
        // lane (lr, lq) holds out[16 ct + 4 lq + e][t] in acc[ct][e]: its token's 4 adjacent columns
        const int t = token(i);
        if (t < seg_end) {
            const size_t row = ((size_t)t * H + h) * D;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                *reinterpret_cast<float4 *>(o + row + 16 * ct + 4 * lq) =
                    make_float4(acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
        }
        if (more) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[ks][e] = xn[ks][e];
            if constexpr (PO) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = accn[ct];
            } else {
                load_o(i + 1, acc);
            }
        }
    }
}

}  // namespace kda

extern "C" hipError_t kda_launch_chunk32(int dk, int in_bf16, unsigned grid, const kda::ChunkParams &p,
                                         hipStream_t stream);

// Workspace of the segmented forward: N sequences cut into NB segments, H heads, d = dk = dv, T
// tokens, nck checkpoints.  off[0] order int32 [NB]; off[1] checkpoint bases int64 [NB]; off[2]
// initial-state map int32 [NB]; off[3] cuB int32 [NB + 1]; off[4] info int32 [2 N]; off[5] the runs'
// final states fp32 [2][NB][H][d][d]; off[6] S_in bf16 [NB][H][2][d][d + 8]; off[7] the transition runs'
// outputs fp32 [T][H][d]; off[8] their checkpoints fp32 [nck][H][d][d]; off[9] the end.
extern "C" __attribute__((visibility("hidden"))) size_t
kda_segments_workspace_layout(int N, int NB, int H, int d, int T, int64_t nck, size_t *off) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t state = (size_t)d * d * 4;
    size_t o[10];
    o[0] = 0;
    o[1] = o[0] + up((size_t)NB * 4);
    o[2] = o[1] + up((size_t)NB * 8);
    o[3] = o[2] + up((size_t)NB * 4);
    o[4] = o[3] + up((size_t)(NB + 1) * 4);
    o[5] = o[4] + up((size_t)N * 2 * 4);
    o[6] = o[5] + up(2 * (size_t)NB * H * state);
    o[7] = o[6] + up((size_t)NB * H * (size_t)2 * d * (d + 8) * 2);   // S_in, split and transposed
    o[8] = o[7] + up((size_t)T * H * d * 4);
    o[9] = o[8] + up((size_t)nck * H * state);
    if (off)
        for (int i = 0; i < 10; ++i) off[i] = o[i];
    return o[9];
}

extern "C" __attribute__((visibility("hidden"))) hipError_t
kda_launch_chunk_segmented(int dk, int in_bf16, int N, int H, int T, int seg, int NB, int64_t nck, const void *q,
                           const void *k, const void *v, const float *g, const float *beta, const int32_t *cu,
                           const float *s0, float *sf, int every, float *ckpt, float *o, float scale,
                           const int32_t *s0_idx, const int32_t *ck_idx, int nslots, int flags, void *workspace,
                           hipStream_t stream) {
    if (N == 0) return hipSuccess;
    if (dk != 64 && dk != 128) return hipErrorInvalidValue;
    size_t off[10];
    kda_segments_workspace_layout(N, NB, H, dk, T, nck, off);
    char *ws = static_cast<char *>(workspace);
    int32_t *order = reinterpret_cast<int32_t *>(ws + off[0]);
    int64_t *ckb = reinterpret_cast<int64_t *>(ws + off[1]);
    int32_t *s0map = reinterpret_cast<int32_t *>(ws + off[2]);
    int32_t *cuB = reinterpret_cast<int32_t *>(ws + off[3]);
    int32_t *info = reinterpret_cast<int32_t *>(ws + off[4]);
    float *st = reinterpret_cast<float *>(ws + off[5]);
    __bf16 *sin_ = reinterpret_cast<__bf16 *>(ws + off[6]);
    float *oI = reinterpret_cast<float *>(ws + off[7]);
    float *ckI = reinterpret_cast<float *>(ws + off[8]);
    const int s0_slots = s0_idx ? nslots : N;
    // 1. the segment list
    hipLaunchKernelGGL(kda::segment_plan_kernel, dim3(1), dim3(1024), 0, stream, cu, N, seg, every, NB, s0, s0_idx,
                       s0_slots, cuB, info, order, ckb, s0map);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 2. both runs of every segment
    kda::ChunkParams p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.cu_seqlens = cuB; p.order = order; p.ckpt_base = ckb;
    p.s0 = s0; p.sf = st; p.ckpt = ckpt; p.o = o; p.s0_idx = s0map; p.ck_idx = ck_idx; p.nslots = nslots;
    p.s0_slots = s0_slots; p.flags = flags | kda::KDA_TRANSITION; p.H = H; p.every = every; p.scale = scale;
    p.nseq = NB; p.o_tr = oI; p.ckpt_tr = ckI;
    e = kda_launch_chunk32(dk, in_bf16, (unsigned)NB * (unsigned)H, p, stream);
    if (e != hipSuccess) return e;
    // 3. the chain: initial states of the later segments, their checkpoints, the final states
    if (dk == 128)
        hipLaunchKernelGGL(kda::segment_chain_kernel<128>, dim3((unsigned)N * H * 8), dim3(512), 0, stream, info, cuB,
                           ckb, H, NB, every, st, sin_, sf, ckpt, ck_idx, nslots, ckI);
    else
        hipLaunchKernelGGL(kda::segment_chain_kernel<64>, dim3((unsigned)N * H * 4), dim3(256), 0, stream, info, cuB,
                           ckb, H, NB, every, st, sin_, sf, ckpt, ck_idx, nslots, ckI);
    e = hipGetLastError();
    if (e != hipSuccess || NB == N) return e;   // NB == N: every segment is a first one
    // 4. the outputs of the later segments: tiles of 128 tokens, several per workgroup when there
    // are many (each workgroup stages its S_in once, and its next tile loads during this one)
    constexpr int NW = kda::CORR_WAVES, TT = 16 * NW;
    const int tiles = (seg + TT - 1) / TT;
    const long long busy = (long long)(NB - N) * tiles * H / kda_cu_count();   // tiles per compute unit
    const int tpw = busy < 2 ? 1 : busy < 6 ? 4 : 8;   // (measured best of 1, 2, 4, 8 at 1, 3 and 7 per CU)
    const int groups = (tiles + tpw - 1) / tpw;
    const dim3 grid((unsigned)NB * groups, (unsigned)H);
#define KDA_CORR(DKV, TPW, PO)                                                                                  \
    hipLaunchKernelGGL((kda::segment_correct_kernel<DKV, NW, TPW, PO>), grid, dim3(64 * NW), 0, stream, cuB, s0map, \
                       H, groups, sin_, oI, o)
    if (dk == 128) {
        switch (tpw) {
            case 1: KDA_CORR(128, 1, false); break;
            case 4: KDA_CORR(128, 4, true); break;
            default: KDA_CORR(128, 8, true); break;
        }
    } else {
        switch (tpw) {
            case 1: KDA_CORR(64, 1, false); break;
            case 4: KDA_CORR(64, 4, true); break;
            default: KDA_CORR(64, 8, true); break;
        }
    }
#undef KDA_CORR
    return hipGetLastError();
}
