// kda_bwd.hip -- backward of the chunked KDA prefill (gfx950): gradients of
// L = sum(dO * O) + sum(dS_T * S_T) with respect to q, k, v, g, beta and S_0.
//
// The recurrence (the delta rule of the "Attention->K3 course, Day 21" quiz Q9 with the
// per-channel forget gate of the skill card's quick facts), written per 32-token chunk with
// S the state entering the chunk, B_r = sum_{r' <= r} g_r' (in-chunk cumulative log decay),
// Gam_r = exp(B_r), Gam_C = exp(B_last), and per-pair factors e^{B_r - B_s} (per channel):
//     A_rs  = sum_i k_ri k_si e^{B_ri - B_si}   (s < r)       T = (I + Diag(beta) A)^-1
//     Aq_rs = sum_i q_ri k_si e^{B_ri - B_si}   (s <= r)
//     X = (Gam K) S,   R = V - X,   Z = Diag(beta) R,   U = T Z
//     O = scale ((Gam Q) S + Aq U),   S' = Gam_C S + Kbar^T U,   Kbar_s = e^{B_last - B_s} k_s
// Given D = dL/dS' (gradient at the chunk's end) its adjoint is
//     dU = scale Aq^T dO + Kbar D                 dZ = T^T dU         dV = Diag(beta) dZ
//     dL/dS = Gam_C D + scale (Gam Q)^T dO - W^T dU,   W = T Diag(beta) (Gam K)
//     dbeta_r = <dZ_r, R_r> - sum_{s<r} <dZ_r, U_s> A_rs
//     dA_rs = -beta_r <dZ_r, U_s> (s < r)        dAq_rs = scale <dO_r, U_s> (s <= r)
//     d(Gam Q) = scale dO S^T    d(Gam K) = -Diag(beta) dZ S^T    dKbar = U D^T
// plus the pair terms of A and Aq.  Every factor that multiplies k_ri with e^{+B_ri} is the
// "row side" of k (dkp), every one with e^{-B_si} the "column side" (dkm); then
// dB = q dq + k dkp - k dkm, the last row also gets Gam_C rowsum(S * D) + sum_s Kbar_s dKbar_s,
// and dg is the reverse cumulative sum of dB over the chunk.
//
// Four launches: the forward in its states-only form with a checkpoint every 32 tokens (states
// at chunk starts, no outputs); a per-chunk prep kernel (A, Aq, T, W, E = scale Aq^T dO); the
// state-gradient scan, sequential over the chunks of a (sequence, head) and split over
// 16-column blocks of d_v; and the per-chunk gradient kernel.  With the fused prologue, a
// prologue kernel materialises the operator's inputs first and an epilogue kernel takes the
// gradients back to the raw inputs last.  Products run on the fp32 MFMA (16x16x4): lane l
// supplies row (or column) l % 16 and contraction index 4 (l / 16) + kk in instruction kk; an
// output tile holds element (4 (l / 16) + e, l % 16) in slot e.  The gradient kernel's stage-2
// and stage-3 products take bf16 hi+lo operand pairs instead when the inputs are bf16.
//
// The pair factors use a reference row m per 16x16 tile (7 and 23 on the diagonal tiles, 15
// below them): e^{B_r - B_s} = e^{B_r - B_m} e^{B_m - B_s} with both factors within e^{40}
// for decays g >= -5.
#include "kda_frag.h"
#include "kda_bwd_flags.h"
#include "kda_side.h"

#include <type_traits>

namespace kda {

constexpr int BC = 32;   // chunk of the backward

struct BwdParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu;
    const int32_t *order;          // sequences, longest first (forward plan)
    const int64_t *ck_base;        // per sequence: its first 32-token checkpoint (forward plan)
    const int32_t *cbase;          // [N + 1]: first chunk of each sequence
    const float *ckpt;             // states after every 32 tokens
    const float *s0, *dO, *dSf;
    float *Dck;                    // [chunks, H, dk, dv]: dL/dS at the end of each chunk
    float *SCk;                    // [chunks, H] records of the scan's operands (ScanRec)
    float *TAk;                    // [chunks, H, 2, 32, 32]: A (masked), T
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    int N, H;
    float scale;
    int pt;                        // the one-workgroup scan: the record's RC region holds P^T, not R,
                                   // and the scan leaves Y = Kbar D in its KB region
    int rrec;                      // (with pt) the recompute left R = V - (Gam K) S in the record (RR)
};

// Per (chunk, head): the operands of the state-gradient scan (and E for the gradient kernel),
// fp32, laid out so that each lane reads 4 consecutive values:
//   KB [32][dk]   Kbar = e^{B_last - B} k       WT [dk][32]  W^T
//   ET [dv][32]   E^T                          GL [dk]      Gam_C = e^{B_last}
//   RC [dk][dv]   R = scale (Gam Q - Aq W)^T dO = scale (Gam Q)^T dO - W^T E, the part of the
//                 update that does not depend on D, in 16x16 tiles (tile (i/16, j/16), then lane
//                 4 (i % 16 / 4) ... as an MFMA output tile: 64 lanes x 4 values); for the
//                 one-workgroup-per-chain scan, P^T [dk][32] (P = scale (Gam Q - Aq W)) instead
// That scan also overwrites KB, once it has read it, with Y = Kbar D [32][dv] (D the gradient at
// the chunk's end), and the states-only recompute that runs with it leaves R = V - (Gam K) S
// [32][dv] in RC after P^T (RR): the gradient kernel reads both instead of forming them.
template <int DK> struct ScanRec {
    static constexpr int DV = DK;
    static constexpr int KB = 0, WT = 32 * DK, ET = 64 * DK, GL = 64 * DK + 32 * DV, RC = GL + DK;
    static constexpr int RR = RC + DK * 32;
    static constexpr int SIZE = RC + DK * DV;
};

// Reference row and tile coordinates of the three lower 16x16 tiles of a 32x32 chunk matrix.
__device__ __forceinline__ void tile_of(int tl, int &rt, int &st, int &m) {
    rt = tl == 0 ? 0 : 1;
    st = tl == 2 ? 1 : 0;
    m = tl == 0 ? 7 : (tl == 1 ? 15 : 23);
}

// Largest n < N with cbase[n] <= gc (the sequence that owns chunk gc; empty sequences own none).
__device__ __forceinline__ int seq_of_chunk(const int32_t *cbase, int N, int gc) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cbase[mid] <= gc) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// v if ok, else zeros, selected per element (a select between whole vectors can end up as a
// select between two stack addresses)
__device__ __forceinline__ float4 keep4(bool ok, const float4 &v) {
    return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
}

__device__ __forceinline__ f32x4_t f4v(const float4 &v) { return f32x4_t{v.x, v.y, v.z, v.w}; }

__device__ __forceinline__ float red16(float t) {   // sum over the 16 lanes of a row group
    t += shfl_xor(t, 1);
    t += shfl_xor(t, 2);
    t += shfl_xor(t, 4);
    t += shfl_xor(t, 8);
    return t;
}

// cbase[n] = sum_{m < n} ceil(L_m / 32), cbase[N] = total (one workgroup of 1024 threads).
__global__ void __launch_bounds__(1024) bwd_plan_kernel(const int32_t *__restrict__ cu, int N,
                                                         int32_t *__restrict__ cbase) {
    __shared__ int32_t part[1024];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 1024) {
        const int n = base + (int)threadIdx.x;
        const int c = n < N ? (cu[n + 1] - cu[n] + BC - 1) / BC : 0;
        part[threadIdx.x] = c;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += v;
            __syncthreads();
        }
        if (n < N) cbase[n] = carry + part[threadIdx.x] - c;
        __syncthreads();
        if (threadIdx.x == 1023) carry += part[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) cbase[N] = carry;
}

// ---- per-chunk prep: A, T, W = T Diag(beta) (Gam K), E = scale Aq^T dO, R -------------------
// One workgroup of dk/16 waves per (chunk, head).
// With p.pt the scan forms R = P^T dO itself (P = scale (Gam Q - Aq W)): the record's RC region
// holds P^T [dk][32] instead of R.
template <int DK, typename IN_T>
__global__ void __launch_bounds__(DK * 4) bwd_prep_kernel(const BwdParams p) {
    constexpr int NW = DK / 16, NT = DK * 4, P = DK + 4, DV = DK;
    __shared__ __attribute__((aligned(16))) float sk[BC][P], sq[BC][P], sb[BC][P], sdo[BC][P];
    __shared__ float sA[BC][BC + 1], sAq[BC][BC + 1], sT[BC][BC + 1];
    __shared__ float sbeta[BC];

    const int H = p.H;
    const int gc = (int)blockIdx.x / H, h = (int)blockIdx.x % H;
    const int n = seq_of_chunk(p.cbase, p.N, gc);
    const int t0 = p.cu[n] + BC * (gc - p.cbase[n]);
    const int nv = min(BC, p.cu[n + 1] - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, q4 = lane >> 4;
    const IN_T *qg = static_cast<const IN_T *>(p.q), *kg = static_cast<const IN_T *>(p.k);

    // staging: every load issued as a 16-byte vector before the first LDS write; rows past the
    // chunk read its last row and are zeroed (no branch around a load)
    {
        constexpr int VE = 16 / (int)sizeof(IN_T);                   // input elements per vector
        constexpr int NKV = BC * DK / VE, NFV = BC * DK / 4;         // vectors of k (q), of g (dO)
        constexpr int UK = (NKV + NT - 1) / NT, UF = (NFV + NT - 1) / NT;
        uint4 kv[UK], qv[UK];
        float4 gv[UF], ov[UF];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int idx = min(tid + u * NT, NKV - 1), r = idx / (DK / VE), i = idx % (DK / VE) * VE;
            const size_t off = ((size_t)(t0 + min(r, nv - 1)) * H + h) * DK + i;
            kv[u] = *reinterpret_cast<const uint4 *>(kg + off);
            qv[u] = *reinterpret_cast<const uint4 *>(qg + off);
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int idx = min(tid + u * NT, NFV - 1), r = idx / (DK / 4), i = idx % (DK / 4) * 4;
            const size_t off = ((size_t)(t0 + min(r, nv - 1)) * H + h) * DK + i;
            gv[u] = *reinterpret_cast<const float4 *>(p.g + off);
            ov[u] = *reinterpret_cast<const float4 *>(p.dO + off);
        }
        const float bv = p.beta[(size_t)(t0 + min(tid % BC, nv - 1)) * H + h];
        // widen the VE inputs of a 16-byte vector to fp32 and store them at dst (zeros if !ok)
        auto put = [&](float *dst, const uint4 x, bool ok) {
            const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < VE / 4; ++j) {
                float4 f;
                if constexpr (sizeof(IN_T) == 2)   // bf16 pairs, the lower element in the low half
                    f = make_float4(lo_bf16_of(wd[2 * j]), hi_bf16_of(wd[2 * j]), lo_bf16_of(wd[2 * j + 1]),
                                    hi_bf16_of(wd[2 * j + 1]));
                else
                    f = make_float4(__uint_as_float(wd[0]), __uint_as_float(wd[1]), __uint_as_float(wd[2]),
                                    __uint_as_float(wd[3]));
                *reinterpret_cast<float4 *>(dst + 4 * j) = keep4(ok, f);
            }
        };
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int idx = tid + u * NT, r = idx / (DK / VE), i = idx % (DK / VE) * VE;
            if (idx < NKV) {
                put(&sk[r][i], kv[u], r < nv);
                put(&sq[r][i], qv[u], r < nv);
            }
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int idx = tid + u * NT, r = idx / (DK / 4), i = idx % (DK / 4) * 4;
            if (idx < NFV) {
                *reinterpret_cast<float4 *>(&sb[r][i]) = keep4(r < nv, gv[u]);
                *reinterpret_cast<float4 *>(&sdo[r][i]) = keep4(r < nv, ov[u]);
            }
        }
        if (tid < BC) sbeta[tid] = tid < nv ? bv : 0.f;
        for (int idx = tid; idx < BC * BC; idx += NT) {
            sA[idx / BC][idx % BC] = 0.f;
            sAq[idx / BC][idx % BC] = 0.f;
        }
    }
    __syncthreads();
    if (tid < DK) {
        float a = 0.f;
        for (int r = 0; r < BC; ++r) {
            a += sb[r][tid];
            sb[r][tid] = a;
        }
    }
    __syncthreads();

    using SR = ScanRec<DK>;
    const size_t cb = blockIdx.x;   // = chunk * H + head
    float *rec = p.SCk + cb * SR::SIZE;
    for (int idx = tid; idx < BC * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        rec[SR::KB + idx] = sk[r][i] * __expf(sb[BC - 1][i] - sb[r][i]);
    }
    if (tid < DK) rec[SR::GL + tid] = __expf(sb[BC - 1][tid]);

    // lower tiles of A (k against k) and Aq (q against k), each over the whole d_k
    for (int it = w; it < 6; it += NW) {
        int rt, st, m;
        tile_of(it % 3, rt, st, m);
        const bool isq = it >= 3;
        const float *xa = isq ? sq[16 * rt + c] : sk[16 * rt + c];
        const float *ba = sb[16 * rt + c], *bm = sb[m], *kb = sk[16 * st + c], *bb = sb[16 * st + c];
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kg4 = 0; kg4 < DK / 4; ++kg4) {
            const int i = 16 * (kg4 >> 2) + 4 * q4 + (kg4 & 3);
            acc = mfma_f32(xa[i] * __expf(ba[i] - bm[i]), kb[i] * __expf(bm[i] - bb[i]), acc);
        }
        float(*M)[BC + 1] = isq ? sAq : sA;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * q4 + e, s = 16 * st + c;
            M[r][s] = (isq ? s <= r : s < r) ? acc[e] : 0.f;
        }
    }
    __syncthreads();

    // T = (I + Diag(beta) A)^-1 (unit lower triangular) by blocks: the 16x16 diagonal blocks by
    // forward substitution (wave b inverts block b, lane s owns its column s), then
    // T10 = -T11 (Diag(beta) A)10 T00 as two 16x16 fp32 MFMA products on wave 0
    if (w < 2 && lane < 16) {
        const int o = __builtin_amdgcn_readfirstlane(16 * w), s = lane;
        const float *Ab = &sA[o][o], *bb = &sbeta[o];
        float *Tb = &sT[o][o + s];
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float a = 0.f;
#pragma unroll
            for (int mm = 0; mm < r; ++mm) a += Ab[r * (BC + 1) + mm] * t[mm];
            t[r] = (r == s ? 1.f : 0.f) - bb[r] * a;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tb[r * (BC + 1)] = t[r];
        if (o == 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[r][16 + s] = 0.f;   // block above the diagonal
    }
    __syncthreads();
    if (w == 0) {
        f32x4_t P = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)   // P = (Diag(beta) A)10 T00
            P = mfma_f32(sbeta[16 + c] * sA[16 + c][4 * q4 + kk], sT[4 * q4 + kk][c], P);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)   // Q = T11 P
            Q = mfma_f32(sT[16 + c][16 + 4 * q4 + kk], P[kk], Q);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[16 + 4 * q4 + e][c] = -Q[e];
    }
    __syncthreads();

    // W = T Diag(beta) (Gam K), stored transposed: wave w writes columns 16 w .. 16 w + 15; then
    // R = scale (Gam Q - Aq W)^T dO for rows 16 w .. 16 w + 15 of R
    {
        const int i = 16 * w + c;
        f32x4_t Wt[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int st = 0; st <= rt; ++st)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int s = 16 * st + 4 * q4 + kk;
                    acc = mfma_f32(sT[16 * rt + c][s], sbeta[s] * sk[s][i] * __expf(sb[s][i]), acc);
                }
            Wt[rt] = acc;
            *reinterpret_cast<float4 *>(rec + SR::WT + i * BC + 16 * rt + 4 * q4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        float Qp[2][4];   // scale (Gam Q - Aq W)[16 rt + 4 q4 + e][i]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st <= rt; ++st)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) aw = mfma_f32(sAq[16 * rt + c][16 * st + 4 * q4 + kk], Wt[st][kk], aw);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * q4 + e;
                Qp[rt][e] = p.scale * (sq[r][i] * __expf(sb[r][i]) - aw[e]);
            }
        }
        if (p.pt) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                *reinterpret_cast<float4 *>(rec + SR::RC + i * BC + 16 * rt + 4 * q4) =
                    make_float4(Qp[rt][0], Qp[rt][1], Qp[rt][2], Qp[rt][3]);
        } else {
            float *Rt = rec + SR::RC + (size_t)w * (DV / 16) * 256 + 4 * lane;
            for (int jt = 0; jt < DV / 16; ++jt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(Qp[rg][kk], sdo[16 * rg + 4 * q4 + kk][16 * jt + c], acc);
                *reinterpret_cast<float4 *>(Rt + jt * 256) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
    // E = scale Aq^T dO, stored transposed: wave w writes value columns 16 w .. 16 w + 15
    {
        const int jj = 16 * w + c;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int rt = st; rt < 2; ++rt)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int r = 16 * rt + 4 * q4 + kk;
                    acc = mfma_f32(sAq[r][16 * st + c], sdo[r][jj], acc);
                }
            *reinterpret_cast<float4 *>(rec + SR::ET + jj * BC + 16 * st + 4 * q4) =
                make_float4(p.scale * acc[0], p.scale * acc[1], p.scale * acc[2], p.scale * acc[3]);
        }
    }
    float *ta = p.TAk + cb * 2 * BC * BC;
    for (int idx = tid; idx < BC * BC; idx += NT) {
        ta[idx] = sA[idx / BC][idx % BC];
        ta[BC * BC + idx] = sT[idx / BC][idx % BC];
    }
}

// ---- state-gradient scan ------------------------------------------------------------------
// One workgroup of 4 waves per (chain, 16-column block of d_v); wave w holds rows
// [dk/4 w, dk/4 (w+1)) of the block of D in registers.  Walking the chunks last to first it
// stores D (the gradient at the chunk's end) and applies
//     D <- Gam_C D + R - W^T (Kbar D),    R = scale (Gam Q)^T dO - W^T E,
// with the operands of chunk j-1 loading into registers while chunk j is processed.
template <int DK> struct ScanOps {
    static constexpr int RT = DK / 64;   // 16-row tiles of d_k per wave
    float4 kb[2][RT];                     // Kbar[16 rt + c][kr0 + 16 kt + 4 q4 ..]
    float4 wt[RT][2];                     // WT[kr0 + 16 kt + c][16 rg + 4 q4 ..]
    float4 gl[RT];                        // GL[kr0 + 16 kt + 4 q4 ..]
    float4 rc[RT];                        // R[kr0 + 16 kt + 4 q4 + e][j0 + c]
};

template <int DK>
__device__ __forceinline__ void scan_load(ScanOps<DK> &o, const BwdParams &p, size_t cb, int kr0, int jb, int lane) {
    using SR = ScanRec<DK>;
    constexpr int RT = ScanOps<DK>::RT, DV = DK;
    const int c = lane & 15, q4 = lane >> 4;
    const float *rec = p.SCk + cb * SR::SIZE;
#pragma unroll
    for (int kt = 0; kt < RT; ++kt) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            o.kb[rt][kt] = *reinterpret_cast<const float4 *>(rec + SR::KB + (16 * rt + c) * DK + kr0 + 16 * kt + 4 * q4);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
            o.wt[kt][rg] = *reinterpret_cast<const float4 *>(rec + SR::WT + (kr0 + 16 * kt + c) * BC + 16 * rg + 4 * q4);
        o.gl[kt] = *reinterpret_cast<const float4 *>(rec + SR::GL + kr0 + 16 * kt + 4 * q4);
        o.rc[kt] = *reinterpret_cast<const float4 *>(rec + SR::RC + (size_t)((kr0 / 16 + kt) * (DV / 16) + jb) * 256 + 4 * lane);
    }
}

__device__ __forceinline__ float f4(const float4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

template <int DK>
__global__ void __launch_bounds__(256) bwd_dstate_kernel(const BwdParams p) {
    constexpr int DV = DK, NBV = DV / 16, KS = DK / 4, RT = ScanOps<DK>::RT;
    __shared__ float part[2][4][BC][17];   // partial Kbar D of each wave, double-buffered

    const int H = p.H, chains = p.N * H;
    // the NBV workgroups of one chain are consecutive modulo 8, so they share an XCD
    const int b = blockIdx.x;
    const int grp = b / (8 * NBV), within = b % (8 * NBV);
    const int gsz = min(8, chains - grp * 8);
    const int ci = grp * 8 + within % gsz, jb = within / gsz;
    const int n = p.order[ci / H], h = ci % H;
    const int seq0 = p.cu[n], L = p.cu[n + 1] - seq0, nch = (L + BC - 1) / BC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, q4 = lane >> 4;
    const int j0 = 16 * jb, kr0 = KS * w;
    const size_t st_off = ((size_t)n * H + h) * DK * DV;
    const int cb0 = p.cbase[n];

    f32x4_t Dr[RT];   // D[kr0 + 16 kt + 4 q4 + e][j0 + c]
#pragma unroll
    for (int kt = 0; kt < RT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Dr[kt][e] = p.dSf ? p.dSf[st_off + (size_t)(kr0 + 16 * kt + 4 * q4 + e) * DV + j0 + c] : 0.f;

    // one chunk of the scan with its operands in `cur`
    auto step = [&](const ScanOps<DK> &cur, int jc) {
        const size_t cb = (size_t)(cb0 + jc) * H + h;
        float *dd = p.Dck + cb * DK * DV;
#pragma unroll
        for (int kt = 0; kt < RT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dd[(size_t)(kr0 + 16 * kt + 4 * q4 + e) * DV + j0 + c] = Dr[kt][e];

        // partial Kbar D over this wave's rows of d_k
        float(*pp)[17] = part[jc & 1][w];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < RT; ++kt)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(f4(cur.kb[rt][kt], kk), Dr[kt][kk], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) pp[16 * rt + 4 * q4 + e][c] = acc[e];
        }
        lds_barrier();

        float nY[2][4];   // -(Kbar D)[16 rg + 4 q4 + kk][j0 + c]
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r = 16 * rg + 4 * q4 + kk;
                float a = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) a += part[jc & 1][ww][r][c];
                nY[rg][kk] = -a;
            }
#pragma unroll
        for (int kt = 0; kt < RT; ++kt) {
            f32x4_t acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = f4(cur.gl[kt], e) * Dr[kt][e] + f4(cur.rc[kt], e);
#pragma unroll
            for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(f4(cur.wt[kt][rg], kk), nY[rg][kk], acc);
            Dr[kt] = acc;
        }
    };
    auto fetch = [&](ScanOps<DK> &o, int jc) { scan_load<DK>(o, p, (size_t)(cb0 + (jc > 0 ? jc : 0)) * H + h, kr0, jb, lane); };
    // two operand sets used in turn: chunk j is processed while chunk j - 1 loads
    ScanOps<DK> opA, opB;
    if (nch > 0) fetch(opA, nch - 1);
    for (int jc = nch - 1; jc >= 0; jc -= 2) {
        fetch(opB, jc - 1);
        step(opA, jc);
        if (jc == 0) break;
        fetch(opA, jc - 2);
        step(opB, jc - 1);
    }
    if (p.dS0)
#pragma unroll
        for (int kt = 0; kt < RT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.dS0[st_off + (size_t)(kr0 + 16 * kt + 4 * q4 + e) * DV + j0 + c] = Dr[kt][e];
}

// ---- state-gradient scan, one workgroup per chain (d = 128, hi/lo bf16 products) -------------
// Wave w of 8 holds value columns 16 w .. 16 w + 15 of D for every d_k row, as 8 output tiles (the
// forward's layout of the state), so no partial product crosses waves.  Per chunk, last to first:
//     D (the gradient at the chunk's end) -> Dck,   Y = Kbar D,   D <- Gam_C D + P^T dO - W^T Y,
// with P^T from the record (R = P^T dO is formed here, not stored) and dO of the wave's columns.
// Kbar, W^T and P^T are staged in LDS as hi/lo bf16 planes in the MFMA fragment layout, in two
// buffers: after chunk r (counted from the last) has run, chunk r + 1's records go from registers
// (loaded two steps earlier) into the other buffer and chunk r + 3's are loaded, with dO of chunk
// r + 2.  Products: hi/lo bf16 pairs (three MFMAs), fp32 accumulation.
template <int DK> struct DScanLds {
    static constexpr int KB = DK / 32;
    static constexpr int KBAR = 0;                          // [32][DK] hl, fofs<KB>
    static constexpr int KBAR_PLANE = 32 * DK * 2;
    static constexpr int WT = KBAR + 2 * KBAR_PLANE;        // [DK][32] hl, fofs<1>
    static constexpr int T_PLANE = DK * 32 * 2;
    static constexpr int PT = WT + 2 * T_PLANE;             // [DK][32] hl, fofs<1>
    static constexpr int GL = PT + 2 * T_PLANE;             // [DK] fp32
    static constexpr int BUF = GL + DK * 4;
    static constexpr int TOTAL = 2 * BUF;
};

template <int DK>
__global__ void __launch_bounds__(512) bwd_dscan_hl_kernel(const BwdParams p) {
    static_assert(DK == 128, "8 waves of 16 value columns");
    constexpr int DV = DK, KB = DK / 32, KT = DK / 16, NT = 512;
    constexpr int RPM = 1024 / NT;   // float4 rounds per staged matrix ([32][DK] or [DK][32])
    using L = DScanLds<DK>;
    using M = Mat<false>;
    using SR = ScanRec<DK>;
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];

    const int H = p.H;
    const int ci = (int)blockIdx.x, n = p.order[ci / H], h = ci % H;
    const int seq0 = p.cu[n], Lq = p.cu[n + 1] - seq0, nch = (Lq + BC - 1) / BC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, q4 = lane >> 4;
    const int j0 = 16 * w;
    const size_t st_off = ((size_t)n * H + h) * DK * DV;
    const int cb0 = p.cbase[n];

    f32x4_t Dt[KT];   // D[16 ct + 4 q4 + e][j0 + c]
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Dt[ct][e] = p.dSf ? p.dSf[st_off + (size_t)(16 * ct + 4 * q4 + e) * DV + j0 + c] : 0.f;
    if (nch == 0) {
        if (p.dS0)
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) p.dS0[st_off + (size_t)(16 * ct + 4 * q4 + e) * DV + j0 + c] = Dt[ct][e];
        return;
    }

    // chunk of relative index r (0: the last), clamped for the loads past the first
    auto chunk_of = [&](int r) { return max(nch - 1 - r, 0); };
    // Addresses: a uniform (scalar) base per row or record plus one 32-bit lane offset, so that
    // no load or store keeps a 64-bit address of its own in registers.
    // (byte offsets: a 32-bit offset register with a scalar base)
    const unsigned d_lane = 4u * (unsigned)(4 * q4 * DV + j0 + c);        // D[4 q4][j0 + c] of a [DK][DV] state
    const unsigned o_lane = 4u * (unsigned)(4 * q4 * H * DV + j0 + c);    // dO[row 4 q4][h][j0 + c], relative
    auto at = [](const float *base, unsigned byte_off) {
        return reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + byte_off);
    };
    // the records of a chunk: thread tid holds float4 tid + 512 u of [Kbar | W^T | P^T] and float4
    // tid % (DK / 4) of Gam_C (written by threads tid < DK / 4)
    struct Stage { float4 x[3 * RPM]; float4 gl; };
    auto sload = [&](Stage &st, int r) {
        const float *rec = p.SCk + ((size_t)(cb0 + chunk_of(r)) * H + h) * SR::SIZE;
#pragma unroll
        for (int u = 0; u < 3 * RPM; ++u) {
            const unsigned f = (unsigned)tid + NT * (u % RPM);   // float4 index within its matrix
            const float *src = u < RPM ? rec + SR::KB : u < 2 * RPM ? rec + SR::WT : rec + SR::RC;
            st.x[u] = *reinterpret_cast<const float4 *>(src + 4 * f);
        }
        st.gl = *reinterpret_cast<const float4 *>(rec + SR::GL + 4 * (unsigned)(tid & (DK / 4 - 1)));
    };
    auto swrite = [&](const Stage &st, char *buf) {
#pragma unroll
        for (int u = 0; u < 3 * RPM; ++u) {
            const int f = tid + NT * (u % RPM);
            const float x[4] = {st.x[u].x, st.x[u].y, st.x[u].z, st.x[u].w};
            if (u < RPM)
                M::template put_hl<4>(buf + L::KBAR, L::KBAR_PLANE, fofs<KB>(f / (DK / 4), 4 * (f % (DK / 4))), x);
            else
                M::template put_hl<4>(buf + (u < 2 * RPM ? L::WT : L::PT), L::T_PLANE, fofs<1>(f / 8, 4 * (f % 8)), x);
        }
        if (tid < DK / 4) *reinterpret_cast<float4 *>(buf + L::GL + 16 * tid) = st.gl;
    };
    // dO of a chunk for this wave's columns, as two output tiles (rows past the chunk: zeros)
    // (rows past the chunk's end read its last row; the step zeroes them, so that no load is
    // waited for here)
    auto dload = [&](f32x4_t (&d)[2], int r) {
        const int jc = chunk_of(r), t0 = seq0 + BC * jc, nv = min(BC, Lq - BC * jc);
        if (nv == BC) {   // (uniform) a full chunk
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) d[rt][e] = *at(p.dO + ((size_t)(t0 + 16 * rt + e) * H + h) * DV, o_lane);
        } else {          // the last chunk of a sequence
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    d[rt][e] = p.dO[((size_t)(t0 + min(16 * rt + 4 * q4 + e, nv - 1)) * H + h) * DV + j0 + c];
        }
    };
    // one chunk (relative index r) with its records in LDS buffer `buf` and its dO in `dcur`
    auto step = [&](int r, const char *buf, const f32x4_t (&dcur)[2]) {
        const int jc = nch - 1 - r;
        float *const dd = p.Dck + ((size_t)(cb0 + jc) * H + h) * DK * DV;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) *const_cast<float *>(at(dd + (size_t)(16 * ct + e) * DV, d_lane)) = Dt[ct][e];
        // Y = Kbar D, then -Y
        f32x4_t Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KB; ++s) {
            const Frag<false> df = M::template from_tiles<true>(Dt[2 * s], Dt[2 * s + 1]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                mma<true, true>(Y[rt], M::template get<true>(buf + L::KBAR, L::KBAR_PLANE, fbase<KB>(rt, s, lane)), df);
            __builtin_amdgcn_sched_barrier(0);   // one K-step's fragments live at a time (registers)
        }
        // Y into the record's KB region (read into LDS two steps ago) for the gradient kernel
        {
            float *const yd = p.SCk + ((size_t)(cb0 + jc) * H + h) * SR::SIZE + SR::KB;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) *const_cast<float *>(at(yd + (16 * rt + e) * DV, d_lane)) = Y[rt][e];
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) Y[rt][e] = -Y[rt][e];
        const Frag<false> yf = M::template from_tiles<true>(Y[0], Y[1]);
        f32x4_t dm[2];   // dO, zero past the chunk's end
        {
            const int nv = min(BC, Lq - BC * jc);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dm[rt][e] = 16 * rt + 4 * q4 + e < nv ? dcur[rt][e] : 0.f;
        }
        const Frag<false> of = M::template from_tiles<true>(dm[0], dm[1]);
        const float *gl = reinterpret_cast<const float *>(buf + L::GL);
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gl + 16 * ct + 4 * q4);
            f32x4_t acc = {g4.x * Dt[ct][0], g4.y * Dt[ct][1], g4.z * Dt[ct][2], g4.w * Dt[ct][3]};
            mma<true, true>(acc, M::template get<true>(buf + L::PT, L::T_PLANE, fbase<1>(ct, 0, lane)), of);
            mma<true, true>(acc, M::template get<true>(buf + L::WT, L::T_PLANE, fbase<1>(ct, 0, lane)), yf);
            Dt[ct] = acc;
            __builtin_amdgcn_sched_barrier(0);   // one tile's fragments live at a time (registers)
        }
    };

    Stage sa, sb;          // register stages: sa for even relative chunks, sb for odd
    f32x4_t da[2], db[2];  // dO: da for even relative chunks, db for odd
    sload(sa, 0);
    swrite(sa, smem);      // chunk 0 (relative) into buffer 0
    sload(sb, 1);
    sload(sa, 2);
    dload(da, 0);
    dload(db, 1);
    // even r: buffer 0 and da, then chunk r + 1 from sb into buffer 1 and chunk r + 3 into sb; odd r:
    // buffer 1 and db, then chunk r + 1 from sa into buffer 0 and chunk r + 3 into sa.  Step 0 and a
    // last odd step are peeled so that the loop runs over whole pairs (no exit between its two
    // steps, where the registers carried around the loop would need copies, and the copies waits
    // for their loads).
    auto even = [&](int r) {
        lds_barrier();
        step(r, smem, da);
        if (r + 1 < nch) swrite(sb, smem + L::BUF);
        sload(sb, r + 3);
        dload(da, r + 2);
    };
    auto odd = [&](int r) {
        lds_barrier();
        step(r, smem + L::BUF, db);
        if (r + 1 < nch) swrite(sa, smem);
        sload(sa, r + 3);
        dload(db, r + 2);
    };
    even(0);
    int r = 1;
    for (; r + 1 < nch; r += 2) {
        odd(r);
        even(r + 1);
    }
    if (r < nch) odd(r);
    if (p.dS0)
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.dS0[st_off + (size_t)(16 * ct + 4 * q4 + e) * DV + j0 + c] = Dt[ct][e];
}

// ---- per-chunk gradients --------------------------------------------------------------------
// One workgroup of dk/16 waves per (chunk, head).  Stage 1: wave w owns value columns
// 16w..16w+15 (X, Kbar D, dZ, U, dv, the <dZ, R> part of dbeta).  Stage 2: the 32x32 products
// <dZ_r, U_s> and <dO_r, U_s>.  Stage 3: wave w owns key channels 16w..16w+15 (dq, dk, dg).
// HL: the stage-2 and stage-3 products take bf16 hi+lo operands (the bf16-input error budget; also
// for the fp32 unit vectors of the fused normalisation), else fp32 MFMA.
template <int DK, typename IN_T, bool HL = sizeof(IN_T) == 2>
__global__ void __launch_bounds__(DK * 4) __attribute__((amdgpu_waves_per_eu(4)))
bwd_grad_kernel(const BwdParams p) {
    constexpr int NW = DK / 16, NT = DK * 4, P = DK + 4, DV = DK;
    // k and q in their input type; sb holds the cumulative log decay, then (per wave, its own
    // columns) dB; sTq holds T for stage 1, then dAq.  With bf16 inputs and d = 128 two
    // workgroups fit in one CU's LDS.
    constexpr int PK = DK + 16 / (int)sizeof(IN_T);   // row pitch of sk, sq: rows start 16-byte aligned
    __shared__ __attribute__((aligned(16))) IN_T sk[BC][PK], sq[BC][PK];
    // U (sx) and dZ (sz): fp32 rows, or with HL hi and lo bf16 planes (written once by the wave that
    // forms them, read as 8-element MFMA fragments in stages 2 and 3)
    constexpr int PB = DK + 8;                              // bf16 plane row pitch (elements)
    constexpr int PLANE = BC * PB * 2;                      // bytes of one plane
    constexpr int XB = HL ? 2 * PLANE : BC * P * 4;
    __shared__ __attribute__((aligned(16))) float sb[BC][P];
    __shared__ __attribute__((aligned(16))) char sxb[XB], szb[XB];
    float(*sx)[P] = reinterpret_cast<float(*)[P]>(sxb);
    float(*sz)[P] = reinterpret_cast<float(*)[P]>(szb);
    __shared__ float sA[BC][BC + 1], sTq[BC][BC + 1];
    float(*sT)[BC + 1] = sTq;
    float(*sdAq)[BC + 1] = sTq;
    __shared__ float sbeta[BC], sdb1[NW][BC], sdb2[3][BC];

    const int H = p.H;
    const int gc = (int)blockIdx.x / H, h = (int)blockIdx.x % H;
    const int n = seq_of_chunk(p.cbase, p.N, gc);
    const int jc = gc - p.cbase[n];
    const int t0 = p.cu[n] + BC * jc;
    const int nv = min(BC, p.cu[n + 1] - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, q4 = lane >> 4;
    const IN_T *qg = static_cast<const IN_T *>(p.q), *kg = static_cast<const IN_T *>(p.k),
               *vg = static_cast<const IN_T *>(p.v);
    const size_t cb = blockIdx.x;
    const float *S = jc == 0 ? (p.s0 ? p.s0 + ((size_t)n * H + h) * DK * DV : nullptr)
                             : p.ckpt + ((size_t)(p.ck_base[n] + jc - 1) * H + h) * DK * DV;
    const float *D = p.Dck + cb * DK * DV;

    // staging: every load issued as a 16-byte vector before the first LDS write; rows past the
    // chunk read its last row and are zeroed (no branch around a load)
    {
        constexpr int VE = 16 / (int)sizeof(IN_T);                 // input elements per vector
        constexpr int NKV = BC * DK / VE, NGV = BC * DK / 4, NTA = 2 * BC * BC / 4;
        constexpr int UK = (NKV + NT - 1) / NT, UG = (NGV + NT - 1) / NT, UT = (NTA + NT - 1) / NT;
        uint4 kv[UK], qv[UK];
        float4 gv[UG], tav[UT];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int idx = min(tid + u * NT, NKV - 1), r = idx / (DK / VE), i = idx % (DK / VE) * VE;
            const size_t off = ((size_t)(t0 + min(r, nv - 1)) * H + h) * DK + i;
            kv[u] = *reinterpret_cast<const uint4 *>(kg + off);
            qv[u] = *reinterpret_cast<const uint4 *>(qg + off);
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            const int idx = min(tid + u * NT, NGV - 1), r = idx / (DK / 4), i = idx % (DK / 4) * 4;
            gv[u] = *reinterpret_cast<const float4 *>(p.g + ((size_t)(t0 + min(r, nv - 1)) * H + h) * DK + i);
        }
        const float *ta = p.TAk + cb * 2 * BC * BC;
#pragma unroll
        for (int u = 0; u < UT; ++u) tav[u] = *reinterpret_cast<const float4 *>(ta + 4 * min(tid + u * NT, NTA - 1));
        const float bv = p.beta[(size_t)(t0 + min(tid % BC, nv - 1)) * H + h];
        const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int idx = tid + u * NT, r = idx / (DK / VE), i = idx % (DK / VE) * VE;
            if (idx < NKV) {
                const bool ok = r < nv;
                *reinterpret_cast<uint4 *>(&sk[r][i]) =
                    make_uint4(ok ? kv[u].x : z.x, ok ? kv[u].y : z.y, ok ? kv[u].z : z.z, ok ? kv[u].w : z.w);
                *reinterpret_cast<uint4 *>(&sq[r][i]) =
                    make_uint4(ok ? qv[u].x : z.x, ok ? qv[u].y : z.y, ok ? qv[u].z : z.z, ok ? qv[u].w : z.w);
            }
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            const int idx = tid + u * NT, r = idx / (DK / 4), i = idx % (DK / 4) * 4;
            if (idx < NGV) *reinterpret_cast<float4 *>(&sb[r][i]) = keep4(r < nv, gv[u]);
        }
#pragma unroll
        for (int u = 0; u < UT; ++u) {
            const int e4 = 4 * (tid + u * NT);
            if (e4 < 2 * BC * BC) {
                const int rs = e4 % (BC * BC), r = rs / BC, s0c = rs % BC;
                float *dst = e4 < BC * BC ? &sA[r][s0c] : &sT[r][s0c];
                dst[0] = tav[u].x;
                dst[1] = tav[u].y;
                dst[2] = tav[u].z;
                dst[3] = tav[u].w;
            }
        }
        if (tid < BC) sbeta[tid] = tid < nv ? bv : 0.f;
    }
    __syncthreads();
    // cumulative log decay down the 32 rows: thread (column i, quarter qq) scans 8 rows, the
    // quarter totals pass through sz (free until stage 1 writes it)
    {
        const int i = tid % DK, qq = tid / DK;   // NT = 4 DK
        float a[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) a[r] = sb[8 * qq + r][i] + (r ? a[r - 1] : 0.f);
        sz[qq][i] = a[7];
        __syncthreads();
        float pre = 0.f;
        for (int u = 0; u < qq; ++u) pre += sz[u][i];
#pragma unroll
        for (int r = 0; r < 8; ++r) sb[8 * qq + r][i] = a[r] + pre;
    }
    __syncthreads();

    // ---- stage 1: value columns jj = 16 w + c
    {
        const int jj = 16 * w + c;
        f32x4_t X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // S and D tiles of column block jj, rows 16 kt + 4 q4 + e; the pair for k-tile kt + 1 loads
        // while the pair for kt is used.  YREC: Y = Kbar D comes from the one-workgroup scan's
        // record, so only S is read here.
        const float *Sc = (S ? S : D) + jj, *Dc = D + jj;
        auto products = [&](auto yrec_c) {
            constexpr bool YREC = decltype(yrec_c)::value;
            auto ld = [&](float (&sv)[4], float (&dv4)[4], int kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * kt + 4 * q4 + e;
                    sv[e] = S ? Sc[(size_t)i * DV] : 0.f;
                    dv4[e] = YREC ? 0.f : Dc[(size_t)i * DV];
                }
            };
            auto use = [&](const float (&sv)[4], const float (&dv4)[4], int kt) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int i = 16 * kt + 4 * q4 + kk, r = 16 * rt + c;
                        const float kv = widen(sk[r][i]), bi = sb[r][i];
                        X[rt] = mfma_f32(kv * __expf(bi), sv[kk], X[rt]);
                        if constexpr (!YREC) Y[rt] = mfma_f32(kv * __expf(sb[BC - 1][i] - bi), dv4[kk], Y[rt]);
                    }
            };
            float sa4[4], da4[4], sb4[4], db4[4];
            ld(sa4, da4, 0);
            for (int kt = 0; kt < DK / 16; kt += 2) {
                ld(sb4, db4, kt + 1);
                use(sa4, da4, kt);
                if (kt + 2 < DK / 16) ld(sa4, da4, kt + 2);
                use(sb4, db4, kt + 1);
            }
        };
        // (with rrec, X holds -R, read from the record: R = V - X below then takes no V)
        const bool rrec = p.pt && p.rrec;
        if (p.pt) {
            const float *yr = p.SCk + cb * ScanRec<DK>::SIZE + ScanRec<DK>::KB + jj;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[rt][e] = yr[(16 * rt + 4 * q4 + e) * DV];
            if (rrec) {
                const float *rr = p.SCk + cb * ScanRec<DK>::SIZE + ScanRec<DK>::RR + jj;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[rt][e] = -rr[(16 * rt + 4 * q4 + e) * DV];
            } else {
                products(std::true_type{});
            }
        } else {
            products(std::false_type{});
        }
        // dU = E + Kbar D, then dZ = T^T dU
        const float *ET = p.SCk + cb * ScanRec<DK>::SIZE + ScanRec<DK>::ET + jj * BC;
        float dU[2][4];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const float4 e4 = *reinterpret_cast<const float4 *>(ET + 16 * rg + 4 * q4);
            dU[rg][0] = e4.x + Y[rg][0];
            dU[rg][1] = e4.y + Y[rg][1];
            dU[rg][2] = e4.z + Y[rg][2];
            dU[rg][3] = e4.w + Y[rg][3];
        }
        f32x4_t dZ[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            dZ[st] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rg = st; rg < 2; ++rg)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) dZ[st] = mfma_f32(sT[16 * rg + 4 * q4 + kk][16 * st + c], dU[rg][kk], dZ[st]);
        }
        // R = V - X, Z = beta R; dv = beta dZ; dbeta part <dZ_r, R_r>
        float Zv[2][4];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * st + 4 * q4 + e;
                const bool ok = s < nv;
                const size_t off = ((size_t)(t0 + s) * H + h) * DV + jj;
                const float R = ok ? (rrec ? 0.f : load_in(vg + off)) - X[st][e] : 0.f;
                const float bs = sbeta[s];
                Zv[st][e] = bs * R;
                if (ok) p.dv[off] = bs * dZ[st][e];
                const float t = red16(dZ[st][e] * R);
                if (c == 0) sdb1[w][s] = t;
                if constexpr (HL) Mat<false>::put_hl1(szb, PLANE, s * PB + jj, dZ[st][e]);
                else sz[s][jj] = dZ[st][e];
            }
        // U = T Z
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st <= rt; ++st)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(sT[16 * rt + c][16 * st + 4 * q4 + kk], Zv[st][kk], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (HL) Mat<false>::put_hl1(sxb, PLANE, (16 * rt + 4 * q4 + e) * PB + jj, acc[e]);
                else sx[16 * rt + 4 * q4 + e][jj] = acc[e];
            }
        }
    }
    __syncthreads();

    // dO[t0 + r][h][j .. j + 3] (zero past the chunk's valid rows)
    auto do4 = [&](int r, int j) {
        return keep4(r < nv, *reinterpret_cast<const float4 *>(p.dO + ((size_t)(t0 + min(r, nv - 1)) * H + h) * DV + j));
    };

    // ---- stage 2: <dZ_r, U_s> -> dA (in place of A) and the A part of dbeta; <dO_r, U_s> -> dAq
    for (int it = w; it < 6; it += NW) {
        int rt, st, m;
        tile_of(it % 3, rt, st, m);
        const bool isq = it >= 3;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HL) {
            // 32 value columns per step: lane group q4, slot e <-> column 32 jb + 8 q4 + e
#pragma unroll 2
            for (int jb = 0; jb < DV / 32; ++jb) {
                const int j = 32 * jb + 8 * q4;
                Frag<false> A;
                if (isq) A = Mat<false>::from_tiles<true>(f4v(do4(16 * rt + c, j)), f4v(do4(16 * rt + c, j + 4)));
                else A = Mat<false>::get<true>(szb, PLANE, (16 * rt + c) * PB + j);
                const Frag<false> B = Mat<false>::get<true>(sxb, PLANE, (16 * st + c) * PB + j);
                mma<true, true>(acc, A, B);
            }
        } else {
            const float *xa = sz[16 * rt + c];
            const float *ub = sx[16 * st + c];
#pragma unroll 4
            for (int jg = 0; jg < DV / 16; ++jg) {
                const float4 a = isq ? do4(16 * rt + c, 16 * jg + 4 * q4)
                                     : *reinterpret_cast<const float4 *>(xa + 16 * jg + 4 * q4);
                const float4 u = *reinterpret_cast<const float4 *>(ub + 16 * jg + 4 * q4);
                acc = mfma_f32(a.x, u.x, acc);
                acc = mfma_f32(a.y, u.y, acc);
                acc = mfma_f32(a.z, u.z, acc);
                acc = mfma_f32(a.w, u.w, acc);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * q4 + e, s = 16 * st + c;
            if (isq) {
                sdAq[r][s] = s <= r ? p.scale * acc[e] : 0.f;
            } else {
                const bool keep = s < r;
                const float t = red16(keep ? -acc[e] * sA[r][s] : 0.f);
                if (c == 0) sdb2[it % 3][r] = t;
                sA[r][s] = keep ? -sbeta[r] * acc[e] : 0.f;
            }
        }
    }
    __syncthreads();

    if (tid < nv) {
        float a = tid < 16 ? sdb2[0][tid] : sdb2[1][tid] + sdb2[2][tid];
        for (int ww = 0; ww < NW; ++ww) a += sdb1[ww][tid];
        p.dbeta[(size_t)(t0 + tid) * H + h] = a;
    }

    // ---- stage 3: key channel i = 16 w + c
    {
        const int i = 16 * w + c;
        f32x4_t dQt[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t dKt[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t dKb[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        float rsd = 0.f;
        if constexpr (HL) {
            // row i of S and D, columns 32 m + 8 q4 .. + 7 (slot e <-> column 32 m + 8 q4 + e); the block
            // for m + 1 loads while m's is used
            const float *Sr = (S ? S : D) + (size_t)i * DV + 8 * q4, *Dr_ = D + (size_t)i * DV + 8 * q4;
            float4 sN0 = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr));
            float4 sN1 = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr + 4));
            float4 dN0 = *reinterpret_cast<const float4 *>(Dr_), dN1 = *reinterpret_cast<const float4 *>(Dr_ + 4);
            for (int m = 0; m < DV / 32; ++m) {
                const int j = 32 * m + 8 * q4;
                const float4 s0 = sN0, s1 = sN1, d0 = dN0, d1 = dN1;
                if (m + 1 < DV / 32) {
                    sN0 = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr + 32 * (m + 1)));
                    sN1 = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr + 32 * (m + 1) + 4));
                    dN0 = *reinterpret_cast<const float4 *>(Dr_ + 32 * (m + 1));
                    dN1 = *reinterpret_cast<const float4 *>(Dr_ + 32 * (m + 1) + 4);
                }
                rsd += s0.x * d0.x + s0.y * d0.y + s0.z * d0.z + s0.w * d0.w;
                rsd += s1.x * d1.x + s1.y * d1.y + s1.z * d1.z + s1.w * d1.w;
                const Frag<false> Bs = Mat<false>::from_tiles<true>(f4v(s0), f4v(s1));
                const Frag<false> Bd = Mat<false>::from_tiles<true>(f4v(d0), f4v(d1));
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const Frag<false> Ao =
                        Mat<false>::from_tiles<true>(f4v(do4(16 * rt + c, j)), f4v(do4(16 * rt + c, j + 4)));
                    const Frag<false> Az = Mat<false>::get<true>(szb, PLANE, (16 * rt + c) * PB + j);
                    const Frag<false> Au = Mat<false>::get<true>(sxb, PLANE, (16 * rt + c) * PB + j);
                    mma<true, true>(dQt[rt], Ao, Bs);
                    mma<true, true>(dKt[rt], Az, Bs);
                    mma<true, true>(dKb[rt], Au, Bd);
                }
            }
        } else {
        // row i of S and D, columns 16 jg + 4 q4 ..; the pair for jg + 1 loads while jg's is used
        const float *Sr = (S ? S : D) + (size_t)i * DV + 4 * q4, *Dr_ = D + (size_t)i * DV + 4 * q4;
        float4 sN = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr));
        float4 dN = *reinterpret_cast<const float4 *>(Dr_);
        for (int jg = 0; jg < DV / 16; ++jg) {
            const int j = 16 * jg + 4 * q4;
            const float4 s4 = sN, d4 = dN;
            if (jg + 1 < DV / 16) {
                sN = keep4(S != nullptr, *reinterpret_cast<const float4 *>(Sr + 16 * (jg + 1)));
                dN = *reinterpret_cast<const float4 *>(Dr_ + 16 * (jg + 1));
            }
            rsd += s4.x * d4.x + s4.y * d4.y + s4.z * d4.z + s4.w * d4.w;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float4 o4 = do4(16 * rt + c, j);
                const float4 z4 = *reinterpret_cast<const float4 *>(&sz[16 * rt + c][j]);
                const float4 u4 = *reinterpret_cast<const float4 *>(&sx[16 * rt + c][j]);
                dQt[rt] = mfma_f32(o4.x, s4.x, dQt[rt]);
                dQt[rt] = mfma_f32(o4.y, s4.y, dQt[rt]);
                dQt[rt] = mfma_f32(o4.z, s4.z, dQt[rt]);
                dQt[rt] = mfma_f32(o4.w, s4.w, dQt[rt]);
                dKt[rt] = mfma_f32(z4.x, s4.x, dKt[rt]);
                dKt[rt] = mfma_f32(z4.y, s4.y, dKt[rt]);
                dKt[rt] = mfma_f32(z4.z, s4.z, dKt[rt]);
                dKt[rt] = mfma_f32(z4.w, s4.w, dKt[rt]);
                dKb[rt] = mfma_f32(u4.x, d4.x, dKb[rt]);
                dKb[rt] = mfma_f32(u4.y, d4.y, dKb[rt]);
                dKb[rt] = mfma_f32(u4.z, d4.z, dKb[rt]);
                dKb[rt] = mfma_f32(u4.w, d4.w, dKb[rt]);
            }
        }
        }
        rsd += shfl_xor(rsd, 16);
        rsd += shfl_xor(rsd, 32);   // rowsum(S * D) of row i

        // pair terms of A and Aq, tile by tile with the tile's reference row m
        f32x4_t G1[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t G3[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t G24[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int tl = 0; tl < 3; ++tl) {
            int rt, st, m;
            tile_of(tl, rt, st, m);
            const float bm = sb[m][i];
            // row side (output rows r of tile rt, contraction over s of tile st)
            f32x4_t t1 = {0.f, 0.f, 0.f, 0.f}, t3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 16 * st + 4 * q4 + kk;
                const float kh = widen(sk[s][i]) * __expf(bm - sb[s][i]);
                t1 = mfma_f32(sA[16 * rt + c][s], kh, t1);
                t3 = mfma_f32(sdAq[16 * rt + c][s], kh, t3);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = __expf(sb[16 * rt + 4 * q4 + e][i] - bm);
                G1[rt][e] += f * t1[e];
                G3[rt][e] += f * t3[e];
            }
            // column side (output rows s of tile st, contraction over r of tile rt)
            f32x4_t t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r = 16 * rt + 4 * q4 + kk;
                const float f = __expf(sb[r][i] - bm);
                t2 = mfma_f32(sA[r][16 * st + c], widen(sk[r][i]) * f, t2);
                t2 = mfma_f32(sdAq[r][16 * st + c], widen(sq[r][i]) * f, t2);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) G24[st][e] += __expf(bm - sb[16 * st + 4 * q4 + e][i]) * t2[e];
        }

        // assemble dq, dk and dB (into sb: this wave's columns only, after its last read of them).
        // Output addresses: a scalar base per row (from a chunk start the compiler cannot hoist,
        // which would keep 64-bit row offsets live through stages 1-3 and spill them) plus a 32-bit
        // lane offset.
        const size_t rowb = ((size_t)opaque_s(t0) * H + h) * DK;
        const unsigned lo_ = (unsigned)(4 * q4 * H * DK + i);
        const float bl = sb[BC - 1][i];
        float cs = 0.f, dBv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * q4 + e;
                const float br = sb[r][i], gm = __expf(br), eb = __expf(bl - br);
                const float dqv = gm * p.scale * dQt[rt][e] + G3[rt][e];
                const float dkp = -gm * sbeta[r] * dKt[rt][e] + G1[rt][e];
                const float kbg = eb * dKb[rt][e];
                const float dkm = kbg + G24[rt][e];
                const float kr = widen(sk[r][i]);
                cs += kr * kbg;
                dBv[rt][e] = widen(sq[r][i]) * dqv + kr * (dkp - dkm);
                if (r < nv) {
                    const size_t rs = rowb + (size_t)(16 * rt + e) * H * DK;   // (scalar)
                    (p.dq + rs)[lo_] = dqv;
                    (p.dk + rs)[lo_] = dkp + dkm;
                }
            }
        cs += shfl_xor(cs, 16);
        cs += shfl_xor(cs, 32);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sb[16 * rt + 4 * q4 + e][i] = dBv[rt][e];
        // dB of the last row also carries dL/dB_last; dg = reverse cumulative sum over the chunk:
        // lane (c, q4) sums rows 8 q4 .. 8 q4 + 7 of column i, the quarter totals pass by shuffles
        wave_lds_sync();
        if (q4 == 0) sb[nv - 1][i] += cs + __expf(bl) * rsd;
        wave_lds_sync();
        float a[8];
#pragma unroll
        for (int r = 7; r >= 0; --r) a[r] = (8 * q4 + r < nv ? sb[8 * q4 + r][i] : 0.f) + (r < 7 ? a[r + 1] : 0.f);
        // totals of quarters q4 ^ 1, q4 ^ 2, q4 ^ 3; each quarter adds those of the later ones
        const float t1 = shfl_xor(a[0], 16), t2 = shfl_xor(a[0], 32), t3 = shfl_xor(t1, 32);
        const float later = q4 == 0 ? t1 + t2 + t3 : q4 == 1 ? t2 + t3 : q4 == 2 ? t1 : 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (8 * q4 + r < nv) p.dg[((size_t)(t0 + 8 * q4 + r) * H + h) * DK + i] = a[r] + later;
    }
}

// ---- fused prologue: the operator's inputs from the raw ones, and the chain rule back ---------
// g = -5 sigmoid(a), beta = sigmoid(b), q / |q| and k / |k| over d_k (the skill card's quick facts:
// lower-bounded scaled sigmoid, g_min = -5).  One wave per (token, head) row; lane l holds the
// row's elements l, l + 64, ...
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += shfl_xor(x, off);
    return x;
}

// With the normalisation the unit vectors stay fp32 (as in the forward's fused prologue), so the
// rest of the backward runs on fp32 inputs and v is widened alongside.
template <int DK>
__global__ void __launch_bounds__(256) prologue_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                            const uint16_t *__restrict__ v, const uint16_t *__restrict__ a,
                                                            const float *__restrict__ b, long long rows, int flags,
                                                            float *__restrict__ qn, float *__restrict__ kn,
                                                            float *__restrict__ vf, float *__restrict__ g,
                                                            float *__restrict__ beta) {
    constexpr int EPL = DK / 64;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;   // whole waves
    const size_t base = (size_t)row * DK + lane;
    if (flags & KDA_PRO_NORM) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const uint16_t *src = which ? k : q;
            float *dst = which ? kn : qn;
            float x[EPL], ss = 0.f;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                x[m] = bf16_bits_to_f32(src[base + 64 * m]);
                ss += x[m] * x[m];
            }
            ss = wave_sum(ss);
            const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;   // a zero row stays zero
#pragma unroll
            for (int m = 0; m < EPL; ++m) dst[base + 64 * m] = x[m] * inv;
        }
#pragma unroll
        for (int m = 0; m < EPL; ++m) vf[base + 64 * m] = bf16_bits_to_f32(v[base + 64 * m]);
    }
    if (flags & KDA_PRO_GATE) {
#pragma unroll
        for (int m = 0; m < EPL; ++m) g[base + 64 * m] = -5.f / (1.f + __expf(-bf16_bits_to_f32(a[base + 64 * m])));
        if (lane == 0) beta[row] = 1.f / (1.f + __expf(-b[row]));
    }
}

// dL/d(raw) from dL/d(prologue output), in place: dq <- (dq - q_n <q_n, dq>) / |q| (the same for k),
// dg <- dg * (-5) s (1 - s) with s = sigmoid(a), dbeta <- dbeta * beta (1 - beta).
template <int DK>
__global__ void __launch_bounds__(256) bwd_epilogue_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                            const uint16_t *__restrict__ a, const float *__restrict__ b,
                                                            long long rows, int flags, float *__restrict__ dq,
                                                            float *__restrict__ dk, float *__restrict__ dg,
                                                            float *__restrict__ dbeta) {
    constexpr int EPL = DK / 64;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;   // whole waves
    const size_t base = (size_t)row * DK + lane;
    if (flags & KDA_PRO_NORM) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const uint16_t *src = which ? k : q;
            float *d = which ? dk : dq;
            float x[EPL], dx[EPL], ss = 0.f;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                x[m] = bf16_bits_to_f32(src[base + 64 * m]);
                dx[m] = d[base + 64 * m];
                ss += x[m] * x[m];
            }
            ss = wave_sum(ss);
            const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
            float dot = 0.f;
#pragma unroll
            for (int m = 0; m < EPL; ++m) dot += x[m] * inv * dx[m];
            dot = wave_sum(dot);
#pragma unroll
            for (int m = 0; m < EPL; ++m) d[base + 64 * m] = (dx[m] - x[m] * inv * dot) * inv;
        }
    }
    if (flags & KDA_PRO_GATE) {
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            const float sg = 1.f / (1.f + __expf(-bf16_bits_to_f32(a[base + 64 * m])));
            dg[base + 64 * m] *= -5.f * sg * (1.f - sg);
        }
        if (lane == 0) {
            const float sb = 1.f / (1.f + __expf(-b[row]));
            dbeta[row] *= sb * (1.f - sb);
        }
    }
}

}  // namespace kda

extern "C" size_t kda_chunk_workspace_layout(int N, size_t *order_off, size_t *base_off);

// Backward workspace: [forward plan][chunk bases][checkpoints every 32][D per chunk]
// [scan operands per chunk][A, T per chunk][with the fused prologue: q_n, k_n, v (fp32, with the
// normalisation), g, beta (with the gate)].
extern "C" __attribute__((visibility("hidden"))) size_t kda_bwd_workspace_layout(int N, int H, int T, int dk, int dv,
                                                                                  int64_t n_ck, int64_t n_chunks,
                                                                                  int flags, size_t *off) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rec = dk == 128 ? kda::ScanRec<128>::SIZE : kda::ScanRec<64>::SIZE;
    size_t o[12];
    o[0] = up(kda_chunk_workspace_layout(N, nullptr, nullptr));           // cbase
    o[1] = o[0] + up((size_t)(N + 1) * 4);                                 // checkpoints
    const bool given = flags & kda::KDA_BWD_STATES_GIVEN;
    o[2] = o[1] + (given ? 0 : up((size_t)n_ck * H * dk * dv * 4));         // (no region)
    o[3] = o[2];                                                            // D
    o[4] = o[3] + up((size_t)n_chunks * H * dk * dv * 4);                   // scan operands
    o[5] = o[4] + up((size_t)n_chunks * H * rec * 4);                       // A, T
    o[6] = o[5] + up((size_t)n_chunks * H * 2 * kda::BC * kda::BC * 4);     // q_n
    const bool nrm = flags & kda::KDA_PRO_NORM, gate = flags & kda::KDA_PRO_GATE;
    o[7] = o[6] + (nrm ? up((size_t)T * H * dk * 4) : 0);                  // k_n
    o[8] = o[7] + (nrm ? up((size_t)T * H * dk * 4) : 0);                  // v (fp32)
    o[9] = o[8] + (nrm ? up((size_t)T * H * dv * 4) : 0);                  // g
    o[10] = o[9] + (gate ? up((size_t)T * H * dk * 4) : 0);                // beta
    o[11] = o[10] + (gate ? up((size_t)T * H * 4) : 0);                    // end
    if (off)
        for (int i = 0; i < 12; ++i) off[i] = o[i];
    return o[11];
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_chunk(
    int chunk, int dk, int in_bf16, int N, int H, const void *q, const void *k, const void *v, const float *g,
    const float *beta, const int32_t *cu, const float *s0, float *sf, int every, float *ckpt, float *o, float scale,
    const int32_t *s0_idx, const int32_t *ck_idx, int nslots, int flags, void *workspace, hipStream_t stream);
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_plan(int N, const int32_t *cu, int every,
                                                                           void *workspace, hipStream_t stream);
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_chunk32_split(int dk, int in_bf16, unsigned chains,
                                                                                    const kda::ChunkParams &p,
                                                                                    int max_split, hipStream_t stream);


// The fused prologue's outputs, materialised (one wave per (token, head) row; see prologue_kernel):
// with KDA_PRO_NORM fp32 q / |q|, k / |k| and v into qn, kn, vf; with KDA_PRO_GATE fp32 g, beta.
// q, k, v are bf16, a (in g's place) bf16 and b fp32, as the ABI's gate_mode defines them.
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_prologue(
    int dk, long long rows, int flags, const void *q, const void *k, const void *v, const float *a, const float *b,
    float *qn, float *kn, float *vf, float *g, float *beta, hipStream_t stream) {
    if (rows <= 0 || flags == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    const uint16_t *qr = static_cast<const uint16_t *>(q), *kr = static_cast<const uint16_t *>(k);
    const uint16_t *vr = static_cast<const uint16_t *>(v), *ar = reinterpret_cast<const uint16_t *>(a);
    if (dk == 128)
        hipLaunchKernelGGL(kda::prologue_kernel<128>, dim3(blocks), dim3(256), 0, stream, qr, kr, vr, ar, b, rows,
                           flags, qn, kn, vf, g, beta);
    else if (dk == 64)
        hipLaunchKernelGGL(kda::prologue_kernel<64>, dim3(blocks), dim3(256), 0, stream, qr, kr, vr, ar, b, rows,
                           flags, qn, kn, vf, g, beta);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// out[i] = cu[first + i] - cu[first], i = 0 .. n: a group's sequence offsets from its first token.
__global__ void __launch_bounds__(256) cu_rebase_kernel(const int32_t *__restrict__ cu, int first, int n,
                                                        int32_t *__restrict__ out) {
    const int32_t base = cu[first];
    for (int i = (int)threadIdx.x; i <= n; i += blockDim.x) out[i] = cu[first + i] - base;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_cu_rebase(const int32_t *cu, int first, int n,
                                                                                int32_t *out, hipStream_t stream) {
    hipLaunchKernelGGL(cu_rebase_kernel, dim3(1), dim3(256), 0, stream, cu, first, n, out);
    return hipGetLastError();
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_bwd(
    int dk, int in_bf16, int N, int H, int T, int64_t n_ck, int64_t n_chunks, const void *q, const void *k,
    const void *v, const float *g, const float *beta, const int32_t *cu, const float *s0, const float *dO,
    const float *dSf, float *dq, float *dkk, float *dv, float *dg, float *dbeta, float *dS0, float scale,
    const float *states, int flags, void *workspace, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    if (states) flags |= kda::KDA_BWD_STATES_GIVEN;
    const int given = flags & kda::KDA_BWD_STATES_GIVEN;
    const bool one_wg = flags & kda::KDA_BWD_ONE_WG_SCAN;
    flags &= kda::KDA_PRO_GATE | kda::KDA_PRO_NORM;   // the prologue bits from here on
    size_t off[12];
    kda_bwd_workspace_layout(N, H, T, dk, dk, n_ck, n_chunks, flags | given, off);
    char *ws = static_cast<char *>(workspace);
    hipError_t e;
    // fused prologue: the operator's inputs, materialised (fp32 q_n, k_n, v; fp32 g, beta) for
    // the per-chunk kernels; the forward recompute applies the prologue itself, exactly as the
    // forward does
    const void *q_raw = q, *k_raw = k, *v_raw = v;
    const float *a_raw = g, *b_raw = beta;
    const int raw_bf16 = in_bf16;
    const long long rows = (long long)T * H;
    const unsigned row_blocks = (unsigned)((rows + 3) / 4);
    if (flags && rows > 0) {
        float *qn = reinterpret_cast<float *>(ws + off[6]), *kn = reinterpret_cast<float *>(ws + off[7]);
        float *vf = reinterpret_cast<float *>(ws + off[8]);
        float *gm = reinterpret_cast<float *>(ws + off[9]), *bm = reinterpret_cast<float *>(ws + off[10]);
        if ((e = kda_launch_prologue(dk, rows, flags, q, k, v, g, beta, qn, kn, vf, gm, bm, stream)) != hipSuccess)
            return e;
        if (flags & kda::KDA_PRO_NORM) { q = qn; k = kn; v = vf; in_bf16 = 0; }
        if (flags & kda::KDA_PRO_GATE) { g = gm; beta = bm; }
    }
    // states at every 32-token boundary, without the outputs (the forward's plan lands at the start
    // of the workspace); the forward's fused prologue exists for d = 128, at d = 64 the recompute
    // reads the materialised inputs
    // (given by the caller instead: the launch plan alone)
    const bool fused_fwd = flags && dk == 128;
    // With the one-workgroup scan on few chains (two workgroups per chain fit the chip), the
    // recompute runs on the side stream, one workgroup per chain, at the same time as the scan;
    // the plan is made here first for both.  Otherwise it runs before everything else.
    // With the one-workgroup scan (d = 128, bf16 error budget) the recompute is launched here (own):
    // it also leaves R = V - (Gam K) S in each chunk's record for the gradient kernel.  On few
    // chains (two workgroups per chain fit the chip) it runs on the side stream, one workgroup per
    // chain, at the same time as the scan; otherwise first, on the caller's stream.
    const bool own = !given && one_wg && dk == 128 && (in_bf16 || raw_bf16);
    const bool side = own && 2LL * N * H <= (long long)kda_cu_count();
    // chunk bases first: the recompute's R records are indexed by them
    hipLaunchKernelGGL(kda::bwd_plan_kernel, dim3(1), dim3(1024), 0, stream, cu, N,
                       reinterpret_cast<int32_t *>(ws + off[0]));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (given || own)
        e = kda_launch_plan(N, cu, kda::BC, ws, stream);
    else
        e = kda_launch_chunk(32, dk, fused_fwd ? raw_bf16 : in_bf16, N, H, fused_fwd ? q_raw : q,
                             fused_fwd ? k_raw : k, fused_fwd ? v_raw : v, fused_fwd ? a_raw : g,
                             fused_fwd ? b_raw : beta, cu, s0, nullptr, kda::BC,
                             reinterpret_cast<float *>(ws + off[1]), nullptr, scale, nullptr, nullptr, 0,
                             (fused_fwd ? flags : 0) | kda::KDA_STATES_ONLY, ws, stream);
    if (e != hipSuccess) return e;
    size_t order_off, base_off;
    kda_chunk_workspace_layout(N, &order_off, &base_off);
    kda::ChunkParams cp;
    cp.q = fused_fwd ? q_raw : q; cp.k = fused_fwd ? k_raw : k; cp.v = fused_fwd ? v_raw : v;
    cp.g = fused_fwd ? a_raw : g; cp.beta = fused_fwd ? b_raw : beta;
    cp.cu_seqlens = cu;
    cp.order = reinterpret_cast<const int32_t *>(ws + order_off);
    cp.ckpt_base = reinterpret_cast<const int64_t *>(ws + base_off);
    cp.s0 = s0; cp.sf = nullptr; cp.ckpt = reinterpret_cast<float *>(ws + off[1]); cp.o = nullptr;
    cp.s0_idx = nullptr; cp.ck_idx = nullptr; cp.nslots = 0; cp.s0_slots = 0;
    cp.flags = (fused_fwd ? flags : 0) | kda::KDA_STATES_ONLY;
    cp.H = H; cp.every = kda::BC; cp.scale = scale; cp.nseq = N;
    cp.o_tr = nullptr; cp.ckpt_tr = nullptr;
    cp.rres = own ? reinterpret_cast<float *>(ws + off[4]) + kda::ScanRec<128>::RR : nullptr;
    cp.rbase = reinterpret_cast<const int32_t *>(ws + off[0]);
    cp.rstride = kda::ScanRec<128>::SIZE;
    const int rec_bf16 = fused_fwd ? raw_bf16 : in_bf16;
    const unsigned chains = (unsigned)N * (unsigned)H;
    if (own && !side &&
        (e = kda_launch_chunk32_split(dk, rec_bf16, chains, cp, 2, stream)) != hipSuccess)
        return e;
    // the side stream's recompute: forked after the prep kernel (so that it shares the chip with
    // the scan, not with the prep), joined before the gradient kernel
    bool forked = false;
    auto fork_recompute = [&]() -> hipError_t {
        const hipStream_t side_s = kda_side_fork(stream);
        if (!side_s)   // no side stream: the recompute goes on the caller's stream, before the scan
            return kda_launch_chunk32_split(dk, rec_bf16, chains, cp, 2, stream);
        forked = true;
        const hipError_t r = kda_launch_chunk32_split(dk, rec_bf16, chains, cp, 1, side_s);
        const hipError_t j = kda_side_forked();
        return r != hipSuccess ? r : j;
    };
    auto join_recompute = [&]() -> hipError_t { return forked ? kda_side_join(stream) : hipSuccess; };
    kda::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.cu = cu;
    p.order = reinterpret_cast<const int32_t *>(ws + order_off);
    p.ck_base = reinterpret_cast<const int64_t *>(ws + base_off);
    p.cbase = reinterpret_cast<const int32_t *>(ws + off[0]);
    p.ckpt = given ? states : reinterpret_cast<const float *>(ws + off[1]);
    p.s0 = s0; p.dO = dO; p.dSf = dSf;
    p.Dck = reinterpret_cast<float *>(ws + off[3]);
    p.SCk = reinterpret_cast<float *>(ws + off[4]);
    p.TAk = reinterpret_cast<float *>(ws + off[5]);
    p.dq = dq; p.dk = dkk; p.dv = dv; p.dg = dg; p.dbeta = dbeta; p.dS0 = dS0;
    p.N = N; p.H = H; p.scale = scale;
    p.rrec = own;
    const unsigned chunk_blocks = (unsigned)(n_chunks * H);
    const unsigned scan_blocks = (unsigned)N * (unsigned)H * (unsigned)(dk / 16);
    // (with the normalising prologue the inputs are fp32 unit vectors, the error budget bf16's)
    // (d = 128 with bf16 error budgets, on batches that suit it: the scan takes one workgroup per
    // chain and forms R itself)
#define KDA_BWD(DKV, T_, HL_)                                                                                      \
    do {                                                                                                           \
        const bool one = DKV == 128 && HL_ && one_wg;                                                              \
        p.pt = one;                                                                                                \
        if (chunk_blocks)                                                                                          \
            hipLaunchKernelGGL((kda::bwd_prep_kernel<DKV, T_>), dim3(chunk_blocks), dim3(DKV * 4), 0, stream, p); \
        if (side && (e = fork_recompute()) != hipSuccess) return e;                                                \
        if (one)                                                                                                   \
            hipLaunchKernelGGL((kda::bwd_dscan_hl_kernel<128>), dim3((unsigned)N * (unsigned)H), dim3(512), 0,     \
                               stream, p);                                                                         \
        else                                                                                                       \
            hipLaunchKernelGGL((kda::bwd_dstate_kernel<DKV>), dim3(scan_blocks), dim3(256), 0, stream, p);         \
        if (side && (e = join_recompute()) != hipSuccess) return e;                                                \
        if (chunk_blocks)                                                                                          \
            hipLaunchKernelGGL((kda::bwd_grad_kernel<DKV, T_, HL_>), dim3(chunk_blocks), dim3(DKV * 4), 0, stream, \
                               p);                                                                                 \
    } while (0)
    if (dk == 128 && in_bf16) KDA_BWD(128, uint16_t, true);
    else if (dk == 128 && raw_bf16) KDA_BWD(128, float, true);
    else if (dk == 128) KDA_BWD(128, float, false);
    else if (dk == 64 && in_bf16) KDA_BWD(64, uint16_t, true);
    else if (dk == 64 && raw_bf16) KDA_BWD(64, float, true);
    else if (dk == 64) KDA_BWD(64, float, false);
    else return hipErrorInvalidValue;
#undef KDA_BWD
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // fused prologue: gradients with respect to the raw inputs
    if (flags && rows > 0) {
        const uint16_t *qr = static_cast<const uint16_t *>(q_raw), *kr = static_cast<const uint16_t *>(k_raw);
        const uint16_t *ar = reinterpret_cast<const uint16_t *>(a_raw);
        if (dk == 128)
            hipLaunchKernelGGL(kda::bwd_epilogue_kernel<128>, dim3(row_blocks), dim3(256), 0, stream, qr, kr, ar, b_raw,
                               rows, flags, dq, dkk, dg, dbeta);
        else
            hipLaunchKernelGGL(kda::bwd_epilogue_kernel<64>, dim3(row_blocks), dim3(256), 0, stream, qr, kr, ar, b_raw,
                               rows, flags, dq, dkk, dg, dbeta);
    }
    return hipGetLastError();
}
