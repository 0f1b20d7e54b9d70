// kda_decode.hip -- one-token KDA state update, in place (gfx950).
//
// Per (sequence n, head h), with alpha = exp(g):
//     a = (alpha * q)^T S          read-out of the decayed state
//     p = (alpha * k)^T S          prediction of v from the decayed state
//     u = beta * (v - p)           delta-rule residual
//     o = scale * (a + (q . k) u)  = scale * S_new^T q
//     S <- Diag(alpha) S + k u^T   written back over S
// (the per-token step of the gated delta rule; "Attention->K3 course, Day 21",
// quiz Q9 for the residual write, interview answer D17 / quiz Q5: decode is a
// matrix-vector pass bound by memory bandwidth).
//
// The pass is HBM-bound: each state (d_k*d_v fp32) is read once and written
// once.  A workgroup holds a state in registers between the column reductions
// and the update, so S crosses HBM exactly twice.  Workgroups are persistent
// (one per compute unit, or fewer states) and walk the (n, h) states with a
// stride of the grid, loading the next state while they reduce and write back
// the current one, so every compute unit keeps reads in flight throughout.
// Thread t owns 4 consecutive columns (float4) of every RG-th row: a wave's
// loads cover whole rows and are fully coalesced.
//
// PRO (compile-time, KDA_PRO_* bits): the prologue of the skill card's quick facts,
// g = -5 sigmoid(a) from bf16 pre-activations a in g's place and beta = sigmoid(b), and/or
// q and k divided by their L2 norm over d_k (a zero vector stays zero).
#include "kda_common.h"

namespace kda {

constexpr int DEC_THREADS = 1024;

template <int DK, int DV, typename IN_T, int PRO = 0>
__global__ void __launch_bounds__(DEC_THREADS)
decode_kernel(const IN_T *__restrict__ q, const IN_T *__restrict__ k, const IN_T *__restrict__ v,
              const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
              const int32_t *__restrict__ slots, int nslots, float *__restrict__ o, int H, int NH,
              float scale) {
    constexpr int CG = DV / 4;                 // column groups (float4 each)
    constexpr int RG = DEC_THREADS / CG;       // row groups
    constexpr int RPT = DK / RG;               // rows per thread
    constexpr int NWAVE = DEC_THREADS / 64;
    static_assert(DK % RG == 0 && CG <= 64 && 64 % CG == 0, "shape");

    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;

    __shared__ float s_aq[DK], s_ak[DK], s_al[DK], s_k[DK], s_qk[DK], s_v[DV];
    __shared__ float s_red[NWAVE][CG][9];

    // state slot of (n, h) = nh: n itself, or the pool slot slots[n]; -1 (or out of range) when
    // the sequence is inactive (no state access, o = 0)
    auto slot_of = [&](int nh_) -> long long {
        const int n = nh_ / H, h = nh_ - n * H;
        const long long sl = slots ? (long long)slots[n] : (long long)n;
        return sl >= 0 && sl < nslots ? sl * H + h : -1;
    };
    int nh = blockIdx.x;                       // n * H + h
    long long sl = slot_of(nh);
    f32x4_t s[RPT], sn[RPT];                   // this state, the next one
    if (sl >= 0) {
        const f32x4_t *S4 = reinterpret_cast<const f32x4_t *>(state + sl * DK * DV);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(&S4[(rg + RG * m) * CG + cg]);
    }
    for (; nh < NH; nh += gridDim.x) {
        const int nxt = nh + (int)gridDim.x;
        const long long sln = nxt < NH ? slot_of(nxt) : -1;
        if (sln >= 0) {
            const f32x4_t *S4n = reinterpret_cast<const f32x4_t *>(state + sln * DK * DV);
#pragma unroll
            for (int m = 0; m < RPT; ++m) sn[m] = __builtin_nontemporal_load(&S4n[(rg + RG * m) * CG + cg]);
        }
        if (sl < 0) {
            // inactive sequence: o = 0, state untouched
            const size_t tok_v = (size_t)nh * DV;
            if (rg == 0) reinterpret_cast<float4 *>(o + tok_v)[cg] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int m = 0; m < RPT; ++m) s[m] = sn[m];
            sl = sln;
            continue;
        }

        const size_t tok_k = (size_t)nh * DK, tok_v = (size_t)nh * DV;
        float qi = 0.f, ki = 0.f, gi = 0.f;
        if (t < DK) {
            qi = load_in(q + tok_k + t);
            ki = load_in(k + tok_k + t);
            if constexpr (PRO & KDA_PRO_GATE) {
                const float ai = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(g)[tok_k + t]);
                gi = -5.f * __builtin_amdgcn_rcpf(1.f + __expf(-ai));
            } else {
                gi = g[tok_k + t];
            }
        }
        if constexpr ((PRO & KDA_PRO_NORM) != 0) {
            // |q|^2 and |k|^2, formed by each of the first DK / 64 waves on its own (every lane
            // reads DK / 64 elements of each, then a wave reduction): no workgroup barrier
            if (t < DK) {
                const int ln = t & 63;
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int m = 0; m < DK / 64; ++m) {
                    const float x = load_in(q + tok_k + ln + 64 * m), y = load_in(k + tok_k + ln + 64 * m);
                    sq += x * x;
                    sk += y * y;
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    sq += shfl_xor(sq, off);
                    sk += shfl_xor(sk, off);
                }
                qi *= sq > 0.f ? rsqrtf(sq) : 0.f;
                ki *= sk > 0.f ? rsqrtf(sk) : 0.f;
            }
        }
        if (t < DK) {
            const float al = __expf(gi);
            s_al[t] = al;
            s_aq[t] = al * qi;
            s_ak[t] = al * ki;
            s_k[t] = ki;
            s_qk[t] = qi * ki;
        }
        if (t < DV) s_v[t] = load_in(v + tok_v + t);
        float b = beta[nh];
        if constexpr (PRO & KDA_PRO_GATE) b = __builtin_amdgcn_rcpf(1.f + __expf(-b));
        __syncthreads();

        float a[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0}, qk = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float aq = s_aq[i], ak = s_ak[i];
            a[0] += aq * s[m][0]; a[1] += aq * s[m][1]; a[2] += aq * s[m][2]; a[3] += aq * s[m][3];
            p[0] += ak * s[m][0]; p[1] += ak * s[m][1]; p[2] += ak * s[m][2]; p[3] += ak * s[m][3];
            qk += s_qk[i];   // every column group sums the same rows; column group 0 is used
        }

        // Reduce the 9 partials across the row groups: first inside the wave
        // (lanes with equal cg differ by multiples of CG), then across waves.
        float r9[9] = {a[0], a[1], a[2], a[3], p[0], p[1], p[2], p[3], qk};
#pragma unroll
        for (int off = CG; off < 64; off *= 2)
#pragma unroll
            for (int j = 0; j < 9; ++j) r9[j] += shfl_xor(r9[j], off);
        const int wave = t / 64, lane = t % 64;
        if (lane < CG)
#pragma unroll
            for (int j = 0; j < 9; ++j) s_red[wave][lane][j] = r9[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) acc += s_red[w][cg][j];
            r9[j] = acc;
        }
        const float qk_all = r9[8];   // every column group summed the same rows of q*k

        float u[4], ov[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] = b * (s_v[4 * cg + c] - r9[4 + c]);
            ov[c] = scale * (r9[c] + qk_all * u[c]);
        }
        if (rg == 0)
            reinterpret_cast<float4 *>(o + tok_v)[cg] = make_float4(ov[0], ov[1], ov[2], ov[3]);

        f32x4_t *S4 = reinterpret_cast<f32x4_t *>(state + sl * DK * DV);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float al = s_al[i], ki = s_k[i];
            f32x4_t r;
            r[0] = al * s[m][0] + ki * u[0];
            r[1] = al * s[m][1] + ki * u[1];
            r[2] = al * s[m][2] + ki * u[2];
            r[3] = al * s[m][3] + ki * u[3];
            __builtin_nontemporal_store(r, &S4[i * CG + cg]);
        }
        __syncthreads();   // the shared vectors and partials are rewritten for the next state
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = sn[m];
        sl = sln;
    }
}

}  // namespace kda

// Launcher used by the C ABI (kda_api.hip).  Returns a hipError_t.
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_decode(int dk, int in_bf16, int N, int H, const void *q, const void *k,
                                        const void *v, const float *g, const float *beta, float *state,
                                        const int32_t *slots, int nslots, float *o, float scale, int flags,
                                        hipStream_t stream) {
    if (N == 0 || H == 0) return hipSuccess;
    const long long nh = (long long)N * H;
    if (nh > 0x7fffffffLL) return hipErrorInvalidValue;
    // persistent: one workgroup per compute unit (or per state, if fewer)
    const int grid = (int)(nh < kda_cu_count() ? nh : kda_cu_count());
#define KDA_DEC(DKV, T, PRO)                                                                                   \
    hipLaunchKernelGGL((kda::decode_kernel<DKV, DKV, T, PRO>), dim3(grid), dim3(kda::DEC_THREADS), 0, stream,   \
                       (const T *)q, (const T *)k, (const T *)v, g, beta, state, slots, slots ? nslots : N, o,  \
                       H, (int)nh, scale)
#define KDA_DEC_PRO(DKV)                                                                                       \
    do {                                                                                                       \
        if (flags == 1) KDA_DEC(DKV, uint16_t, 1);                                                             \
        else if (flags == 2) KDA_DEC(DKV, uint16_t, 2);                                                        \
        else KDA_DEC(DKV, uint16_t, 3);                                                                        \
    } while (0)
    if (flags != 0) {
        // the prologue: bf16 inputs
        if (!in_bf16 || flags > 3) return hipErrorInvalidValue;
        if (dk == 128) KDA_DEC_PRO(128);
        else if (dk == 64) KDA_DEC_PRO(64);
        else return hipErrorInvalidValue;
    } else if (dk == 128 && in_bf16) KDA_DEC(128, uint16_t, 0);
    else if (dk == 128) KDA_DEC(128, float, 0);
    else if (dk == 64 && in_bf16) KDA_DEC(64, uint16_t, 0);
    else if (dk == 64) KDA_DEC(64, float, 0);
    else return hipErrorInvalidValue;
#undef KDA_DEC_PRO
#undef KDA_DEC
    return hipGetLastError();
}
