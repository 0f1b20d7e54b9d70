// kda_chunk.hip -- chunked KDA prefill over packed variable-length sequences (gfx950).
//
// Operator: per (sequence, head), tokens in order,
//     S <- Diag(exp(g_t)) S ;  u_t = beta_t (v_t - S^T k_t) ;  S <- S + k_t u_t^T ;  o_t = scale S^T q_t
// (the gated delta rule with a per-channel forget gate: "Attention->K3 course,
// Day 21", quiz Q9 and answer D19; skillsmp K3 skill card, quick facts).
//
// Chunk-recurrent form (chunk C = 64, the entering state S, G_r = log-decay
// summed over the chunk up to row r, Gamma = exp(G)):
//     A_kk[r,i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic}   (i <  r)
//     A_qk[r,i] =        sum_c q_rc k_ic e^{G_rc - G_ic}   (i <= r)
//     T   = (I + A_kk)^{-1} Diag(beta)
//     U   = T (V - (Gamma*K) S)                        delta-rule residuals of the chunk
//     O   = scale [ (Gamma*Q) S + A_qk U ]
//     S  <- Diag(Gamma_last) S + (e^{G_last - G} * K)^T U
// ("parallel inside a chunk, recurrent across chunks": scripod show notes,
// chapter 2.1; the bounded log-decay g >= -5 from the K3 skill card's quick
// facts is what lets the pairwise decay factor be split per 16-row sub-chunk,
// e^{G_r - G_i} = e^{G_r - G_ref} e^{G_ref - G_i}, with both factors inside fp32
// range because 16 * 5 = 80 < 88, so every Gram tile is a dense MFMA product).
//
// Design (one workgroup per (sequence, head), NW = d_v/16 waves):
//   * Decay factors come from exp(g) and running products inside each 16-row
//     sub-chunk (E_start: from the sub-chunk start, E_end: to its end), never
//     from exponentials of long sums.
//   * Gram tiles A_kk, A_qk: 10 lower 16x16 tiles each, as MFMA products of
//     Ks_a = k * E_start (rows of sub-chunk a) with Kn^(a)_b = k * e^{G_ref(a) - G}
//     (rows of sub-chunk b <= a); operands in hi+lo bf16 (3 MFMA passes).
//   * T: the four 16x16 diagonal inverses by forward substitution (one wave),
//     then the off-diagonal blocks by fp32-MFMA block products (32x32 blocked
//     inverse), in fp32.
//   * The recurrence is separable over value columns, so wave w owns value
//     columns [16w, 16w+16): it keeps its d_k x 16 slice of S in registers (fp32)
//     for the whole sequence and runs U, O and the state update for its slice
//     with no inter-wave traffic; the d_v-independent operands (T, A_qk,
//     Gamma*K, Gamma*Q, e^{G_last-G}*K) are shared through LDS.
//   * Precision (bf16 inputs): every product that feeds the outputs is formed
//     from hi+lo bf16 operand pairs except V - (Gamma*K) S, which uses single bf16
//     operands; accumulation is fp32; o and S are fp32.  The fp32 path uses fp32
//     MFMA throughout.
#include "kda_frag.h"

namespace kda {

constexpr int CH = 64;    // chunk size (tokens)

// ---- LDS map -------------------------------------------------------------------
template <int DK, bool F32P>
struct Lds {
    static constexpr int ES = Mat<F32P>::ES;
    // Gram phase (region G)
    static constexpr int KQS_PLANE = 64 * DK * ES;             // Ks, later Qs
    static constexpr int KN_PLANE = 160 * DK * ES;             // Kn^(a)_b, 10 row blocks
    static constexpr int KQS = 0;
    static constexpr int KN = KQS + 64 * DK * 4;
    static constexpr int G_END = KN + 160 * DK * 4;
    // scan operands (region X, aliases G)
    static constexpr int GK = 0;                               // Gamma*K   [64][DK]   single carrier
    static constexpr int QT_PLANE = 64 * DK * ES;              // Gamma*Q   [64][DK]   hl
    static constexpr int QT = GK + 64 * DK * ES;
    static constexpr int KHT_PLANE = DK * 64 * ES;             // (e^{G_last-G}*K)^T [DK][64]  hl
    static constexpr int KHT = QT + 64 * DK * 4;
    static constexpr int X_END = KHT + DK * 64 * 4;
    static_assert(X_END <= G_END, "scan operands must fit in the Gram region");
    // region Y: T and A_qk, 6 blocks each, hl
    static constexpr int TRI_PLANE = 6 * 64 * 8 * ES;
    static constexpr int TM = G_END;
    static constexpr int AQK = TM + 6 * 64 * 8 * 4;
    // region Z: 14 fp32 16x16 tiles for the inverse (L/M tiles 0..9, X tiles 10..13)
    static constexpr int Z = AQK + 6 * 64 * 8 * 4;
    static constexpr int XCHG = Z;                             // [8][DK] fp32 half-products, aliases Z
    static constexpr int Z_END = Z + 14 * TSZ * 4;
    static_assert(8 * DK * 4 <= 14 * TSZ * 4, "exchange buffer must fit in Z");
    static constexpr int BETA = Z_END;                         // [64] fp32
    static constexpr int GC = BETA + 64 * 4;                   // [DK] fp32
    static constexpr int TOTAL = GC + DK * 4;
};


template <int DK, bool F32P, typename IN_T>
__global__ void __launch_bounds__(DK * 4)
chunk_fwd_kernel(const ChunkParams p) {
    constexpr int DV = DK;
    constexpr int NW = DV / 16;          // waves; wave w owns value columns [16w, 16w+16)
    constexpr int NT = NW * 64;
    constexpr int KB = DK / 32;          // K-steps over d_k
    constexpr int KT = DK / 16;          // 16-row tiles over d_k
    constexpr int NCP = DK / 2;          // channel pairs
    using L = Lds<DK, F32P>;
    using M = Mat<F32P>;
    using F = Frag<F32P>;
    static_assert(NT / NCP == 8, "8 row groups of 8 rows");

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;

    const int h = blockIdx.x % p.H;
    const int n = p.order[blockIdx.x / p.H];
    const int seq_start = p.cu_seqlens[n];
    const int seq_len = p.cu_seqlens[n + 1] - seq_start;
    const int H = p.H;

    // Elementwise role (inside the chunk loop): channel pair cp (channels 2cp, 2cp+1),
    // rows [8 rg, 8 rg + 8), sub-chunk sa = rg/2, half hf = rg%2.
    // Scan role: value columns [j0, j0 + 16).
    const int j0 = 16 * wave;

    // Zero the structurally-zero tiles of T and A_qk (upper tiles (0,1) and (2,3)).
    for (int idx = tid; idx < 2 * 16 * 16; idx += NT) {
        const int t = idx >> 8, rr = (idx >> 4) & 15, cc = idx & 15;
        const int r = t == 0 ? rr : 32 + rr, c = t == 0 ? 16 + cc : 48 + cc;
        M::put_hl1(smem + L::TM, L::TRI_PLANE, tofs(r, c), 0.f);
        M::put_hl1(smem + L::AQK, L::TRI_PLANE, tofs(r, c), 0.f);
    }

    // State slice in registers: Sr[ct][e] = S[16 ct + 4 lq + e][j0 + lr].
    f32x4_t Sr[KT];
    const size_t st_off = ((size_t)n * H + h) * DK * DV;
    const long long s0o = s0_offset(p, n, h, DK * DV);
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sr[ct][e] = s0o >= 0 ? p.s0[s0o + (16 * ct + 4 * lq + e) * DV + j0 + lr] : 0.f;

    const IN_T *qg = reinterpret_cast<const IN_T *>(p.q);
    const IN_T *kg = reinterpret_cast<const IN_T *>(p.k);
    const IN_T *vg = reinterpret_cast<const IN_T *>(p.v);
    const int nchunks = (seq_len + CH - 1) / CH;

    for (int ci = 0; ci < nchunks; ++ci) {
        // Per-lane indices and LDS offsets are rederived every chunk (see opaque_v).
        char *const sm = smem + opaque_s(0);
        float *const zt = reinterpret_cast<float *>(sm + L::Z);
        float *const s_beta = reinterpret_cast<float *>(sm + L::BETA);
        float *const s_gc = reinterpret_cast<float *>(sm + L::GC);
        float *const s_xchg = reinterpret_cast<float *>(sm + L::XCHG);
        const int tid = opaque_v((int)threadIdx.x);
        const int lane = tid & 63;
        const int lr = lane & 15, lq = lane >> 4;
        const int cp = tid % NCP, rg = tid / NCP;
        const int c0 = 2 * cp;
        const int sa = rg >> 1, hf = rg & 1;
        const int t0 = seq_start + ci * CH;
        const int nvalid = min(CH, seq_len - ci * CH);

        // -- S1: inputs, per-channel decay products ------------------------------
        float kv[8][2], qv[8][2], Es[8][2], Ee[8][2];
        {
            float al[8][2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * rg + i;
                if (r < nvalid) {
                    const size_t off = ((size_t)(t0 + r) * H + h) * DK + c0;
                    kv[i][0] = load_in(kg + off); kv[i][1] = load_in(kg + off + 1);
                    qv[i][0] = load_in(qg + off); qv[i][1] = load_in(qg + off + 1);
                    const float2 gg = *reinterpret_cast<const float2 *>(p.g + off);
                    al[i][0] = __expf(gg.x); al[i][1] = __expf(gg.y);
                } else {
                    kv[i][0] = kv[i][1] = qv[i][0] = qv[i][1] = 0.f;
                    al[i][0] = al[i][1] = 1.f;
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float f = 1.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) { f *= al[i][c]; Es[i][c] = f; }
                float b = 1.f;
#pragma unroll
                for (int i = 7; i >= 0; --i) { Ee[i][c] = b; b *= al[i][c]; }
                s_xchg[rg * DK + c0 + c] = f;   // product over this row group
            }
            if (cp == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * rg + i;
                    s_beta[r] = r < nvalid ? p.beta[(size_t)(t0 + r) * H + h] : 0.f;
                }
            }
        }
        __syncthreads();
        float Pm[4][2], pre[2], post[2], cfac[4][2];
        {
            float hp[8][2];
#pragma unroll
            for (int m = 0; m < 8; ++m) { hp[m][0] = s_xchg[m * DK + c0]; hp[m][1] = s_xchg[m * DK + c0 + 1]; }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int m = 0; m < 4; ++m) Pm[m][c] = hp[2 * m][c] * hp[2 * m + 1][c];
                // rows of the first half before us / of the second half after us
                const float lead = hf ? s_xchg[(rg - 1) * DK + c0 + c] : 1.f;
                const float tail = hf ? 1.f : s_xchg[(rg + 1) * DK + c0 + c];
#pragma unroll
                for (int i = 0; i < 8; ++i) { Es[i][c] *= lead; Ee[i][c] *= tail; }
                float pr = 1.f, po = 1.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) { if (m < sa) pr *= Pm[m][c]; if (m > sa) po *= Pm[m][c]; }
                pre[c] = pr; post[c] = po;
                // column-side factor of tile (a', sa): 1/P_sa on the diagonal, else the
                // decay of the sub-chunks strictly between sa and a'
                float run = 1.f;
#pragma unroll
                for (int ap = 0; ap < 4; ++ap) {
                    if (ap == sa) cfac[ap][c] = 1.f / Pm[sa][c];
                    else if (ap > sa) { cfac[ap][c] = run; run *= Pm[ap][c]; }
                    else cfac[ap][c] = 0.f;
                }
            }
            if (rg == 0) {
                s_gc[c0] = Pm[0][0] * Pm[1][0] * Pm[2][0] * Pm[3][0];
                s_gc[c0 + 1] = Pm[0][1] * Pm[1][1] * Pm[2][1] * Pm[3][1];
            }
        }

        // -- S2: Gram operands Ks (rows of sub-chunk sa) and Kn^(a')_sa ------------------
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const float ks[2] = {kv[i][0] * Es[i][0], kv[i][1] * Es[i][1]};
            M::template put_hl<2>(sm + L::KQS, L::KQS_PLANE, fofs<KB>(r, c0), ks);
#pragma unroll
            for (int ap = 0; ap < 4; ++ap) {
                if (ap < sa) continue;
                const int vr = 16 * vidx(ap, sa) + (r - 16 * sa);
                const float kn[2] = {kv[i][0] * Ee[i][0] * cfac[ap][0], kv[i][1] * Ee[i][1] * cfac[ap][1]};
                M::template put_hl<2>(sm + L::KN, L::KN_PLANE, fofs<KB>(vr, c0), kn);
            }
        }
        __syncthreads();

        // -- S3: A_kk tiles (transposed products: lane holds A[16a+lr][16b+4lq+e]) --------
        for (int t = wave; t < 10; t += NW) {
            const int a = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int b = t - vidx(a, 0);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const F fa = M::template get<true>(sm + L::KN, L::KN_PLANE, fbase<KB>(vidx(a, b), s, lane));
                const F fb = M::template get<true>(sm + L::KQS, L::KQS_PLANE, fbase<KB>(a, s, lane));
                mma<true, true>(acc, fa, fb);
                __builtin_amdgcn_sched_barrier(0);
            }
            const float br = s_beta[16 * a + lr];
            float4 w;
            float *wv = reinterpret_cast<float *>(&w);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * lq + e;
                wv[e] = (b < a || i < lr) ? br * acc[e] : 0.f;
            }
            *reinterpret_cast<float4 *>(zt + vidx(a, b) * TSZ + lr * TP + 4 * lq) = w;
        }
        __syncthreads();

        // -- S4: Qs over Ks; diagonal blocks of (I + A_kk)^{-1} (wave 0) --------------
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const float qs[2] = {qv[i][0] * Es[i][0], qv[i][1] * Es[i][1]};
            M::template put_hl<2>(sm + L::KQS, L::KQS_PLANE, fofs<KB>(r, c0), qs);
        }
        if (wave == 0) {
            const int a = lane >> 4, j = lane & 15;
            float *Lt = zt + vidx(a, a) * TSZ;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= Lt[r * TP + i] * x[i];
                x[r] = acc;
                __builtin_amdgcn_sched_barrier(0);   // keep row loads next to their use
            }
            const float bj = s_beta[16 * a + j];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                Lt[r * TP + j] = x[r];
                M::put_hl1(sm + L::TM, L::TRI_PLANE, tofs(16 * a + r, 16 * a + j), x[r] * bj);
            }
        }
        __syncthreads();

        // -- S5: A_qk tiles; level-1 off-diagonal inverse blocks M10, M32 --------------
        for (int t = wave; t < 10; t += NW) {
            const int a = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int b = t - vidx(a, 0);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const F fa = M::template get<true>(sm + L::KN, L::KN_PLANE, fbase<KB>(vidx(a, b), s, lane));
                const F fb = M::template get<true>(sm + L::KQS, L::KQS_PLANE, fbase<KB>(a, s, lane));
                mma<true, true>(acc, fa, fb);
                __builtin_amdgcn_sched_barrier(0);
            }
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (b < a || 4 * lq + e <= lr) ? acc[e] : 0.f;
            M::template put_hl<4>(sm + L::AQK, L::TRI_PLANE, tofs(16 * a + lr, 16 * b + 4 * lq), w);
        }
        if (wave == NW - 1 || wave == NW - 2) {
            // M_{a,a-1} = -M_aa L_{a,a-1} M_{a-1,a-1} for a = 1 (wave NW-2) and a = 3 (wave NW-1)
            const int a = wave == NW - 2 ? 1 : 3;
            f32x4_t R = {0.f, 0.f, 0.f, 0.f}, Mo = {0.f, 0.f, 0.f, 0.f};
            tmm_ll(R, zt + vidx(a, a - 1) * TSZ, zt + vidx(a - 1, a - 1) * TSZ, lane);
            tmm_lr(Mo, zt + vidx(a, a) * TSZ, R, lane);
            const float bj = s_beta[16 * (a - 1) + lr];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Mo[e] = -Mo[e];
                M::put_hl1(sm + L::TM, L::TRI_PLANE, tofs(16 * a + 4 * lq + e, 16 * (a - 1) + lr), Mo[e] * bj);
            }
            tile_store(zt + vidx(a, a - 1) * TSZ, Mo, lane);
        }
        __syncthreads();

        // -- S6: scan operands (region X over G); X = L_BL M_TL (waves 0..3) ------------
        // -- value slice for the scan (consumed after the next two barriers) --------------
        f32x4_t Vt[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * lq + e;
                Vt[rt][e] = r < nvalid ? load_in(vg + ((size_t)(t0 + r) * H + h) * DV + j0 + lr) : 0.f;
            }

#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            M::put_h2(sm + L::GK, fofs<KB>(r, c0), kv[i][0] * Es[i][0] * pre[0], kv[i][1] * Es[i][1] * pre[1]);
            const float qt[2] = {qv[i][0] * Es[i][0] * pre[0], qv[i][1] * Es[i][1] * pre[1]};
            M::template put_hl<2>(sm + L::QT, L::QT_PLANE, fofs<KB>(r, c0), qt);
        }
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const int r = 8 * rg + i;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float kh[2] = {kv[i][c] * Ee[i][c] * post[c], kv[i + 1][c] * Ee[i + 1][c] * post[c]};
                M::template put_hl<2>(sm + L::KHT, L::KHT_PLANE, fofs<2>(c0 + c, r), kh);
            }
        }
        if (wave < 4) {
            // X_20 = L20 M00 + L21 M10 ; X_21 = L21 M11 ; X_30 = L30 M00 + L31 M10 ; X_31 = L31 M11
            const int a = 2 + (wave >> 1), b = wave & 1;
            f32x4_t X = {0.f, 0.f, 0.f, 0.f};
            if (b == 0) {
                tmm_ll(X, zt + vidx(a, 0) * TSZ, zt + vidx(0, 0) * TSZ, lane);
                tmm_ll(X, zt + vidx(a, 1) * TSZ, zt + vidx(1, 0) * TSZ, lane);
            } else {
                tmm_ll(X, zt + vidx(a, 1) * TSZ, zt + vidx(1, 1) * TSZ, lane);
            }
            tile_store(zt + (10 + wave) * TSZ, X, lane);
        }
        __syncthreads();

        // -- S7: M_BL = -M_BR X (waves 0..3) and its T blocks ------------------------------
        if (wave < 4) {
            const int a = 2 + (wave >> 1), b = wave & 1;
            f32x4_t Mo = {0.f, 0.f, 0.f, 0.f};
            if (a == 2) {
                tmm_ll(Mo, zt + vidx(2, 2) * TSZ, zt + (10 + b) * TSZ, lane);
            } else {
                tmm_ll(Mo, zt + vidx(3, 2) * TSZ, zt + (10 + b) * TSZ, lane);
                tmm_ll(Mo, zt + vidx(3, 3) * TSZ, zt + (12 + b) * TSZ, lane);
            }
            const float bj = s_beta[16 * b + lr];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                M::put_hl1(sm + L::TM, L::TRI_PLANE, tofs(16 * a + 4 * lq + e, 16 * b + lr), -Mo[e] * bj);
        }
        __syncthreads();

        // -- S8: scan for value columns [j0, j0+16) ------------------------------------------
        {
            // Y = V - (Gamma*K) S and Oa = (Gamma*Q) S, accumulated over d_k in 32-wide
            // steps so that only one step's S fragments are live at a time
            f32x4_t Y[4], Oa[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) { Y[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; Oa[rt] = Y[rt]; }
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const F sh = M::template from_tiles<false>(Sr[2 * s], Sr[2 * s + 1]);
                const F shl = M::template from_tiles<true>(Sr[2 * s], Sr[2 * s + 1]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const F fg = M::template get<false>(sm + L::GK, 0, fbase<KB>(rt, s, lane));
                    mma<false, false>(Y[rt], fg, sh);
                    const F fq = M::template get<true>(sm + L::QT, L::QT_PLANE, fbase<KB>(rt, s, lane));
                    mma<true, true>(Oa[rt], fq, shl);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[rt][e] = Vt[rt][e] - Y[rt][e];
            F YF[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) YF[s] = M::template from_tiles<true>(Y[2 * s], Y[2 * s + 1]);
            // U = T Y
            f32x4_t U[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= (rt >> 1); ++s) {
                    const F fa = M::template get<true>(sm + L::TM, L::TRI_PLANE, tbase(rt, s, lane));
                    mma<true, true>(acc, fa, YF[s]);
                }
                U[rt] = acc;
            }
            F UF[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) UF[s] = M::template from_tiles<true>(U[2 * s], U[2 * s + 1]);
            // O = scale [ (Gamma*Q) S + A_qk U ]
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4_t acc = Oa[rt];
#pragma unroll
                for (int s = 0; s <= (rt >> 1); ++s) {
                    const F fa = M::template get<true>(sm + L::AQK, L::TRI_PLANE, tbase(rt, s, lane));
                    mma<true, true>(acc, fa, UF[s]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * lq + e;
                    if (r < nvalid) p.o[((size_t)(t0 + r) * H + h) * DV + j0 + lr] = p.scale * acc[e];
                }
            }
            // S <- Diag(Gamma_last) S + (e^{G_last-G} K)^T U
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                f32x4_t acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = s_gc[16 * ct + 4 * lq + e] * Sr[ct][e];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const F fa = M::template get<true>(sm + L::KHT, L::KHT_PLANE, fbase<2>(ct, s, lane));
                    mma<true, true>(acc, fa, UF[s]);
                }
                Sr[ct] = acc;
            }
            // state snapshot at in-sequence positions that are multiples of `every`
            if (p.every > 0 && nvalid == CH && ((ci + 1) * CH) % p.every == 0) {
                const int64_t m = p.ckpt_base[n] + ((ci + 1) * CH) / p.every - 1;
                float *dst = ckpt_dst(p, m, h, DK * DV);
                if (dst)
#pragma unroll
                    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + 4 * lq + e) * DV + j0 + lr] = Sr[ct][e];
            }
        }
        __syncthreads();
    }

    if (p.sf) {
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.sf[st_off + (size_t)(16 * ct + 4 * lq + e) * DV + j0 + lr] = Sr[ct][e];
    }
}

// Launch plan, part 1: sequences ordered longest first (ties: lower index first), so the
// longest (sequence, head) chains are dispatched first.  One thread per sequence counts the
// sequences that go before it; the lengths are staged through LDS 1024 at a time.
constexpr int PLAN_RANK_THREADS = 256;
__global__ void __launch_bounds__(PLAN_RANK_THREADS)
plan_rank_kernel(const int32_t *__restrict__ cu, int N, int32_t *__restrict__ order) {
    __shared__ int32_t sl[1024];
    const int nn = (int)blockIdx.x * PLAN_RANK_THREADS + (int)threadIdx.x;
    const int Ln = nn < N ? cu[nn + 1] - cu[nn] : 0;
    int rank = 0;
    for (int base = 0; base < N; base += 1024) {
        __syncthreads();
        for (int i = threadIdx.x; i < 1024; i += PLAN_RANK_THREADS)
            sl[i] = base + i < N ? cu[base + i + 1] - cu[base + i] : 0;
        __syncthreads();
        const int lim = min(1024, N - base);
        for (int m = 0; m < lim; ++m) {
            const int Lm = sl[m];
            rank += (Lm > Ln) || (Lm == Ln && base + m < nn);
        }
    }
    if (nn < N) order[rank] = nn;
}

// Launch plan, part 2: per sequence, the index of its first checkpoint (an exclusive scan of
// floor(L / every)).  One workgroup.
__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t *__restrict__ cu, int N, int every, int64_t *__restrict__ ckpt_base) {
    if (every > 0) {
        __shared__ int64_t carry;
        if (threadIdx.x == 0) carry = 0;
        __syncthreads();
        __shared__ int64_t part[1024];
        for (int base = 0; base < N; base += blockDim.x) {
            const int nn = base + threadIdx.x;
            const int64_t c = nn < N ? (int64_t)((cu[nn + 1] - cu[nn]) / every) : 0;
            part[threadIdx.x] = c;
            __syncthreads();
            for (int off = 1; off < (int)blockDim.x; off <<= 1) {   // inclusive scan
                const int64_t v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
                __syncthreads();
                part[threadIdx.x] += v;
                __syncthreads();
            }
            if (nn < N) ckpt_base[nn] = carry + part[threadIdx.x] - c;
            __syncthreads();
            if (threadIdx.x == blockDim.x - 1) carry += part[threadIdx.x];
            __syncthreads();
        }
    }
}

}  // namespace kda

// Workspace: [order: N int32, padded to 256 B][ckpt_base: N int64].
extern "C" __attribute__((visibility("hidden"))) size_t kda_chunk_workspace_layout(int N, size_t *order_off, size_t *base_off) {
    const size_t o = 0, b = ((size_t)N * 4 + 255) / 256 * 256;
    if (order_off) *order_off = o;
    if (base_off) *base_off = b;
    return b + ((size_t)N * 8 + 255) / 256 * 256 + 256;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t
kda_launch_chunk32(int dk, int in_bf16, unsigned grid, const kda::ChunkParams &p, hipStream_t stream);

// The launch plan alone (sequence order, per-sequence checkpoint bases for `every`) into the
// start of `workspace`, as kda_launch_chunk lays it out.
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_plan(int N, const int32_t *cu, int every,
                                                                           void *workspace, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    size_t oo, bo;
    kda_chunk_workspace_layout(N, &oo, &bo);
    int32_t *order = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + oo);
    int64_t *base = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + bo);
    hipLaunchKernelGGL(kda::plan_rank_kernel, dim3((N + kda::PLAN_RANK_THREADS - 1) / kda::PLAN_RANK_THREADS),
                       dim3(kda::PLAN_RANK_THREADS), 0, stream, cu, N, order);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || every <= 0) return err;
    hipLaunchKernelGGL(kda::plan_kernel, dim3(1), dim3(1024), 0, stream, cu, N, every, base);
    return hipGetLastError();
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_launch_chunk(int chunk, int dk, int in_bf16, int N, int H,
                                       const void *q, const void *k,
                                       const void *v, const float *g, const float *beta, const int32_t *cu,
                                       const float *s0, float *sf, int every, float *ckpt, float *o,
                                       float scale, const int32_t *s0_idx, const int32_t *ck_idx,
                                       int nslots, int flags, void *workspace, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    if (flags != 0 && chunk != 32) return hipErrorInvalidValue;   // fused prologue: chunk 32 only
    size_t oo, bo;
    kda_chunk_workspace_layout(N, &oo, &bo);
    const int32_t *order = reinterpret_cast<const int32_t *>(static_cast<char *>(workspace) + oo);
    const int64_t *base = reinterpret_cast<const int64_t *>(static_cast<char *>(workspace) + bo);
    hipError_t err = kda_launch_plan(N, cu, every, workspace, stream);
    if (err != hipSuccess) return err;

    kda::ChunkParams p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.cu_seqlens = cu; p.order = order;
    p.ckpt_base = base; p.s0 = s0; p.sf = sf; p.ckpt = ckpt; p.o = o; p.H = H; p.every = every;
    p.scale = scale; p.s0_idx = s0_idx; p.ck_idx = ck_idx; p.nslots = nslots; p.s0_slots = nslots; p.flags = flags; p.nseq = N;
    p.o_tr = nullptr; p.ckpt_tr = nullptr;
    const dim3 grid((unsigned)N * (unsigned)H);
    if (chunk == 32) return kda_launch_chunk32(dk, in_bf16, grid.x, p, stream);
#define KDA_CHUNK(DKV, F32P, T) \
    hipLaunchKernelGGL((kda::chunk_fwd_kernel<DKV, F32P, T>), grid, dim3(DKV * 4), 0, stream, p)
    if (dk == 128 && in_bf16) KDA_CHUNK(128, false, uint16_t);
    else if (dk == 128) KDA_CHUNK(128, true, float);
    else if (dk == 64 && in_bf16) KDA_CHUNK(64, false, uint16_t);
    else if (dk == 64) KDA_CHUNK(64, true, float);
    else return hipErrorInvalidValue;
#undef KDA_CHUNK
    return hipGetLastError();
}
