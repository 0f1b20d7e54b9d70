// kda_chunk32.hip -- software-pipelined chunked KDA prefill, 32-token chunks (gfx950).
//
// Same operator and chunk algebra as kda_chunk.hip (the chunk-recurrent form of
// the gated delta rule; "Attention->K3 course, Day 21", quiz Q9 / answer D19;
// skillsmp K3 skill card, quick facts: per-channel gate, g >= -5), with a chunk
// of two 16-row sub-chunks a = 0, 1.  With G the in-chunk cumulative log-decay,
// G_ref(a) its value before the first row of sub-chunk a, P0 = e^{G_ref(1)}:
//     KS = K * e^{G - G_ref},  QS = Q * e^{G - G_ref}          (entries <= |x|)
//     Gamma*K and Gamma*Q equal KS and QS on rows 0..15 (G_ref(0) = 0); rows
//     16..31 are KS and QS times P0, stored separately (KG, QT)
//     A_kk, A_qk   lower 16x16 Gram tiles (0,0), (1,0), (1,1) of KS/QS against
//                  K * e^{G_ref(a) - G} (in fp32 range: 16 * 5 = 80 < 88)
//     (I + A_kk) U = Diag(beta) Y block by block, A_kk strictly lower, beta-scaled rows:
//         U0 = T00 Y0,   W = A10 U0,   U1 = T11 Y1 - M11 W
//         with M_aa = (I + A_aa)^{-1}, T_aa = M_aa Diag(beta_a)
//     Y  = V - (Gamma*K) S ;  O = scale [ (Gamma*Q) S + A_qk U ]
//     (the scan accumulates -Y = (Gamma*K) S - V on top of -V, and the diagonal
//     blocks are stored as -T_aa, so U comes out with the right sign)
//     S <- Diag(Gamma_last) S + (e^{G_last-G} * K)^T U
//
// Workgroup = one (sequence, head): DV/32 "scan waves" and 4*DK/64 "prep waves".
// Scan wave w owns value columns 32w .. 32w+31 and keeps that d_k x 32 slice of S
// in registers (fp32) for the whole sequence.  Prep waves build the
// S-independent operands of the NEXT chunk while the scan waves consume the
// current one.  The two roles run separate loops with the same three
// LDS-only barriers per iteration (global loads stay in flight across them):
//
//            scan waves (chunk i)                      prep waves (chunk i+1)
//   seg 1    a(i): -Y = (Gamma*K) S - V, (Gamma*Q) S   P1: exp(g), 4-row running products, group totals;
//                                                      inverses of chunk i's diagonal blocks -> -T00, [-M11 -T11]
//   seg 2    b(i): U; o(i): O                          P2: decayed operands KS, QS, KG, Kn -> LDS
//   seg 3    c(i): S <- Gamma_last S + Khat^T U        P3: Khat^T, Gamma_last, Gamma*Q, -V -> LDS;
//                                                      Gram tiles
//
// so the scan's dependent chain a -> b -> c occupies every segment.  Every LDS
// operand is written in a segment after its last read by the previous chunk;
// (e^{G_last-G} K)^T and Gamma_last, written in segment 3 while stage c reads
// the previous chunk's, are double-buffered.  Prep waves load the raw rows of
// chunk i+2 straight into registers while preparing chunk i+1; every load is
// unconditional (rows past the end of the sequence re-read its last row and
// are masked where used).
//
// Precision: hi+lo bf16 operand pairs on every product feeding the outputs
// except (Gamma*K) S and the KS side of A_kk (single bf16 there; hi+lo in the
// states-only runs that hand R = V - (Gamma*K) S to the backward), fp32
// accumulation, fp32 o and S.  The fp32-input instantiation uses fp32 MFMA
// throughout.
#include <type_traits>

#include "kda_frag.h"

namespace kda {

constexpr int C32 = 32;

template <int DK, int NSW, int JT, bool F32P, typename IN_T>
struct Lds32 {
    static constexpr int ES = Mat<F32P>::ES;
    // operands of a chunk, written by the prep waves, read by the scan waves
    static constexpr int KS = 0;                          // [32][DK] single: K * e^{G - G_ref}
    static constexpr int QS = KS + 32 * DK * ES;          // [32][DK] hl: Q * e^{G - G_ref}
    static constexpr int SQ_PLANE = 32 * DK * ES;
    // rows 16..31 only of the next two (rows 0..15 of Gamma*K and Gamma*Q are those of KS and QS);
    // addressed with the 32-row offsets from a base moved back by 16 rows (QT_AT, KG_AT)
    static constexpr int QT = QS + 32 * DK * 4;           // [16][DK] hl: Gamma * Q, rows 16..31
    static constexpr int QT_PLANE = 16 * DK * ES;
    static constexpr int QT_AT = QT - 16 * DK * ES;
    static constexpr int KG = QT + 16 * DK * 4;           // [16][DK] single: Gamma * K, rows 16..31
    static constexpr int KG_AT = KG - 16 * DK * ES;
    // states-only runs that hand R on keep KS and KG as hl, their lo planes in the unused QS and QT
    static constexpr int KG_LO = QT - KG;                 // (a negative plane distance)
    static constexpr int KHT = KG + 16 * DK * ES;         // 2 x [DK][32] hl: (e^{G_last-G} K)^T
    static constexpr int KHT_PLANE = DK * 32 * ES;
    static constexpr int KHT_BUF = DK * 32 * 4;
    static constexpr int TM = KHT + 2 * KHT_BUF;          // [32][32] hl: [T00 0 ; -M11 T11]
    static constexpr int TRI_PLANE = 32 * 32 * ES;
    static constexpr int AQK = TM + 32 * 32 * 4;          // [32][32] hl: A_qk, lower incl. diagonal
    static constexpr int AW = AQK + 32 * 32 * 4;          // [16][32] hl: [A10 0]
    static constexpr int AW_PLANE = 16 * 32 * ES;
    static constexpr int GC = AW + 16 * 32 * 4;           // 2 x [DK] fp32: Gamma_last
    // padded row pitch (bytes) of the value rows: the rows 4 apart that one read spans start
    // 8 (JT = 2) or 4 (JT = 1) banks apart modulo the row of 64 banks it reads
    static constexpr int VPITCH = DK * 4 + 16 * JT;
    static constexpr int VB = GC + 2 * DK * 4;            // [32][VPITCH] fp32: -V of a chunk
    // prep-wave scratch
    static constexpr int KN = VB + 32 * VPITCH;           // [32][DK] hl: K e^{G_ref(a) - G}, sub-chunk a's rows
    static constexpr int KN_PLANE = 32 * DK * ES;
    // the strictly lower, beta-scaled diagonal A_kk blocks, from the Gram tiles to the inverses:
    // block a as Z (ZR + a TSZ) and as Z^T (ZT + a TSZ), fp32 [16][TP]
    static constexpr int ZR = KN + 32 * DK * 4;
    static constexpr int ZT = ZR + 2 * TSZ * 4;
    static constexpr int XCHG = ZT + 2 * TSZ * 4;         // [8][DK] fp32: decay over each 4-row group
    static constexpr int BETA = XCHG + 8 * DK * 4;        // 2 x [32] fp32
    // scan-wave stash: each scan lane parks its 8 JT (Gamma*Q) S partial outputs here between
    // segments 1 and 2 (register pressure), tile j of lane l at OST + (j * 64 NSW + l) * 16 bytes
    static constexpr int NRM = BETA + 2 * 32 * 4;         // 2 x [32][2] fp32: 1/|k|, 1/|q| per row (fused prologue)
    static constexpr int NRM_BUF = 32 * 2 * 4;
    static constexpr int OST = NRM + 2 * NRM_BUF;
    static constexpr int TOTAL = OST + 2 * JT * 64 * NSW * 16;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Two adjacent input elements, kept in their storage format until used.
template <typename T> struct Pair;
template <> struct Pair<uint16_t> {
    using raw = uint32_t;
    __device__ static raw load(const uint16_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ static raw zero() { return 0u; }
    __device__ static float lo(raw w) { return lo_bf16_of(w); }
    __device__ static float hi(raw w) { return hi_bf16_of(w); }
};
template <> struct Pair<float> {
    using raw = float2;
    __device__ static raw load(const float *p) { return *reinterpret_cast<const float2 *>(p); }
    __device__ static raw zero() { return make_float2(0.f, 0.f); }
    __device__ static float lo(raw w) { return w.x; }
    __device__ static float hi(raw w) { return w.y; }
};

// SPLIT workgroups share one (sequence, head), each owning DV / SPLIT value columns (the
// state's columns evolve independently) and each preparing the chunk operands itself.  A scan
// wave owns 16 value columns when a workgroup has at most 64, else 32.  With four 16-column scan
// waves (d_k = 128, two workgroups per chain) the workgroup also gets 4 "role" waves for the
// diagonal inverses and Gram tiles: 16 waves, 4 per SIMD, one scan, two prep and one role wave
// on each.  Otherwise prep waves 0..2 take those roles on top of their own work.
template <int DK, int SPLIT> constexpr int chunk32_scan_cols() { return DK / SPLIT <= 64 ? 16 : 32; }
template <int DK, int SPLIT> constexpr int chunk32_scan_waves() { return DK / SPLIT / chunk32_scan_cols<DK, SPLIT>(); }
template <int DK, int SPLIT> constexpr int chunk32_role_waves() {
    return chunk32_scan_waves<DK, SPLIT>() == 4 && chunk32_scan_cols<DK, SPLIT>() == 16 ? 4 : 0;
}
template <int DK, int SPLIT> constexpr int chunk32_threads() {
    return 64 * (chunk32_scan_waves<DK, SPLIT>() + DK / 16 + chunk32_role_waves<DK, SPLIT>());
}

// Decay table of the fused gate, alpha = exp(-5 sigmoid(a)) for every bf16 pre-activation a that
// changes it in fp32: per sign, entry 0 stands for |a| < 2^-24 (where 1 + e^-a rounds as at a = 0),
// entries 1 .. 29 * 128 for the binades 2^-24 <= |a| < 32 (bf16 exponents 103 .. 131, 128 mantissas
// each), and the last entry for |a| >= 32 (alpha is then exactly e^-5 for a > 0, 1 for a < 0; the
// same rounding already holds from |a| > 17).  The entries are formed with the instructions of the
// arithmetic path, so a lookup returns that path's value.  Only the two-workgroup kernels take it:
// their LDS has room for its 29,712 bytes.
constexpr int GT_U0 = 103 * 128 - 1;          // magnitude bits (exponent, mantissa) of entry 0
constexpr int GT_ROW = 1 + 29 * 128 + 1;      // entries per sign
__device__ __forceinline__ float gate_decay(float a) {
    return __expf(-5.f * __builtin_amdgcn_rcpf(1.f + __expf(-a)));
}
__device__ __forceinline__ int gate_index(uint32_t b) {   // b: the 16 bits of a in its low half
    const int j = min(max((int)(b & 0x7FFFu) - GT_U0, 0), GT_ROW - 1);
    return (int)((b >> 15) & 1u) * GT_ROW + j;
}
__device__ __forceinline__ float gate_entry(int i) {
    const int sgn = i >= GT_ROW, j = i - sgn * GT_ROW;
    const uint32_t mag = j == 0 ? 0u : j == GT_ROW - 1 ? (132u << 7) : (uint32_t)(j + GT_U0);
    return gate_decay(__uint_as_float(((uint32_t)sgn << 31) | (mag << 16)));
}

// JT adjacent fp32 values (the columns one scan lane owns in a row) from / to memory
template <int JT> __device__ __forceinline__ void load_cols(const float *ptr, float (&x)[JT]) {
    if constexpr (JT == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(ptr);
        x[0] = v.x;
        x[1] = v.y;
    } else {
        x[0] = *ptr;
    }
}
template <int JT> __device__ __forceinline__ void store_cols(float *ptr, const float (&x)[JT]) {
    if constexpr (JT == 2) *reinterpret_cast<float2 *>(ptr) = make_float2(x[0], x[1]);
    else *ptr = x[0];
}

// PRO: the fused prologue (KDA_PRO_* bits), a compile-time choice so that the plain path keeps
// none of its code; with KDA_STATES_ONLY the kernel produces the states alone (no q, no o).
template <int DK, int SPLIT, bool F32P, typename IN_T, int PRO = 0>
__global__ void __launch_bounds__((chunk32_threads<DK, SPLIT>()))
chunk32_kernel(const ChunkParams p) {
    constexpr int DV = DK;
    constexpr int SWC = chunk32_scan_cols<DK, SPLIT>();   // value columns of a scan wave
    constexpr int JT = SWC / 16;                          // 16-column MFMA tiles of a scan wave
    constexpr int NSW = DV / SPLIT / SWC;                 // scan waves
    constexpr int NRW = chunk32_role_waves<DK, SPLIT>();  // role waves (inverses, Gram tiles)
    static_assert(SPLIT == 1 || SPLIT == 2, "a chain's value columns go to one or two workgroups");
    constexpr int NPW = DK / 16;        // prep waves: 8 four-row groups x DK/2 channel pairs
    constexpr int KB = DK / 32;         // 32-wide K-steps over d_k
    constexpr int KT = DK / 16;         // 16-row tiles over d_k
    constexpr int NCP = DK / 2;         // channel pairs
    using L = Lds32<DK, NSW, JT, F32P, IN_T>;
    using M = Mat<F32P>;
    using F = Frag<F32P>;
    using PR = Pair<IN_T>;
    constexpr bool SO = (PRO & KDA_STATES_ONLY) != 0;   // states only: q, Gamma*Q, A_qk and o skipped
    constexpr bool TR = (PRO & KDA_TRANSITION) != 0;    // the paired segment pass (see KDA_TRANSITION)
    static_assert(!TR || (!SO && SPLIT == 1), "the paired pass: outputs and states, one workgroup per run");

    // the fused gate's decay table after the operands (two workgroups per chain, d_k = 128)
    constexpr bool GTAB = (PRO & KDA_PRO_GATE) != 0 && NRW > 0;
    constexpr int GT_BYTES = GTAB ? 2 * GT_ROW * 4 : 0;
    static_assert(L::TOTAL % 16 == 0 && L::TOTAL + GT_BYTES <= 160 * 1024, "LDS budget with the gate table");
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL + GT_BYTES];

    const int H = p.H;
    // Workgroups are handed to the 8 XCDs round-robin by index, and each XCD has its own L2.  The
    // workgroups that split one chain read the same k, q, g and beta, so they take indices 8 apart
    // (same XCD, one L2 fetch serves both): within each group of 16, index 8 r + x (r = 0, 1) is
    // part r of chain 8 j + x.  A tail of fewer than 16 falls back to adjacent indices.
    // The paired segment pass places the two runs of a chain (kind 0 and 1) the same way.
    int part, hn;
    {
        const int b = (int)blockIdx.x;
        constexpr bool PAIRED = SPLIT == 2 || TR;
        const int full = PAIRED ? ((int)gridDim.x & ~15) : 0;
        if (!PAIRED) {
            part = 0; hn = b;
        } else if (b < full) {
            part = (b >> 3) & 1; hn = ((b >> 4) << 3) + (b & 7);
        } else {
            part = (b - full) & 1; hn = (full >> 1) + ((b - full) >> 1);
        }
    }
    const int kind = TR ? part : 0;           // paired segment pass: 1 = the transition run
    if (TR) part = 0;
    const int h = hn % H;
    const int n = p.order[hn / H];
    if (TR && kind && p.s0_idx[n] != -2) return;   // a sequence's first segment needs no transition run
    const int col0 = (DV / SPLIT) * part;     // first value column of this workgroup
    const int seq_start = p.cu_seqlens[n];
    const int seq_len = p.cu_seqlens[n + 1] - seq_start;
    const int nchunks = (seq_len + C32 - 1) / C32;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // wave-uniform: scalar register
    // Waves are placed on the 4 SIMDs round-robin.  The scan waves take the indices that put them on
    // the SIMDs holding the fewest waves (with 12 waves: one on each SIMD; with 10: SIMDs 2 and 3);
    // the prep waves take the rest, in order.
    constexpr int NWAVES = NSW + DK / 16 + NRW;
    constexpr int SCAN0 = (NSW + DK / 16) % 4;
    const bool is_scan = wave >= SCAN0 && wave < SCAN0 + NSW;
    const bool is_role = wave >= NSW + DK / 16;      // role waves come last
    const int sw = wave - SCAN0;                     // scan wave index (scan waves only)

    if constexpr (GTAB) {
        float *tab = reinterpret_cast<float *>(smem + L::TOTAL);
        for (int i = (int)threadIdx.x; i < 2 * GT_ROW; i += 64 * NWAVES) tab[i] = gate_entry(i);
        __syncthreads();
    }

    const IN_T *qg = reinterpret_cast<const IN_T *>(p.q);
    const IN_T *kg = reinterpret_cast<const IN_T *>(p.k);
    const IN_T *vg = reinterpret_cast<const IN_T *>(p.v);

    // Diagonal block a of chunk ch: M = (I + N)^{-1} for the strictly lower, beta-scaled N, given
    // as NA = N[lr][4 lq + e] ("A" form) and NB = N[4 lq + e][lr] ("B" form), as
    //     M = (I + X)(I + X^2)(I + X^4)(I + X^8),  X = -N,  N^16 = 0,
    // with 16x16 MFMA products held in registers (four dependent levels instead of a 16-step
    // substitution; hi/lo bf16 operands, or fp32 MFMA for fp32 inputs).  -T_aa = -M Diag(beta_a)
    // (and -M11) -> TM, read by stage b in segment 2.  In two parts: the first three levels
    // (inv_front: X8 and A3 = (I + X)(I + X^2)(I + X^4)), then M = A3 + A3 X^8 and the stores
    // (inv_back), which the role waves run in the next iteration's segment 1.
    // (Z W) in B form = inv_mm(Z_A, W_B); in A form = inv_mm(W_B, Z_A)
    auto inv_mm = [](const f32x4_t &za, const f32x4_t &wb) {
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
        if constexpr (F32P) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) d = mfma_f32(za[kk], wb[kk], d);
        } else {
            // hi/lo bf16 split in two 16x16x32 MFMAs: K-slots 0..15 carry the hi parts and
            // 16..31 the lo parts of Z, so [Zh Zl][Wh; Wh] + [Zh Zh][Wl; 0] = Zh Wh + Zl Wh + Zh Wl
            uint32_t zh[2], zl[2], wh[2], wl[2];
            split_hl2(za[0], za[1], zh[0], zl[0]);
            split_hl2(za[2], za[3], zh[1], zl[1]);
            split_hl2(wb[0], wb[1], wh[0], wl[0]);
            split_hl2(wb[2], wb[3], wh[1], wl[1]);
            const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, (uint4){zh[0], zh[1], zl[0], zl[1]});
            const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, (uint4){wh[0], wh[1], wh[0], wh[1]});
            const bf16x8_t a2 = __builtin_bit_cast(bf16x8_t, (uint4){zh[0], zh[1], zh[0], zh[1]});
            const bf16x8_t b2 = __builtin_bit_cast(bf16x8_t, (uint4){wl[0], wl[1], 0u, 0u});
            d = mfma_bf16(a1, b1, d);
            d = mfma_bf16(a2, b2, d);
        }
        return d;
    };
    // M = A1 (I + X^2)(I + X^4)(I + X^8) with A1 = I + X, each factor applied as A += A X^(2^k)
    auto inv_front = [&](int lane, const f32x4_t &NA, const f32x4_t &NB, f32x4_t &X8B, f32x4_t &A3A) {
        const int lr = lane & 15, lq = lane >> 4;
        const f32x4_t XA = {-NA[0], -NA[1], -NA[2], -NA[3]}, XB = {-NB[0], -NB[1], -NB[2], -NB[3]};
        f32x4_t A1A;
#pragma unroll
        for (int e = 0; e < 4; ++e) A1A[e] = ((4 * lq + e == lr) ? 1.f : 0.f) + XA[e];
        const f32x4_t X2B = inv_mm(XA, XB), X2A = inv_mm(XB, XA);
        const f32x4_t X4B = inv_mm(X2A, X2B), X4A = inv_mm(X2B, X2A), Y2A = inv_mm(X2B, A1A);
        f32x4_t A2A;
#pragma unroll
        for (int e = 0; e < 4; ++e) A2A[e] = A1A[e] + Y2A[e];
        X8B = inv_mm(X4A, X4B);
        const f32x4_t Y3A = inv_mm(X4B, A2A);
#pragma unroll
        for (int e = 0; e < 4; ++e) A3A[e] = A2A[e] + Y3A[e];
    };
    auto inv_back = [&](char *sm, int a, int ch, int lane, const f32x4_t &X8B, const f32x4_t &A3A) {
        const int lr = lane & 15, lq = lane >> 4;
        const float *beta_ch = reinterpret_cast<const float *>(sm + L::BETA) + (ch & 1) * 32;
        const f32x4_t Y4A = inv_mm(X8B, A3A);
        f32x4_t MA;                                      // A form: M[lr][4 lq + e]
#pragma unroll
        for (int e = 0; e < 4; ++e) MA[e] = A3A[e] + Y4A[e];
        const float4 b4 = *reinterpret_cast<const float4 *>(beta_ch + 16 * a + 4 * lq);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
        float tv[4], nm[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) { tv[e] = -(MA[e] * bv[e]); nm[e] = -MA[e]; }
        M::template put_hl<4>(sm + L::TM, L::TRI_PLANE, fofs<1>(16 * a + lr, 16 * a + 4 * lq), tv);
        if (a == 1) M::template put_hl<4>(sm + L::TM, L::TRI_PLANE, fofs<1>(16 + lr, 4 * lq), nm);
    };
    auto diag_inverse = [&](char *sm, int a, int ch, int lane, const f32x4_t &NA, const f32x4_t &NB) {
        f32x4_t X8B, A3A;
        inv_front(lane, NA, NB, X8B, A3A);
        inv_back(sm, a, ch, lane, X8B, A3A);
    };

    // Gram product of Kn block knb (16 rows) with rows 16 a .. 16 a + 15 of KS (or QS), or with
    // GAMMA of Gamma*K (or Gamma*Q; a = 1 only): lane holds element (row 16 a + lr, Kn row 4 lq + e)
    // of the tile.  Two accumulator chains (even and odd K-steps) keep two products in flight for
    // one final 4-element add.
    auto gram_prod = [&](char *sm, int knb, int a, bool use_q, int lane, bool gamma = false) {
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KB; ++s) {
            const F fn = M::template get<true>(sm + L::KN, L::KN_PLANE, fbase<KB>(knb, s, lane));
            if (use_q)
                mma<true, true>(acc[s & 1], fn, gamma ? M::template get<true>(sm + L::QT_AT, L::QT_PLANE, fbase<KB>(a, s, lane))
                                                      : M::template get<true>(sm + L::QS, L::SQ_PLANE, fbase<KB>(a, s, lane)));
            else
                mma<true, false>(acc[s & 1], fn, M::template get<false>(sm + (gamma ? L::KG_AT : L::KS), 0, fbase<KB>(a, s, lane)));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[0][e] += acc[1][e];
        return acc[0];
    };
    // The same product of Kn block knb with KS rows 16 a .. 16 a + 15 in both orientations: gA as
    // gram_prod, gB[e] = element (row 16 a + 4 lq + e, Kn row lr) (operands swapped); one
    // accumulator chain per orientation, the two chains interleaved
    auto gram_prod_ab = [&](char *sm, int knb, int a, int lane, f32x4_t &gA, f32x4_t &gB) {
        gA = f32x4_t{0.f, 0.f, 0.f, 0.f};
        gB = gA;
#pragma unroll
        for (int s = 0; s < KB; ++s) {
            const F fn = M::template get<true>(sm + L::KN, L::KN_PLANE, fbase<KB>(knb, s, lane));
            const F fx = M::template get<false>(sm + L::KS, 0, fbase<KB>(a, s, lane));
            mma<true, false>(gA, fn, fx);
            mma<false, true>(gB, fx, fn);
        }
    };
    // A_qk tile (a, b) (lower incl. diagonal on the diagonal tiles) -> AQK
    auto store_aqk = [&](char *sm, int a, int b, const f32x4_t &gq, int lane) {
        const int lr = lane & 15, lq = lane >> 4;
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (b < a || 4 * lq + e <= lr) ? gq[e] : 0.f;
        M::template put_hl<4>(sm + L::AQK, L::TRI_PLANE, fofs<1>(16 * a + lr, 16 * b + 4 * lq), w);
    };
    // beta-scaled rows of a Gram tile of sub-chunk a of chunk ch (row lr of the lane)
    auto beta_row = [&](char *sm, int a, int ch, int lane) {
        return reinterpret_cast<const float *>(sm + L::BETA)[(ch & 1) * 32 + 16 * a + (lane & 15)];
    };
    // strictly lower part of a diagonal A_kk tile with beta-scaled rows (A form)
    auto strict_lower = [&](const f32x4_t &gk, float br, int lane) {
        const int lr = lane & 15, lq = lane >> 4;
        f32x4_t z;
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = 4 * lq + e < lr ? br * gk[e] : 0.f;
        return z;
    };
    // Gram tile t of chunk ch, from the Kn block it shares with the A_qk tile of the same place
    // (the waves that invert the diagonal blocks run in a later segment and read ZR / ZT):
    //   t 0: tile (0,0)  A_kk -> ZR/ZT block 0   and A_qk(0,0)
    //   t 1: tile (1,1)  A_kk -> ZR/ZT block 1   and A_qk(1,1)
    //   t 2: tile (1,0)  A10 -> AW               and A_qk(1,0): Gamma*K (Gamma*Q) rows 16..31 against
    //        K e^{-G} rows 0..15 (Kn block 0), since k_r e^{G_r} k_i e^{-G_i} = k_r k_i e^{G_r - G_i}
    auto gram_tile = [&](char *sm, int t, int ch, int lane) {
        const int lr = lane & 15, lq = lane >> 4;
        const int knb = t == 1 ? 1 : 0;
        const int a = t == 0 ? 0 : 1, b = t == 1 ? 1 : 0;
        const f32x4_t gk = gram_prod(sm, knb, a, false, lane, t == 2);
        if constexpr (!SO) store_aqk(sm, a, b, gram_prod(sm, knb, a, true, lane, t == 2), lane);
        const float br = beta_row(sm, a, ch, lane);
        if (t == 2) {
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = br * gk[e];
            M::template put_hl<4>(sm + L::AW, L::AW_PLANE, fofs<1>(lr, 4 * lq), w);
        } else {
            const f32x4_t z = strict_lower(gk, br, lane);
            float *zr = reinterpret_cast<float *>(sm + L::ZR) + t * TSZ;
            float *zt = reinterpret_cast<float *>(sm + L::ZT) + t * TSZ;
            *reinterpret_cast<float4 *>(zr + lr * TP + 4 * lq) = make_float4(z[0], z[1], z[2], z[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) zt[(4 * lq + e) * TP + lr] = z[e];
        }
    };
    // the inverse of diagonal block a of chunk ch from the tile gram_tile left in ZR / ZT
    auto diag_inverse_lds = [&](char *sm, int a, int ch, int lane) {
        const int lr = lane & 15, lq = lane >> 4;
        const float4 na4 = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(sm + L::ZR) + a * TSZ + lr * TP + 4 * lq);
        const float4 nb4 = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(sm + L::ZT) + a * TSZ + lr * TP + 4 * lq);
        diag_inverse(sm, a, ch, lane, f32x4_t{na4.x, na4.y, na4.z, na4.w}, f32x4_t{nb4.x, nb4.y, nb4.z, nb4.w});
    };

    if (NRW > 0 && is_role) {
        // ============================== role waves ==============================
        // In segment 3 of iteration it, the operands of chunk it + 1 being in LDS, wave rw forms
        //   rw 0, 1: A_kk(rw, rw), then inverts diagonal block rw -> TM
        //   rw 2:    A_qk(0,0), A_qk(1,1)
        //   rw 3:    A10 -> AW, A_qk(1,0)
        const int rw = wave - (NSW + DK / 16);
        // their work is a chain of dependent MFMA products: issue it ahead of the other waves
        __builtin_amdgcn_s_setprio(3);
        // With the fused normalisation they also form 1/|k| and 1/|q| of every row of chunk it + 2 in
        // segment 2 (where they are otherwise idle and the scan waves' products are few; chunk 0's
        // before the loop), at the lowest priority, into the buffer of that chunk's parity, which
        // the prep waves read in segment 1 of the next iteration, off their segment-2 path.  A row's
        // sum of squares is the diagonal entry of the Gram product of the raw rows with themselves,
        // formed on the matrix cores (bf16 products are exact in fp32, fp32 accumulation): wave rw
        // takes the 16 rows 16 (rw & 1) .. of k (rw < 2) or q (rw >= 2), and lane (lr, lq) holds
        // values 32 s + 8 lq .. + 7 of row lr for K-step s, which is both the A and the B fragment
        // of the 16x16x32 product.  The raw rows load one iteration ahead.
        constexpr bool RNORM = (PRO & KDA_PRO_NORM) != 0;
        const bool nwave = !SO || rw < 2;   // states only: q and its norms are not used
        uint4 xr_[KB];
        auto nload = [&](int ch) {
            const int t0 = seq_start + ch * C32, nv = min(C32, seq_len - ch * C32), lane = lane_id();
            const int r = min(16 * (rw & 1) + (lane & 15), nv - 1);
            const uint16_t *src = reinterpret_cast<const uint16_t *>(rw < 2 ? p.k : p.q) +
                                  ((size_t)(t0 + r) * H + h) * DK + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < KB; ++s) xr_[s] = *reinterpret_cast<const uint4 *>(src + 32 * s);
        };
        auto nstore = [&](char *sm, int ch) {   // 1/|x| of the wave's 16 rows of chunk ch (0 for a zero row)
            const int lane = lane_id(), lr = lane & 15, lq = lane >> 4;
            f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const bf16x8_t x = __builtin_bit_cast(bf16x8_t, xr_[s]);
                acc[s & 1] = mfma_bf16(x, x, acc[s & 1]);
            }
            // lane (lr, lq) holds entries (4 lq + e, lr): the diagonal entry of row lr where lr / 4 == lq
            if ((lr >> 2) == lq) {
                const int e = lr & 3;
                const float ss = (e == 0 ? acc[0][0] + acc[1][0] : e == 1 ? acc[0][1] + acc[1][1]
                                  : e == 2 ? acc[0][2] + acc[1][2] : acc[0][3] + acc[1][3]);
                reinterpret_cast<float *>(sm + L::NRM + (ch & 1) * L::NRM_BUF + (16 * (rw & 1) + lr) * 8)[rw >> 1] =
                    ss > 0.f ? rsqrtf(ss) : 0.f;
            }
        };
        if constexpr (RNORM) {
            static_assert(DK == 128 && sizeof(IN_T) == 2, "the normalisation reads bf16 rows, four K-steps of 32");
            if (nwave && nchunks > 0) {
                nload(0);
                nstore(smem + opaque_s(0), 0);
                nload(min(1, nchunks - 1));
            }
            lds_barrier();   // chunk 0's norms before the prep waves' first segment 1 (all roles pass one)
        }
        // role waves 0, 1: the last level of the pending chunk's inverse, in segment 1 where the
        // chunk's T is not yet read (stage b reads it in segment 2); the other levels in segment 3
        f32x4_t x8b = {0.f, 0.f, 0.f, 0.f}, a3a = x8b;
        for (int it = -1; it < nchunks; ++it) {
            char *const sm = smem + opaque_s(0);
            const int lane = lane_id(), lr = lane & 15, lq = lane >> 4;
            if (rw < 2 && it >= 0) inv_back(sm, rw, it, lane, x8b, a3a);
            lds_barrier();
            if constexpr (RNORM) {
                if (nwave && it + 2 < nchunks) {
                    __builtin_amdgcn_s_setprio(0);   // behind the prep waves' segment 2
                    nstore(sm, it + 2);
                    nload(min(it + 3, nchunks - 1));
                    __builtin_amdgcn_s_setprio(3);
                }
            }
            lds_barrier();
            const int ch = it + 1;
            if (ch < nchunks) {
                if (rw < 2) {
                    // A_kk(rw, rw) with beta-scaled rows, strictly lower, in both forms
                    f32x4_t gA, gB, z, zb;
                    gram_prod_ab(sm, rw, rw, lane, gA, gB);
                    const float *bt = reinterpret_cast<const float *>(sm + L::BETA) + (ch & 1) * 32 + 16 * rw;
                    const float br = bt[lr];
                    const float4 bc = *reinterpret_cast<const float4 *>(bt + 4 * lq);
                    const float bcv[4] = {bc.x, bc.y, bc.z, bc.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        z[e] = 4 * lq + e < lr ? br * gA[e] : 0.f;          // (lr, 4 lq + e)
                        zb[e] = lr < 4 * lq + e ? bcv[e] * gB[e] : 0.f;     // (4 lq + e, lr)
                    }
                    inv_front(lane, z, zb, x8b, a3a);
                } else if (rw == 2) {
                    if constexpr (!SO) {
                        store_aqk(sm, 0, 0, gram_prod(sm, 0, 0, true, lane), lane);
                        store_aqk(sm, 1, 1, gram_prod(sm, 1, 1, true, lane), lane);
                    }
                } else {
                    const f32x4_t gk = gram_prod(sm, 0, 1, false, lane, true);
                    const float br = beta_row(sm, 1, ch, lane);
                    float w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = br * gk[e];
                    M::template put_hl<4>(sm + L::AW, L::AW_PLANE, fofs<1>(lr, 4 * lq), w);
                    if constexpr (!SO) store_aqk(sm, 1, 0, gram_prod(sm, 0, 1, true, lane, true), lane);
                }
            }
            lds_barrier();
        }
    } else if (is_scan) {
        // ============================== scan waves ==============================
        // Lane (lq, lr) of scan wave w owns value columns c(jt) = SWC w + JT lr + jt (jt < JT),
        // adjacent in memory, so V, o and S move as JT-element groups.
        // Sr[jt][ct][e] = S[16 ct + 4 lq + e][col0 + c(jt)]
        const size_t st_off = ((size_t)(kind * p.nseq + n) * H + h) * DK * DV;
        f32x4_t Sr[JT][KT];
        {
            const long long s0o = s0_offset(p, n, h, DK * DV);
            const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x[JT];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt)
                        x[jt] = kind && 16 * ct + 4 * lq + e == col0 + SWC * sw + JT * lr + jt ? 1.f : 0.f;
                    if (!kind && s0o >= 0)
                        load_cols<JT>(p.s0 + s0o + (16 * ct + 4 * lq + e) * DV + col0 + SWC * sw + JT * lr, x);
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) Sr[jt][ct][e] = x[jt];
                }
        }
        const int every_chunks = p.every / C32;   // checkpoint_every is a multiple of the chunk size
        int ck_left = every_chunks, ck_idx = 0;
        if constexpr (NRW > 0 && (PRO & KDA_PRO_NORM) != 0) lds_barrier();   // the role waves' first norms

        for (int it = -1; it < nchunks; ++it) {
            char *const sm = smem + opaque_s(0);
            const int lane = lane_id(), lr = lane & 15, lq = lane >> 4;
            const int t0 = seq_start + it * C32, nv = min(C32, seq_len - it * C32);
            f32x4_t Yacc[2][JT], Oacc[2][JT];
            F UF[JT];

            // ---- seg 1, a(it): Yacc = (Gamma*K) S - V and Oacc = (Gamma*Q) S, S = the state entering
            // chunk it ((Gamma*K) single bf16).  The prep waves invert this chunk's diagonal blocks.
            if (it >= 0) {
                // Yacc starts from -V (rows past the end hold zeros)
                const char *vb = sm + L::VB + (col0 + SWC * sw + JT * lr) * 4;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x[JT];
                        load_cols<JT>(reinterpret_cast<const float *>(vb + (16 * rt + 4 * lq + e) * L::VPITCH), x);
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) Yacc[rt][jt][e] = x[jt];
                    }
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) Oacc[rt][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KB; ++s) {
                    if constexpr (SO) {
                        if (p.rres) {
                            // hi/lo products: R = -Yacc is handed to the backward's gradient kernel
                            const F fk0 = M::template get<true>(sm + L::KS, L::SQ_PLANE, fbase<KB>(0, s, lane));
                            const F fk1 = M::template get<true>(sm + L::KG_AT, L::KG_LO, fbase<KB>(1, s, lane));
#pragma unroll
                            for (int jt = 0; jt < JT; ++jt) {
                                const F sf = M::template from_tiles<true>(Sr[jt][2 * s], Sr[jt][2 * s + 1]);
                                mma<true, true>(Yacc[0][jt], fk0, sf);
                                mma<true, true>(Yacc[1][jt], fk1, sf);
                            }
                        } else {
                            const F fk0 = M::template get<false>(sm + L::KS, 0, fbase<KB>(0, s, lane));
                            const F fk1 = M::template get<false>(sm + L::KG_AT, 0, fbase<KB>(1, s, lane));
#pragma unroll
                            for (int jt = 0; jt < JT; ++jt) {
                                const F sf = M::template from_tiles<false>(Sr[jt][2 * s], Sr[jt][2 * s + 1]);
                                mma<false, false>(Yacc[0][jt], fk0, sf);
                                mma<false, false>(Yacc[1][jt], fk1, sf);
                            }
                        }
                    } else {
                        const F fk0 = M::template get<false>(sm + L::KS, 0, fbase<KB>(0, s, lane));
                        const F fk1 = M::template get<false>(sm + L::KG_AT, 0, fbase<KB>(1, s, lane));
                        const F fq0 = M::template get<true>(sm + L::QS, L::SQ_PLANE, fbase<KB>(0, s, lane));
                        const F fq1 = M::template get<true>(sm + L::QT_AT, L::QT_PLANE, fbase<KB>(1, s, lane));
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            const F sf = M::template from_tiles<true>(Sr[jt][2 * s], Sr[jt][2 * s + 1]);
                            mma<false, false>(Yacc[0][jt], fk0, sf);
                            mma<true, true>(Oacc[0][jt], fq0, sf);
                            mma<true, true>(Oacc[1][jt], fq1, sf);
                            mma<false, false>(Yacc[1][jt], fk1, sf);
                        }
                    }
                }
                // park the output partials in LDS until stage o (this lane's private slots)
                if constexpr (!SO)
#pragma unroll
                    for (int j = 0; j < 2 * JT; ++j)
                        *reinterpret_cast<f32x4_t *>(sm + L::OST + (j * 64 * NSW + 64 * sw + lane) * 16) = Oacc[j / JT][j % JT];
            }
            lds_barrier();

            // ---- seg 2, b(it): U from -Y = Yacc ;  o(it) = scale [ (Gamma*Q) S + A_qk U ]
            if (it >= 0) {
                const f32x4_t (&Y)[2][JT] = Yacc;   // -Y
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    // U0 = (-T00)(-Y0) ; W = A10 U0 ; U1 = (-T11)(-Y1) - M11 W
                    f32x4_t u0 = {0.f, 0.f, 0.f, 0.f}, w = u0, u1 = u0;
                    {
                        const F t0f = M::template get<true>(sm + L::TM, L::TRI_PLANE, fbase<1>(0, 0, lane));
                        mma<true, true>(u0, t0f, M::template from_tiles<true>(Y[0][jt], Y[1][jt]));
                    }
                    {
                        const F awf = M::template get<true>(sm + L::AW, L::AW_PLANE, fbase<1>(0, 0, lane));
                        mma<true, true>(w, awf, M::template from_tiles<true>(u0, Y[1][jt]));
                    }
                    {
                        const F t1f = M::template get<true>(sm + L::TM, L::TRI_PLANE, fbase<1>(1, 0, lane));
                        mma<true, true>(u1, t1f, M::template from_tiles<true>(w, Y[1][jt]));
                    }
                    UF[jt] = M::template from_tiles<true>(u0, u1);
                }
                if constexpr (SO) {
                    // R = V - (Gamma K) S of chunk it (here, where its products have long completed)
                    if (p.rres) {
                        float *const rb = p.rres + ((long long)(p.rbase[n] + it) * H + h) * p.rstride + col0 +
                                          SWC * sw + JT * lr;
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x[JT];
#pragma unroll
                                for (int jt = 0; jt < JT; ++jt) x[jt] = -Y[rt][jt][e];
                                store_cols<JT>(rb + (unsigned)((16 * rt + 4 * lq + e) * DV), x);
                            }
                    }
                }
                // Output rows 16 rt + 4 lq + e: the part that varies by (rt, e) is uniform and goes into
                // a scalar row base; the lane's own part (its 4-row group and columns) is one 32-bit
                // offset, so each store needs no address arithmetic of its own.
                const unsigned o_lane = (unsigned)(4 * lq * H * DV + SWC * sw + JT * lr);
                float *const obase = TR && kind ? p.o_tr : p.o;
#pragma unroll
                for (int rt = 0; rt < 2 && !SO; ++rt) {
                    const F fa = M::template get<true>(sm + L::AQK, L::TRI_PLANE, fbase<1>(rt, 0, lane));
                    f32x4_t acc[JT];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt)
                        acc[jt] = *reinterpret_cast<const f32x4_t *>(sm + L::OST + ((JT * rt + jt) * 64 * NSW + 64 * sw + lane) * 16);
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) mma<true, true>(acc[jt], fa, UF[jt]);
                    float x[4][JT];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) x[e][jt] = p.scale * acc[jt][e];
                    if (nv == C32) {   // (uniform) a full chunk: no row past the end
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            store_cols<JT>(obase + ((size_t)(t0 + 16 * rt + e) * H + h) * DV + col0 + o_lane, x[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * rt + 4 * lq + e < nv)
                                store_cols<JT>(obase + ((size_t)(t0 + 16 * rt + e) * H + h) * DV + col0 + o_lane, x[e]);
                    }
                }
            }
            lds_barrier();

            // ---- seg 3, c(it): S <- Diag(Gamma_last) S + (e^{G_last-G} K)^T U
            if (it >= 0) {
                const int buf = it & 1;
                const float *s_gc = reinterpret_cast<const float *>(sm + L::GC) + buf * DK;
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) {
                    const F fk = M::template get<true>(sm + L::KHT + buf * L::KHT_BUF, L::KHT_PLANE,
                                                       fbase<1>(ct, 0, lane));
                    const float4 gc = *reinterpret_cast<const float4 *>(s_gc + 16 * ct + 4 * lq);
                    const float gcv[4] = {gc.x, gc.y, gc.z, gc.w};
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        f32x4_t acc;
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = gcv[e] * Sr[jt][ct][e];
                        mma<true, true>(acc, fk, UF[jt]);
                        Sr[jt][ct] = acc;
                    }
                }
                if (every_chunks > 0 && --ck_left == 0 && nv == C32) {
                    // state after in-sequence position (it + 1) * 32, a multiple of checkpoint_every
                    ck_left = every_chunks;
                    const int64_t m = p.ckpt_base[n] + ck_idx++;
                    float *const dbase = TR && kind ? p.ckpt_tr + ((size_t)m * H + h) * DK * DV
                                                    : ckpt_dst(p, m, h, DK * DV);   // NULL: not kept
                    if (dbase) {
                        float *const dst = dbase + col0;
#pragma unroll
                        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x[JT];
#pragma unroll
                                for (int jt = 0; jt < JT; ++jt) x[jt] = Sr[jt][ct][e];
                                store_cols<JT>(dst + (unsigned)((16 * ct + 4 * lq + e) * DV + SWC * sw + JT * lr), x);
                            }
                    }
                }
            }
            lds_barrier();
        }

        if (p.sf) {
            // (lane index recomputed opaquely: row offsets shared with the initial-state loads
            // would otherwise be kept live in registers across the whole loop)
            const int lane = lane_id(), lr = lane & 15, lq = lane >> 4;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x[JT];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) x[jt] = Sr[jt][ct][e];
                    store_cols<JT>(p.sf + st_off + (size_t)(16 * ct + 4 * lq + e) * DV + col0 + SWC * sw + JT * lr, x);
                }
        }
    } else {
        // ============================== prep waves ==============================
        // Thread pt = (rgp, cp): rows 4 rgp .. 4 rgp + 3 of the chunk, channels 2 cp, 2 cp + 1.
        const int pw = wave < SCAN0 ? wave : wave - NSW;     // prep wave index
        const int pt = 64 * pw + ((int)threadIdx.x & 63);
        const int cp = pt % NCP, c0 = 2 * cp;
        // the 4-row group is uniform across a wave when a wave covers one group (DK = 128)
        const int rgp = NCP >= 64 ? __builtin_amdgcn_readfirstlane(pt / NCP) : pt / NCP;
        // the sub-chunk is wave-uniform either way (with DK = 64 a wave holds groups 2 pw, 2 pw + 1)
        const int sa = __builtin_amdgcn_readfirstlane(rgp >> 2), gi = rgp & 3;
        // The waves of the second sub-chunk carry its extra operands (Gamma*K and Gamma*Q of rows
        // 16..31) and are the longest path of every segment: they issue ahead of the other prep and
        // scan waves (the role waves, at 3, still go first).
        if (NRW > 0 && sa) __builtin_amdgcn_s_setprio(2);
        const int lane = pt & 63, lr = lane & 15, lq = lane >> 4;
        // per-thread LDS element offsets and input row offsets, fixed for the whole sequence
        int ks_off[4], kn_off[4], vb_off[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rgp + i, rl = r - 16 * sa;
            ks_off[i] = fofs<KB>(r, c0);                 // KS and QS share the layout
            kn_off[i] = fofs<KB>(16 * sa + rl, c0);
            vb_off[i] = r * L::VPITCH + c0 * 4;
        }
        const int kht_off0 = fofs<1>(c0, 4 * rgp), kht_off1 = fofs<1>(c0 + 1, 4 * rgp);

        // structurally zero blocks: columns 16..31 of TM rows 0..15, of AQK rows 0..15, of AW
        for (int idx = pt; idx < 256; idx += 64 * NPW) {
            const int r = idx >> 4, c = 16 + (idx & 15);
            M::put_hl1(smem + L::TM, L::TRI_PLANE, fofs<1>(r, c), 0.f);
            M::put_hl1(smem + L::AQK, L::TRI_PLANE, fofs<1>(r, c), 0.f);
            M::put_hl1(smem + L::AW, L::AW_PLANE, fofs<1>(r, c), 0.f);
        }

        typename PR::raw kn_[4], qn_[4], vn_[4];   // raw rows of the chunk prepared next
        float2 gn_[4];
        float bn_ = 0.f;
        auto prefetch = [&](int ch) {
            // chunk base in a scalar register, per-thread 32-bit row offsets
            const int t0 = seq_start + ch * C32, nv = min(C32, seq_len - ch * C32);
            const size_t base = (size_t)t0 * H * DK;
            const IN_T *kb = kg + base, *qb = qg + base;
            const float *gb = p.g + base;
            const uint16_t *ab = reinterpret_cast<const uint16_t *>(p.g) + base;   // bf16 pre-activations
            constexpr bool pre = PRO & KDA_PRO_GATE;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = min(4 * rgp + i, nv - 1);
                const unsigned off = (unsigned)((r * H + h) * DK + c0);
                kn_[i] = PR::load(kb + off);
                if constexpr (SO) qn_[i] = PR::zero();
                else qn_[i] = PR::load(qb + off);
                if constexpr (pre) gn_[i].x = __uint_as_float(*reinterpret_cast<const uint32_t *>(ab + off));   // a pair
                else gn_[i] = *reinterpret_cast<const float2 *>(gb + off);
            }
            bn_ = p.beta[(size_t)t0 * H + (unsigned)(min(4 * rgp + (cp & 3), nv - 1) * H + h)];
        };
        auto vfetch = [&](int ch) {   // value rows: staged to LDS in segment 3, so fetched separately
            if (kind) {
#pragma unroll
                for (int i = 0; i < 4; ++i) vn_[i] = PR::zero();
                return;
            }
            const int t0 = seq_start + ch * C32, nv = min(C32, seq_len - ch * C32);
            const IN_T *vb = vg + (size_t)t0 * H * DV;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = min(4 * rgp + i, nv - 1);
                vn_[i] = PR::load(vb + (unsigned)((r * H + h) * DV + c0));
            }
        };
        if (nchunks > 0) {
            prefetch(0);
            vfetch(0);
        }

        typename PR::raw kr[4], qr[4];   // this chunk's k, q pairs from P1 to P2
        float Fw[4][2], Bw[4][2];        // decay products within the 4-row group: through row i / after row i
        float kh[2][4], gl[2];           // (e^{G_last-G} K)^T entries and Gamma_last, from P2 to P3
        float2 nrm[4];                   // 1/|k|, 1/|q| of this thread's rows, from P1 to P2 (fused normalisation)
        if constexpr (NRW > 0 && (PRO & KDA_PRO_NORM) != 0) lds_barrier();   // the role waves' first norms

        for (int it = -1; it < nchunks; ++it) {
            char *const sm = smem + opaque_s(0);
            const int nxt = it + 1;
            const bool have = nxt < nchunks;
            float *s_xchg = reinterpret_cast<float *>(sm + L::XCHG);
            float *s_beta = reinterpret_cast<float *>(sm + L::BETA) + (nxt & 1) * 32;   // chunk nxt's

            // ---- seg 1, P1(nxt): alpha = exp(g), running products over the 4-row group
            if (have) {
                if constexpr ((PRO & KDA_PRO_NORM) != 0 && NRW > 0) {
                    // formed by the role waves one iteration ahead: read first thing here (off segment
                    // 2's path), so that the reads' latency passes under this segment's work
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        nrm[i] = *reinterpret_cast<const float2 *>(sm + L::NRM + (nxt & 1) * L::NRM_BUF + (4 * rgp + i) * 8);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int nv = min(C32, seq_len - nxt * C32);
                constexpr bool pre = PRO & KDA_PRO_GATE;
                float al[4][2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = 4 * rgp + i < nv;   // padded rows: k = q = 0, alpha = 1, beta = 0
                    kr[i] = valid ? kn_[i] : PR::zero();
                    qr[i] = valid ? qn_[i] : PR::zero();
                    if constexpr (pre && GTAB) {
                        // fused gate from the table: alpha of a bf16 pair a in one LDS read each
                        const uint32_t ab = __float_as_uint(gn_[i].x);
                        const float *tab = reinterpret_cast<const float *>(sm + L::TOTAL);
                        const float t0 = tab[gate_index(ab)], t1 = tab[gate_index(ab >> 16)];
                        al[i][0] = valid ? t0 : 1.f;
                        al[i][1] = valid ? t1 : 1.f;
                    } else if constexpr (pre) {
                        // fused gate: alpha = exp(-5 sigmoid(a)), a a bf16 pair
                        const uint32_t ab = __float_as_uint(gn_[i].x);
                        al[i][0] = valid ? gate_decay(lo_bf16_of(ab)) : 1.f;
                        al[i][1] = valid ? gate_decay(hi_bf16_of(ab)) : 1.f;
                    } else {
                        al[i][0] = valid ? __expf(gn_[i].x) : 1.f;
                        al[i][1] = valid ? __expf(gn_[i].y) : 1.f;
                    }
                }
                if (cp < 4) {
                    float bv = bn_;
                    if constexpr (pre) bv = __builtin_amdgcn_rcpf(1.f + __expf(-bn_));   // sigmoid(b)
                    s_beta[4 * rgp + cp] = 4 * rgp + cp < nv ? bv : 0.f;
                }
                if constexpr ((PRO & KDA_PRO_NORM) != 0 && NRW == 0) {
                    // 1/|k|, 1/|q| of each row (0 for a zero row): sums of squares over the NCP lanes
                    // holding the row, then one lane per group -> LDS for P2
                    float ss[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float k0 = PR::lo(kr[i]), k1 = PR::hi(kr[i]), q0 = PR::lo(qr[i]), q1 = PR::hi(qr[i]);
                        ss[2 * i] = k0 * k0 + k1 * k1;
                        ss[2 * i + 1] = q0 * q0 + q1 * q1;
                    }
                    // inside each row of 16 lanes by DPP rotations, then across the rows
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        ss[j] += dpp_f32<0x128>(ss[j]);   // row_ror:8
                        ss[j] += dpp_f32<0x124>(ss[j]);   // row_ror:4
                        ss[j] += dpp_f32<0x122>(ss[j]);   // row_ror:2
                        ss[j] += dpp_f32<0x121>(ss[j]);   // row_ror:1
                    }
                    // across the four 16-lane rows by DPP row broadcasts (rows 1, 3 take the row
                    // before; rows 2, 3 take lane 31): lane 63 ends with the total, read out uniformly
                    static_assert(NCP == 64, "a row's channel pairs span the whole wave");
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        ss[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss[j]), 0x142, 0xA, 0xF, false));
                        ss[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss[j]), 0x143, 0xC, 0xF, false));
                        ss[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss[j]), 63));
                    }
                    if (cp == 0) {
                        float nr[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) nr[j] = ss[j] > 0.f ? rsqrtf(ss[j]) : 0.f;
                        float4 *dn = reinterpret_cast<float4 *>(sm + L::NRM + 4 * rgp * 8);
                        dn[0] = make_float4(nr[0], nr[1], nr[2], nr[3]);
                        dn[1] = make_float4(nr[4], nr[5], nr[6], nr[7]);
                    }
                }
                float tot[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float f = 1.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) { f *= al[i][c]; Fw[i][c] = f; }
                    float b = 1.f;
#pragma unroll
                    for (int i = 3; i >= 0; --i) { Bw[i][c] = b; b *= al[i][c]; }
                    tot[c] = f;
                }
                *reinterpret_cast<float2 *>(s_xchg + rgp * DK + c0) = make_float2(tot[0], tot[1]);
                // Unconditional (the last chunk re-reads itself): a conditional refill would make
                // the loop-carried registers a join of old and new values, and the compiler
                // would then wait for the loads right here to copy them over.
                prefetch(min(nxt + 1, nchunks - 1));
            }
            if (NRW == 0 && it >= 0 && pw < 2) diag_inverse_lds(sm, pw, it, lane);
            lds_barrier();

            // ---- seg 2, P2(nxt): decayed operands
            // (sub-chunk SA and group GI of this thread's rows: compile-time constants where a wave
            // holds one row group, so the selections below fold away)
            auto p2 = [&](auto sa_c, auto gi_c) {
                const int SA = sa_c, GI = gi_c;
                // group products of this sub-chunk (xs) and of the other one (xo)
                float xs[4][2], xo[2] = {1.f, 1.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float2 a2 = *reinterpret_cast<const float2 *>(s_xchg + (4 * SA + m) * DK + c0);
                    const float2 o2 = *reinterpret_cast<const float2 *>(s_xchg + (4 * (1 - SA) + m) * DK + c0);
                    xs[m][0] = a2.x; xs[m][1] = a2.y;
                    xo[0] *= o2.x; xo[1] *= o2.y;
                }
                float lead[2], tail[2], P0[2], P1[2], dgf[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    lead[c] = 1.f;   // decay from the sub-chunk start to this group
                    tail[c] = 1.f;   // decay from the end of this group to the sub-chunk end
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        if (m < GI) lead[c] *= xs[m][c];
                        if (m > GI) tail[c] *= xs[m][c];
                    }
                    const float psub = (xs[0][c] * xs[1][c]) * (xs[2][c] * xs[3][c]);
                    P0[c] = SA ? xo[c] : psub;
                    P1[c] = SA ? psub : xo[c];
                    dgf[c] = __builtin_amdgcn_rcpf(SA ? P1[c] : P0[c]);   // column factor of the diagonal Gram tile
                }
                gl[0] = P0[0] * P1[0];
                gl[1] = P0[1] * P1[1];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ks[2], qs[2], ke[2], kd[2];
                    float kv[2] = {PR::lo(kr[i]), PR::hi(kr[i])}, qv[2] = {PR::lo(qr[i]), PR::hi(qr[i])};
                    if constexpr ((PRO & KDA_PRO_NORM) != 0) {   // fused normalisation: row factors from P1
                        const float2 nr = NRW > 0 ? nrm[i]
                                                  : *reinterpret_cast<const float2 *>(sm + L::NRM + (4 * rgp + i) * 8);
                        kv[0] *= nr.x; kv[1] *= nr.x;
                        qv[0] *= nr.y; qv[1] *= nr.y;
                    }
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const float es = Fw[i][c] * lead[c];   // e^{G_r - G_ref}
                        const float ee = Bw[i][c] * tail[c];   // e^{G_end(sub-chunk) - G_r}
                        ks[c] = kv[c] * es;
                        qs[c] = qv[c] * es;
                        ke[c] = kv[c] * ee;
                        kd[c] = ke[c] * dgf[c];
                        // (e^{G_last-G} K)^T entry: sub-chunk 0 decays on through sub-chunk 1
                        kh[c][i] = SA ? ke[c] : ke[c] * P1[c];
                    }
                    if (SO && p.rres) M::template put_hl<2>(sm + L::KS, L::SQ_PLANE, ks_off[i], ks);
                    else M::put_h2(sm + L::KS, ks_off[i], ks[0], ks[1]);
                    if constexpr (!SO) M::template put_hl<2>(sm + L::QS, L::SQ_PLANE, ks_off[i], qs);
                    // Kn rows (K e^{G_ref(a) - G}): sub-chunk 0 feeds tiles (0,0) and (1,0), sub-chunk 1 (1,1)
                    M::template put_hl<2>(sm + L::KN, L::KN_PLANE, kn_off[i], kd);
                    if (SA) {
                        // Gamma * K and Gamma * Q of rows 16..31 (decay from the chunk start): read by
                        // the (1,0) Gram tiles in segment 3 and by stage a in segment 1 of the next iteration
                        if (SO && p.rres) {
                            const float kg2[2] = {ks[0] * P0[0], ks[1] * P0[1]};
                            M::template put_hl<2>(sm + L::KG_AT, L::KG_LO, ks_off[i], kg2);
                        } else {
                            M::put_h2(sm + L::KG_AT, ks_off[i], ks[0] * P0[0], ks[1] * P0[1]);
                        }
                        if constexpr (!SO) {
                            const float qt[2] = {qs[0] * P0[0], qs[1] * P0[1]};
                            M::template put_hl<2>(sm + L::QT_AT, L::QT_PLANE, ks_off[i], qt);
                        }
                    }
                }
            };
            if (have) {
                if constexpr (NCP >= 64) {
                    using Z = std::integral_constant<int, 0>;
                    using O = std::integral_constant<int, 1>;
                    switch (rgp) {
                        case 0: p2(Z{}, Z{}); break;
                        case 1: p2(Z{}, O{}); break;
                        case 2: p2(Z{}, std::integral_constant<int, 2>{}); break;
                        case 3: p2(Z{}, std::integral_constant<int, 3>{}); break;
                        case 4: p2(O{}, Z{}); break;
                        case 5: p2(O{}, O{}); break;
                        case 6: p2(O{}, std::integral_constant<int, 2>{}); break;
                        default: p2(O{}, std::integral_constant<int, 3>{}); break;
                    }
                } else {
                    // (a wave's rows share their sub-chunk: dispatch on it, the group stays per lane)
                    if (sa) p2(std::integral_constant<int, 1>{}, gi);
                    else p2(std::integral_constant<int, 0>{}, gi);
                }
            }
            lds_barrier();

            // ---- seg 3, P3(nxt): Khat^T, Gamma_last, Gamma*Q, -V; Gram tiles (here or on the scan waves)
            if (have) {
                // (e^{G_last-G} K)^T and Gamma_last of chunk nxt, read by stage c in segment 3 of the
                // next iteration (double-buffered: stage c of chunk it reads the other buffer now).
                // The 4 rows of this group are 4 consecutive K-slots of one fragment.
                const int buf = nxt & 1;
                M::template put_hl<4>(sm + L::KHT + buf * L::KHT_BUF, L::KHT_PLANE, kht_off0, kh[0]);
                M::template put_hl<4>(sm + L::KHT + buf * L::KHT_BUF, L::KHT_PLANE, kht_off1, kh[1]);
                if (rgp == 0)
                    *reinterpret_cast<float2 *>(sm + L::GC + (buf * DK + c0) * 4) = make_float2(gl[0], gl[1]);
                // -V of chunk nxt in fp32, read by stage a in segment 1 of the next iteration (stage a
                // of chunk it has finished with the buffer); then fetch chunk nxt + 1's
                const int nv = min(C32, seq_len - nxt * C32);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float2 *>(sm + L::VB + vb_off[i]) =
                        4 * rgp + i < nv ? make_float2(-PR::lo(vn_[i]), -PR::hi(vn_[i])) : make_float2(0.f, 0.f);
                vfetch(min(nxt + 1, nchunks - 1));
            }
            if (NRW == 0 && have && pw < 3) gram_tile(sm, pw, nxt, lane);
            lds_barrier();
        }
    }
}

}  // namespace kda

// max_split 1 keeps one workgroup per chain, for a launch that shares the chip with another kernel.
extern "C" __attribute__((visibility("hidden"))) hipError_t
kda_launch_chunk32_split(int dk, int in_bf16, unsigned chains, const kda::ChunkParams &p, int max_split,
                         hipStream_t stream) {
    // One workgroup per (sequence, head) chain; when the chains would leave more than half the
    // compute units idle, split each chain's value columns over two workgroups.
    const int split = max_split >= 2 && (long long)chains * 2 <= kda_cu_count() ? 2 : 1;
#define KDA_C32(DKV, SP, F32P, T, PRO)                                                                   \
    hipLaunchKernelGGL((kda::chunk32_kernel<DKV, SP, F32P, T, PRO>),                                    \
                       dim3(chains * SP * (((PRO) & kda::KDA_TRANSITION) ? 2 : 1)),                     \
                       dim3(kda::chunk32_threads<DKV, SP>()), 0, stream, p)
    const int pro = p.flags & (kda::KDA_PRO_GATE | kda::KDA_PRO_NORM);
    if (p.flags & ~(kda::KDA_PRO_GATE | kda::KDA_PRO_NORM | kda::KDA_STATES_ONLY | kda::KDA_TRANSITION))
        return hipErrorInvalidValue;
    if ((p.flags & kda::KDA_TRANSITION) && (p.flags & kda::KDA_STATES_ONLY)) return hipErrorInvalidValue;
    if (pro != 0 && (dk != 128 || !in_bf16)) return hipErrorInvalidValue;   // fused prologue: bf16, d_k = 128
    // (S: SPLIT, F: the flags, both compile-time)
#define KDA_C32_DT(S, F)                                                                                    \
    do {                                                                                                   \
        if (dk == 128 && in_bf16) KDA_C32(128, S, false, uint16_t, F);                                     \
        else if (dk == 128) KDA_C32(128, S, true, float, F);                                               \
        else if (dk == 64 && in_bf16) KDA_C32(64, S, false, uint16_t, F);                                  \
        else if (dk == 64) KDA_C32(64, S, true, float, F);                                                 \
        else return hipErrorInvalidValue;                                                                  \
    } while (0)
#define KDA_C32_FLAGS(S)                                                                                    \
    do {                                                                                                   \
        switch (p.flags) {                                                                                 \
            case 0: KDA_C32_DT(S, 0); break;                                                               \
            case 1: KDA_C32(128, S, false, uint16_t, 1); break;                                            \
            case 2: KDA_C32(128, S, false, uint16_t, 2); break;                                            \
            case 3: KDA_C32(128, S, false, uint16_t, 3); break;                                            \
            case 4: KDA_C32_DT(S, 4); break;                                                               \
            case 5: KDA_C32(128, S, false, uint16_t, 5); break;                                            \
            case 6: KDA_C32(128, S, false, uint16_t, 6); break;                                            \
            case 7: KDA_C32(128, S, false, uint16_t, 7); break;                                            \
            default: return hipErrorInvalidValue;                                                          \
        }                                                                                                  \
    } while (0)
    if (p.flags & kda::KDA_TRANSITION) {
        // the paired segment pass: one workgroup per chain and kind
        switch (p.flags) {
            case 16: KDA_C32_DT(1, 16); break;
            case 17: KDA_C32(128, 1, false, uint16_t, 17); break;
            case 18: KDA_C32(128, 1, false, uint16_t, 18); break;
            case 19: KDA_C32(128, 1, false, uint16_t, 19); break;
            default: return hipErrorInvalidValue;
        }
    } else if (split == 2) {
        KDA_C32_FLAGS(2);
    } else {
        KDA_C32_FLAGS(1);
    }
#undef KDA_C32_FLAGS
#undef KDA_C32_DT
#undef KDA_C32
    return hipGetLastError();
}

extern "C" __attribute__((visibility("hidden"))) hipError_t
kda_launch_chunk32(int dk, int in_bf16, unsigned chains, const kda::ChunkParams &p, hipStream_t stream) {
    return kda_launch_chunk32_split(dk, in_bf16, chains, p, 2, stream);
}
