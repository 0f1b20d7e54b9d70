// kda_api.hip -- the C ABI of libkda (declared in include/kda.h).
//
// Host-side argument validation (pure host code: it runs before any launch
// and touches no device memory), workspace sizing, and kernel dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kda.h"

extern "C" hipError_t kda_launch_decode(int dk, int in_bf16, int N, int H, const void *q, const void *k,
                                        const void *v, const float *g, const float *beta, float *state,
                                        const int32_t *slots, int nslots, float *o, float scale, int flags,
                                        hipStream_t stream);
extern "C" size_t kda_chunk_workspace_layout(int N, size_t *order_off, size_t *base_off);
extern "C" hipError_t kda_launch_chunk(int chunk, int dk, int in_bf16, int N, int H, const void *q, const void *k,
                                       const void *v, const float *g, const float *beta, const int32_t *cu,
                                       const float *s0, float *sf, int every, float *ckpt, float *o,
                                       float scale, const int32_t *s0_idx, const int32_t *ck_idx,
                                       int nslots, int flags, void *workspace, hipStream_t stream);
extern "C" hipError_t kda_launch_prologue(int dk, long long rows, int flags, const void *q, const void *k,
                                          const void *v, const float *a, const float *b, float *qn, float *kn,
                                          float *vf, float *g, float *beta, hipStream_t stream);
extern "C" size_t kda_bwd_workspace_layout(int N, int H, int T, int dk, int dv, int64_t n_ck, int64_t n_chunks,
                                           int flags, size_t *off);
extern "C" hipError_t kda_launch_bwd(int dk, int in_bf16, int N, int H, int T, int64_t n_ck, int64_t n_chunks,
                                     const void *q, const void *k, const void *v, const float *g, const float *beta,
                                     const int32_t *cu, const float *s0, const float *dO, const float *dSf, float *dq,
                                     float *dkk, float *dv, float *dg, float *dbeta, float *dS0, float scale,
                                     const float *states, int flags, void *workspace, hipStream_t stream);

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_dims(int dk, int dv, kda_dtype dt) {
    if (dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Validation shared by kda_chunk_fwd and the workspace query.
kda_status validate_fwd(const kda_fwd_args *a) {
    if (!a) return KDA_ERR_INVALID_ARGUMENT;
    if (a->struct_size != sizeof(kda_fwd_args)) return KDA_ERR_INVALID_ARGUMENT;
    if (a->num_seqs < 0 || a->total_tokens < 0 || a->num_heads <= 0) return KDA_ERR_INVALID_ARGUMENT;
    const kda_status d = check_dims(a->dk, a->dv, a->in_dtype);
    if (d != KDA_OK) return d;
    if (a->chunk_size != 32 && a->chunk_size != 64) return KDA_ERR_UNSUPPORTED;
    if (a->checkpoint_every < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (a->checkpoint_every > 0 && a->checkpoint_every % a->chunk_size != 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!a->cu_seqlens_host) return KDA_ERR_INVALID_ARGUMENT;
    if (a->num_seqs > 0 && !a->cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
    const int32_t *cu = a->cu_seqlens_host;
    if (cu[0] != 0) return KDA_ERR_INVALID_ARGUMENT;
    for (int n = 0; n < a->num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return KDA_ERR_INVALID_ARGUMENT;
    if (cu[a->num_seqs] != a->total_tokens) return KDA_ERR_INVALID_ARGUMENT;
    if (a->total_tokens > 0) {
        if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->g) ||
            !aligned16(a->beta) || !aligned16(a->o))
            return KDA_ERR_INVALID_ARGUMENT;
        if ((const void *)a->o == a->q || (const void *)a->o == a->k || (const void *)a->o == a->v ||
            (const void *)a->o == a->g || (const void *)a->o == a->beta)
            return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((a->initial_state && !aligned16(a->initial_state)) || (a->final_state && !aligned16(a->final_state)))
        return KDA_ERR_INVALID_ARGUMENT;
    if (a->checkpoint_every > 0) {
        int64_t m = 0;
        for (int n = 0; n < a->num_seqs; ++n) m += (cu[n + 1] - cu[n]) / a->checkpoint_every;
        if (m > 0 && (!a->checkpoints || !aligned16(a->checkpoints))) return KDA_ERR_INVALID_ARGUMENT;
    }
    if (!(a->scale == a->scale)) return KDA_ERR_INVALID_ARGUMENT;  // NaN scale
    // paged pool: the indices need their pool, and the pool a size
    if ((a->initial_state_indices || a->checkpoint_indices) && a->num_slots < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (a->initial_state_indices && a->num_seqs > 0 && !a->initial_state) return KDA_ERR_INVALID_ARGUMENT;
    if (a->checkpoint_indices && a->checkpoint_every == 0) return KDA_ERR_INVALID_ARGUMENT;
    // fused prologue
    if ((a->gate_mode != KDA_GATE_LOG_DECAY && a->gate_mode != KDA_GATE_PREACTIVATION) ||
        (a->normalize_qk != 0 && a->normalize_qk != 1))
        return KDA_ERR_INVALID_ARGUMENT;
    if ((a->gate_mode != KDA_GATE_LOG_DECAY || a->normalize_qk) && a->in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

int fwd_flags(const kda_fwd_args *a) {
    return (a->gate_mode == KDA_GATE_PREACTIVATION ? 1 : 0) | (a->normalize_qk ? 2 : 0);
}

// The forward's workspace: the launch plan, then, when the prologue cannot be fused (it is fused
// for chunk 32 at dk = 128), its outputs: fp32 q / |q|, k / |k|, v (normalisation) and g, beta
// (gate).  off[0..5]: qn, kn, vf, g, beta, end.
size_t fwd_workspace(const kda_fwd_args *a, size_t *off) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const int flags = fwd_flags(a);
    const bool mat = flags != 0 && !(a->chunk_size == 32 && a->dk == 128);
    const size_t rows = (size_t)a->total_tokens * a->num_heads;
    size_t o[6];
    o[0] = up(kda_chunk_workspace_layout(a->num_seqs, nullptr, nullptr));
    const bool nrm = mat && (flags & 2), gate = mat && (flags & 1);
    o[1] = o[0] + (nrm ? up(rows * a->dk * 4) : 0);
    o[2] = o[1] + (nrm ? up(rows * a->dk * 4) : 0);
    o[3] = o[2] + (nrm ? up(rows * a->dv * 4) : 0);
    o[4] = o[3] + (gate ? up(rows * a->dk * 4) : 0);
    o[5] = o[4] + (gate ? up(rows * 4) : 0);
    if (off)
        for (int i = 0; i < 6; ++i) off[i] = o[i];
    return mat ? o[5] : kda_chunk_workspace_layout(a->num_seqs, nullptr, nullptr);
}

// Validation of kda_chunk_bwd (and its workspace query); also counts the 32-token checkpoints
// and chunks the workspace holds.
kda_status validate_bwd(const kda_bwd_args *a, int64_t *n_ck, int64_t *n_chunks) {
    if (!a) return KDA_ERR_INVALID_ARGUMENT;
    if (a->struct_size != sizeof(kda_bwd_args)) return KDA_ERR_INVALID_ARGUMENT;
    if (a->num_seqs < 0 || a->total_tokens < 0 || a->num_heads <= 0) return KDA_ERR_INVALID_ARGUMENT;
    const kda_status d = check_dims(a->dk, a->dv, a->in_dtype);
    if (d != KDA_OK) return d;
    if (!(a->scale == a->scale)) return KDA_ERR_INVALID_ARGUMENT;
    if (!a->cu_seqlens_host) return KDA_ERR_INVALID_ARGUMENT;
    if (a->num_seqs > 0 && !a->cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
    const int32_t *cu = a->cu_seqlens_host;
    if (cu[0] != 0) return KDA_ERR_INVALID_ARGUMENT;
    int64_t ck = 0, ch = 0;
    for (int n = 0; n < a->num_seqs; ++n) {
        if (cu[n + 1] < cu[n]) return KDA_ERR_INVALID_ARGUMENT;
        ck += (cu[n + 1] - cu[n]) / 32;
        ch += (cu[n + 1] - cu[n] + 31) / 32;
    }
    if (cu[a->num_seqs] != a->total_tokens) return KDA_ERR_INVALID_ARGUMENT;
    const void *in[] = {a->q, a->k, a->v, a->g, a->beta, a->d_o, a->initial_state, a->d_final_state, a->states};
    const void *out[] = {a->dq, a->dk_out, a->dv_out, a->dg, a->dbeta, a->d_initial_state};
    if (a->total_tokens > 0) {
        for (int i = 0; i < 6; ++i)
            if (!in[i] || !aligned16(in[i])) return KDA_ERR_INVALID_ARGUMENT;
        for (int i = 0; i < 5; ++i)
            if (!out[i] || !aligned16(out[i])) return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((a->initial_state && !aligned16(a->initial_state)) || (a->d_final_state && !aligned16(a->d_final_state)) ||
        (a->d_initial_state && !aligned16(a->d_initial_state)) || (a->states && !aligned16(a->states)))
        return KDA_ERR_INVALID_ARGUMENT;
    // no output may alias another output or an input
    for (int i = 0; i < 6; ++i) {
        if (!out[i]) continue;
        for (int j = 0; j < 9; ++j)
            if (out[i] == in[j]) return KDA_ERR_INVALID_ARGUMENT;
        for (int j = i + 1; j < 6; ++j)
            if (out[i] == out[j]) return KDA_ERR_INVALID_ARGUMENT;
    }
    // fused prologue (as in the forward): gate pre-activations and/or normalisation, bf16 inputs
    if ((a->gate_mode != KDA_GATE_LOG_DECAY && a->gate_mode != KDA_GATE_PREACTIVATION) ||
        (a->normalize_qk != 0 && a->normalize_qk != 1))
        return KDA_ERR_INVALID_ARGUMENT;
    if ((a->gate_mode != KDA_GATE_LOG_DECAY || a->normalize_qk) && a->in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (n_ck) *n_ck = ck;
    if (n_chunks) *n_chunks = ch;
    return KDA_OK;
}

// prologue bits, and 8 when the caller passes the states (the workspace then holds none)
int bwd_flags(const kda_bwd_args *a) {
    return (a->gate_mode == KDA_GATE_PREACTIVATION ? 1 : 0) | (a->normalize_qk ? 2 : 0) | (a->states ? 8 : 0);
}

}  // namespace

extern "C" {

uint32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_chunk_fwd_workspace_bytes(const kda_fwd_args *a) {
    if (validate_fwd(a) != KDA_OK) return 0;
    return fwd_workspace(a, nullptr);
}

kda_status kda_chunk_fwd(const kda_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    const kda_status st = validate_fwd(a);
    if (st != KDA_OK) return st;
    size_t off[6];
    const size_t need = fwd_workspace(a, off);
    if (a->num_seqs > 0) {
        if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_INVALID_ARGUMENT;
    }
    if (a->num_seqs == 0) return KDA_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int flags = fwd_flags(a), in_bf16 = a->in_dtype == KDA_BF16;
    const void *q = a->q, *k = a->k, *v = a->v;
    const float *g = a->g, *beta = a->beta;
    if (flags != 0 && !(a->chunk_size == 32 && a->dk == 128)) {
        // the prologue runs as its own pass; the kernels then see its outputs
        char *ws = static_cast<char *>(workspace);
        float *qn = reinterpret_cast<float *>(ws + off[0]), *kn = reinterpret_cast<float *>(ws + off[1]);
        float *vf = reinterpret_cast<float *>(ws + off[2]), *gm = reinterpret_cast<float *>(ws + off[3]);
        float *bm = reinterpret_cast<float *>(ws + off[4]);
        if (kda_launch_prologue(a->dk, (long long)a->total_tokens * a->num_heads, flags, q, k, v, g, beta, qn, kn,
                                vf, gm, bm, s) != hipSuccess)
            return KDA_ERR_DEVICE;
        if (flags & 2) { q = qn; k = kn; v = vf; in_bf16 = 0; }
        if (flags & 1) { g = gm; beta = bm; }
        flags = 0;
    }
    const hipError_t e = kda_launch_chunk(a->chunk_size, a->dk, in_bf16, a->num_seqs, a->num_heads, q, k, v, g, beta,
                                          a->cu_seqlens, a->initial_state, a->final_state, a->checkpoint_every,
                                          a->checkpoints, a->o, a->scale, a->initial_state_indices,
                                          a->checkpoint_indices, a->num_slots, flags, workspace, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

size_t kda_chunk_bwd_workspace_bytes(const kda_bwd_args *a) {
    int64_t ck, ch;
    if (validate_bwd(a, &ck, &ch) != KDA_OK) return 0;
    return kda_bwd_workspace_layout(a->num_seqs, a->num_heads, a->total_tokens, a->dk, a->dv, ck, ch, bwd_flags(a),
                                    nullptr);
}

kda_status kda_chunk_bwd(const kda_bwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    int64_t ck = 0, ch = 0;
    const kda_status st = validate_bwd(a, &ck, &ch);
    if (st != KDA_OK) return st;
    if (a->num_seqs == 0) return KDA_OK;
    const size_t need = kda_bwd_workspace_layout(a->num_seqs, a->num_heads, a->total_tokens, a->dk, a->dv, ck, ch,
                                                 bwd_flags(a), nullptr);
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_INVALID_ARGUMENT;
    const hipError_t e = kda_launch_bwd(a->dk, a->in_dtype == KDA_BF16, a->num_seqs, a->num_heads, a->total_tokens,
                                        ck, ch, a->q, a->k, a->v, a->g, a->beta, a->cu_seqlens, a->initial_state,
                                        a->d_o, a->d_final_state, a->dq, a->dk_out, a->dv_out, a->dg, a->dbeta,
                                        a->d_initial_state, a->scale, a->states, bwd_flags(a) & 3, workspace,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status kda_decode_step(const kda_decode_args *a, void *stream) {
    if (!a || a->struct_size != sizeof(kda_decode_args)) return KDA_ERR_INVALID_ARGUMENT;
    if (a->num_seqs < 0 || a->num_heads <= 0) return KDA_ERR_INVALID_ARGUMENT;
    const kda_status d = check_dims(a->dk, a->dv, a->in_dtype);
    if (d != KDA_OK) return d;
    if (a->state_indices && a->num_slots < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!(a->scale == a->scale)) return KDA_ERR_INVALID_ARGUMENT;
    if ((a->gate_mode != KDA_GATE_LOG_DECAY && a->gate_mode != KDA_GATE_PREACTIVATION) ||
        (a->normalize_qk != 0 && a->normalize_qk != 1))
        return KDA_ERR_INVALID_ARGUMENT;
    if ((a->gate_mode != KDA_GATE_LOG_DECAY || a->normalize_qk) && a->in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->num_seqs == 0) return KDA_OK;
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->state || !a->o) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(a->state) || !aligned16(a->o) || !aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) ||
        !aligned16(a->g) || !aligned16(a->beta))
        return KDA_ERR_INVALID_ARGUMENT;
    if ((void *)a->o == (void *)a->state) return KDA_ERR_INVALID_ARGUMENT;
    const hipError_t e = kda_launch_decode(a->dk, a->in_dtype == KDA_BF16, a->num_seqs, a->num_heads, a->q, a->k,
                                           a->v, a->g, a->beta, a->state, a->state_indices, a->num_slots, a->o,
                                           a->scale,
                                           (a->gate_mode == KDA_GATE_PREACTIVATION ? 1 : 0) | (a->normalize_qk ? 2 : 0),
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

}  // extern "C"
