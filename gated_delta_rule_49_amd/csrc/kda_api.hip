// kda_api.hip -- the C ABI of libkda (declared in include/kda.h).
//
// Host-side argument validation (pure host code: it runs before any launch
// and touches no device memory), workspace sizing, and kernel dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "kda.h"
#include "kda_common.h"
#include "kda_bwd_flags.h"
#include "kda_side.h"

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
extern "C" size_t kda_segments_workspace_layout(int N, int NB, int H, int d, int T, int64_t nck, size_t *off);
extern "C" hipError_t kda_launch_chunk_segmented(int dk, int in_bf16, int N, int H, int T, int seg, int NB,
                                                 int64_t nck, const void *q, const void *k, const void *v,
                                                 const float *g, const float *beta, const int32_t *cu, const float *s0,
                                                 float *sf, int every, float *ckpt, float *o, float scale,
                                                 const int32_t *s0_idx, const int32_t *ck_idx, int nslots, int flags,
                                                 void *workspace, hipStream_t stream);
extern "C" hipError_t kda_launch_prologue(int dk, long long rows, int flags, const void *q, const void *k,
                                          const void *v, const float *a, const float *b, float *qn, float *kn,
                                          float *vf, float *g, float *beta, hipStream_t stream);
extern "C" size_t kda_bwd_workspace_layout(int N, int H, int T, int dk, int dv, int64_t n_ck, int64_t n_chunks,
                                           int flags, size_t *off);
extern "C" hipError_t kda_launch_cu_rebase(const int32_t *cu, int first, int n, int32_t *out, hipStream_t stream);
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
    // segments
    if (a->segment_tokens < -1) return KDA_ERR_INVALID_ARGUMENT;
    if (a->segment_tokens > 0) {
        if (a->segment_tokens % 32 != 0) return KDA_ERR_INVALID_ARGUMENT;
        if (a->checkpoint_every > 0 && a->segment_tokens % a->checkpoint_every != 0) return KDA_ERR_INVALID_ARGUMENT;
        if (a->chunk_size != 32) return KDA_ERR_UNSUPPORTED;
        // the segment launches' grids (2 workgroups per segment and head) stay within int range
        int64_t nb = 0;
        for (int n = 0; n < a->num_seqs; ++n) {
            const int32_t L = cu[n + 1] - cu[n];
            nb += L > 0 ? (L + (int64_t)a->segment_tokens - 1) / a->segment_tokens : 1;
        }
        if (nb * a->num_heads * 2 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    }
    return KDA_OK;
}

// Where the forward cuts its sequences into segments (see segment_tokens): returns the segment
// length, 0 for no cut, the number of segments in *nb and of checkpoints in *nck.  The library's own
// choice (segment_tokens 0) cuts only when the uncut launch leaves most of the chip idle --
// (sequence, head) pairs at most half the compute units, each pair then running on two workgroups
// -- into about CUs / 2 (segment, head) pairs, whose two runs then fill the chip; and only when the
// longest sequence spans at least 3 segments (the cut runs most segments twice, so the critical
// path must shrink by more).  Validated arguments only.
int segment_plan(const kda_fwd_args *a, int *nb, int64_t *nck) {
    *nb = 0;
    *nck = 0;
    if (a->segment_tokens < 0 || a->chunk_size != 32 || a->num_seqs == 0) return 0;
    const int32_t *cu = a->cu_seqlens_host;
    const int N = a->num_seqs, H = a->num_heads;
    int64_t seg = a->segment_tokens;
    if (seg == 0) {
        const int cus = kda_cu_count();
        if ((int64_t)N * H * 2 > cus) return 0;
        const int target = cus / (2 * H);
        if (target < 2) return 0;
        const int64_t unit = a->checkpoint_every > 0 ? a->checkpoint_every : 32;   // a multiple of 32
        seg = ((int64_t)a->total_tokens + target - 1) / target;
        seg = seg < 512 ? 512 : seg;   // shorter segments: launches and the chain of maps dominate
        seg = (seg + unit - 1) / unit * unit;
        int32_t lmax = 0;
        for (int n = 0; n < N; ++n) lmax = cu[n + 1] - cu[n] > lmax ? cu[n + 1] - cu[n] : lmax;
        if (lmax < 3 * seg || seg > INT32_MAX) return 0;
    }
    int64_t count = 0, ck = 0;
    for (int n = 0; n < N; ++n) {
        const int32_t L = cu[n + 1] - cu[n];
        count += L > 0 ? (L + seg - 1) / seg : 1;
        ck += a->checkpoint_every > 0 ? L / a->checkpoint_every : 0;
    }
    *nb = (int)count;
    *nck = ck;
    return (int)seg;
}

int fwd_flags(const kda_fwd_args *a) {
    return (a->gate_mode == KDA_GATE_PREACTIVATION ? 1 : 0) | (a->normalize_qk ? 2 : 0);
}

// The forward's workspace: the launch plan, then, when the prologue cannot be fused (it is fused
// for chunk 32 at dk = 128), its outputs: fp32 q / |q|, k / |k|, v (normalisation) and g, beta
// (gate); then, when the sequences are cut into segments, the segments' plan and states.
// off[0..6]: qn, kn, vf, g, beta, segments, end.
size_t fwd_workspace(const kda_fwd_args *a, size_t *off) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const int flags = fwd_flags(a);
    const bool mat = flags != 0 && !(a->chunk_size == 32 && a->dk == 128);
    const size_t rows = (size_t)a->total_tokens * a->num_heads;
    size_t o[7];
    o[0] = up(kda_chunk_workspace_layout(a->num_seqs, nullptr, nullptr));
    const bool nrm = mat && (flags & 2), gate = mat && (flags & 1);
    o[1] = o[0] + (nrm ? up(rows * a->dk * 4) : 0);
    o[2] = o[1] + (nrm ? up(rows * a->dk * 4) : 0);
    o[3] = o[2] + (nrm ? up(rows * a->dv * 4) : 0);
    o[4] = o[3] + (gate ? up(rows * a->dk * 4) : 0);
    o[5] = o[4] + (gate ? up(rows * 4) : 0);
    int nb = 0;
    int64_t nck = 0;
    const int seg = segment_plan(a, &nb, &nck);
    o[6] = o[5] + (seg > 0 ? kda_segments_workspace_layout(a->num_seqs, nb, a->num_heads, a->dk, a->total_tokens,
                                                           nck, nullptr)
                           : 0);
    if (off)
        for (int i = 0; i < 7; ++i) off[i] = o[i];
    return mat || seg > 0 ? o[6] : kda_chunk_workspace_layout(a->num_seqs, nullptr, nullptr);
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

// The state-gradient scan with one workgroup per chain serves batches whose chains all run the whole
// scan at full load: at least 3 x 8 column-block workgroups per compute unit's worth of chains for
// the scan split over column blocks (which that one runs at contention), and sequences of nearly
// equal length (the longest at most 5/4 of the mean), since a long chain's tail runs faster split.
int bwd_scan_choice(const int32_t *cu, int first, int last, int H) {
    const int n = last - first;
    int longest = 0;
    for (int i = first; i < last; ++i) longest = cu[i + 1] - cu[i] > longest ? cu[i + 1] - cu[i] : longest;
    const long long total = (long long)cu[last] - cu[first];
    const bool full = (long long)n * H * 8 >= 3LL * kda_cu_count();
    const bool even = total > 0 && 4LL * longest * n <= 5LL * total;
    return full && even ? kda::KDA_BWD_ONE_WG_SCAN : 0;
}

// Workspace of the backward of sequences [first, last) run as a group of their own: its layout
// plus their offsets rebased to the group's first token.  Validated arguments only.
size_t bwd_group_bytes(const kda_bwd_args *a, int first, int last) {
    const int32_t *cu = a->cu_seqlens_host;
    int64_t ck = 0, ch = 0;
    for (int n = first; n < last; ++n) {
        ck += (cu[n + 1] - cu[n]) / 32;
        ch += (cu[n + 1] - cu[n] + 31) / 32;
    }
    const size_t body = kda_bwd_workspace_layout(last - first, a->num_heads, cu[last] - cu[first], a->dk, a->dv, ck,
                                                 ch, bwd_flags(a), nullptr);
    return (body + 255) / 256 * 256 + ((size_t)(last - first + 1) * 4 + 255) / 256 * 256;
}

// ---- scratch of the allocation-free forward ------------------------------------------------
// kda_chunk_fwd_noalloc keeps its launch plan (sequence order, int32 [N] padded to 256 B, then
// per-sequence checkpoint bases, int64 [N] padded to 256 B, then 256 B) in this file-scope
// device array instead of a caller workspace.  Each GPU holds its own copy until the process
// ends.  In host code the name `scratch` is not a device address: the address on the current
// device is looked up once per device with hipGetSymbolAddress and only that pointer is used.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)KDA_NOALLOC_MAX_SEQS * 4 + (size_t)KDA_NOALLOC_MAX_SEQS * 8 + 256;
static_assert(KDA_NOALLOC_MAX_SEQS % 64 == 0, "both plan arrays stay multiples of 256 bytes");
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];   // per device, resolved on the first call with that device current

hipError_t scratch_on_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
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
    size_t off[7];
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
    int nb = 0;
    int64_t nck = 0;
    const int seg = segment_plan(a, &nb, &nck);
    if (seg > 0) {
        const hipError_t e = kda_launch_chunk_segmented(
            a->dk, in_bf16, a->num_seqs, a->num_heads, a->total_tokens, seg, nb, nck, q, k, v, g, beta,
            a->cu_seqlens, a->initial_state,
            a->final_state, a->checkpoint_every, a->checkpoints, a->o, a->scale, a->initial_state_indices,
            a->checkpoint_indices, a->num_slots, flags, static_cast<char *>(workspace) + off[5], s);
        return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
    }
    const hipError_t e = kda_launch_chunk(a->chunk_size, a->dk, in_bf16, a->num_seqs, a->num_heads, q, k, v, g, beta,
                                          a->cu_seqlens, a->initial_state, a->final_state, a->checkpoint_every,
                                          a->checkpoints, a->o, a->scale, a->initial_state_indices,
                                          a->checkpoint_indices, a->num_slots, flags, workspace, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status kda_chunk_fwd_noalloc(const kda_fwd_args *a, void *stream) {
    const kda_status st = validate_fwd(a);
    if (st != KDA_OK) return st;
    if (a->num_seqs > KDA_NOALLOC_MAX_SEQS) return KDA_ERR_WORKSPACE_TOO_SMALL;
    // the launch plan is the only scratch: the prologue's outputs (not fused at this shape) would
    // need caller memory
    if (fwd_flags(a) != 0 && !(a->chunk_size == 32 && a->dk == 128)) return KDA_ERR_UNSUPPORTED;
    if (a->segment_tokens > 0) return KDA_ERR_UNSUPPORTED;   // the segments' states need a workspace
    if (a->num_seqs == 0) return KDA_OK;
    if (kda_chunk_workspace_layout(a->num_seqs, nullptr, nullptr) > NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess) return KDA_ERR_DEVICE;
    const hipError_t e = kda_launch_chunk(a->chunk_size, a->dk, a->in_dtype == KDA_BF16, a->num_seqs, a->num_heads, a->q,
                                          a->k, a->v, a->g, a->beta, a->cu_seqlens, a->initial_state, a->final_state,
                                          a->checkpoint_every, a->checkpoints, a->o, a->scale,
                                          a->initial_state_indices, a->checkpoint_indices, a->num_slots, fwd_flags(a),
                                          ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

size_t kda_chunk_bwd_workspace_bytes(const kda_bwd_args *a) {
    int64_t ck, ch;
    if (validate_bwd(a, &ck, &ch) != KDA_OK) return 0;
    return kda_bwd_workspace_layout(a->num_seqs, a->num_heads, a->total_tokens, a->dk, a->dv, ck, ch, bwd_flags(a),
                                    nullptr);
}

size_t kda_chunk_bwd_workspace_min_bytes(const kda_bwd_args *a) {
    int64_t ck, ch;
    if (validate_bwd(a, &ck, &ch) != KDA_OK) return 0;
    const size_t full = kda_bwd_workspace_layout(a->num_seqs, a->num_heads, a->total_tokens, a->dk, a->dv, ck, ch,
                                                 bwd_flags(a), nullptr);
    size_t least = 0;
    for (int n = 0; n < a->num_seqs; ++n) {
        const size_t need = bwd_group_bytes(a, n, n + 1);
        least = need > least ? need : least;
    }
    return least < full ? least : full;
}

kda_status kda_chunk_bwd(const kda_bwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    int64_t ck = 0, ch = 0;
    const kda_status st = validate_bwd(a, &ck, &ch);
    if (st != KDA_OK) return st;
    if (a->num_seqs == 0) return KDA_OK;
    const size_t need = kda_bwd_workspace_layout(a->num_seqs, a->num_heads, a->total_tokens, a->dk, a->dv, ck, ch,
                                                 bwd_flags(a), nullptr);
    if (!workspace) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_INVALID_ARGUMENT;
    const hipStream_t sm = static_cast<hipStream_t>(stream);
    if (workspace_bytes >= need) {
        const hipError_t e = kda_launch_bwd(a->dk, a->in_dtype == KDA_BF16, a->num_seqs, a->num_heads,
                                            a->total_tokens, ck, ch, a->q, a->k, a->v, a->g, a->beta, a->cu_seqlens,
                                            a->initial_state, a->d_o, a->d_final_state, a->dq, a->dk_out, a->dv_out,
                                            a->dg, a->dbeta, a->d_initial_state, a->scale, a->states,
                                            (bwd_flags(a) & 3) | bwd_scan_choice(a->cu_seqlens_host, 0, a->num_seqs,
                                                                                 a->num_heads),
                                            workspace, sm);
        return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
    }
    // A smaller workspace: consecutive groups of whole sequences, each within it, one after the
    // other on the stream (the sequences are independent; each group is the same computation).
    const int N = a->num_seqs;
    for (int n = 0; n < N; ++n)
        if (bwd_group_bytes(a, n, n + 1) > workspace_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
    const int32_t *cu = a->cu_seqlens_host;
    const int H = a->num_heads, dk = a->dk, dv = a->dv;
    const size_t in_es = a->in_dtype == KDA_BF16 ? 2 : 4;
    const size_t g_es = a->gate_mode == KDA_GATE_PREACTIVATION ? 2 : 4;   // bf16 pre-activations a
    const size_t state = (size_t)H * dk * dv;
    auto shift = [](const void *p, size_t bytes) -> const void * {
        return p ? static_cast<const char *>(p) + bytes : nullptr;
    };
    auto shiftf = [](float *p, size_t elems) { return p ? p + elems : nullptr; };
    int64_t ck_before = 0;
    for (int first = 0; first < N;) {
        int last = first + 1;
        while (last < N && bwd_group_bytes(a, first, last + 1) <= workspace_bytes) ++last;
        const int Ng = last - first;
        const size_t t0 = (size_t)cu[first];
        const int Tg = cu[last] - cu[first];
        int64_t ckg = 0, chg = 0;
        for (int n = first; n < last; ++n) {
            ckg += (cu[n + 1] - cu[n]) / 32;
            chg += (cu[n + 1] - cu[n] + 31) / 32;
        }
        const size_t body = kda_bwd_workspace_layout(Ng, H, Tg, dk, dv, ckg, chg, bwd_flags(a), nullptr);
        int32_t *cu_g = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + (body + 255) / 256 * 256);
        hipError_t e = kda_launch_cu_rebase(a->cu_seqlens, first, Ng, cu_g, sm);
        if (e == hipSuccess)
            e = kda_launch_bwd(dk, a->in_dtype == KDA_BF16, Ng, H, Tg, ckg, chg, shift(a->q, t0 * H * dk * in_es),
                               shift(a->k, t0 * H * dk * in_es), shift(a->v, t0 * H * dv * in_es),
                               static_cast<const float *>(shift(a->g, t0 * H * dk * g_es)),
                               static_cast<const float *>(shift(a->beta, t0 * H * 4)), cu_g,
                               static_cast<const float *>(shift(a->initial_state, first * state * 4)),
                               static_cast<const float *>(shift(a->d_o, t0 * H * dv * 4)),
                               static_cast<const float *>(shift(a->d_final_state, first * state * 4)),
                               shiftf(a->dq, t0 * H * dk), shiftf(a->dk_out, t0 * H * dk), shiftf(a->dv_out, t0 * H * dv),
                               shiftf(a->dg, t0 * H * dk), shiftf(a->dbeta, t0 * H),
                               shiftf(a->d_initial_state, first * state), a->scale,
                               static_cast<const float *>(shift(a->states, (size_t)ck_before * state * 4)),
                               (bwd_flags(a) & 3) | bwd_scan_choice(cu, first, last, H), workspace, sm);
        if (e != hipSuccess) return KDA_ERR_DEVICE;
        ck_before += ckg;
        first = last;
    }
    return KDA_OK;
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

// ---- the side stream (kda_side.h) ----------------------------------------------------------
namespace {
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];
SideStream *g_side_cur = nullptr;   // between kda_side_fork and kda_side_forked (lock held)

// (with g_side_mu held) the current device's side stream; null when it cannot be had
SideStream *side_stream() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    SideStream &ss = g_side[dev];
    if (!ss.s) {
        hipStream_t st = nullptr;
        hipEvent_t a = nullptr, b = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            (void)hipStreamDestroy(st);
            return nullptr;
        }
        ss.s = st; ss.fork = a; ss.join = b;
    }
    return &ss;
}
}  // namespace

extern "C" __attribute__((visibility("hidden"))) hipStream_t kda_side_fork(hipStream_t s) {
    g_side_mu.lock();
    SideStream *ss = side_stream();
    if (!ss || hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess) {
        g_side_mu.unlock();
        return nullptr;
    }
    g_side_cur = ss;
    return ss->s;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_side_forked(void) {
    SideStream *ss = g_side_cur;
    g_side_cur = nullptr;
    const hipError_t e = ss ? hipEventRecord(ss->join, ss->s) : hipErrorInvalidValue;
    g_side_mu.unlock();
    return e;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t kda_side_join(hipStream_t s) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream *ss = side_stream();
    return ss ? hipStreamWaitEvent(s, ss->join, 0) : hipErrorInvalidValue;
}
