/*
 * kda.h -- C ABI of libkda, an MI355X (gfx950) implementation of the Kimi
 * Delta Attention (KDA) operator: a gated delta-rule linear attention with a
 * per-channel forget gate.
 *
 * The operator (per sequence n, per head h, tokens t in order; S is d_k x d_v,
 * fp32, row-major, one per (sequence, head)):
 *
 *     S   <- Diag(exp(g_t)) S                      per-channel forget gate
 *     u_t  = beta_t * (v_t - S^T k_t)              delta-rule residual
 *     S   <- S + k_t u_t^T                         targeted overwrite
 *     o_t  = scale * S^T q_t                       read-out after the write
 *
 * i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 * alpha_t = exp(g_t).  Sources (pages on the Kimi K3 technical report):
 *   - "Attention->K3 30-day course, Day 21", quiz Q9 (the delta rule: the old
 *     memory predicts v_t and only the residual is written back), Q8 and
 *     interview answer D19 (fixed d x d state formed as K^T V, per-channel
 *     decay gate), D17 and Q5 (decode is memory-bound);
 *   - skillsmp "kimi-k3-tech-report" skill card, quick facts: the log-decay is
 *     a lower-bounded scaled sigmoid with g_min = -5, which lets the diagonal
 *     tiles of the chunked form run as dense matrix-core products;
 *   - t.iss.one digest of the report: a fixed-size recurrent state per KDA
 *     layer, and prefix reuse at 512-token boundaries (the checkpoints below).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - Layouts are token-major with heads interleaved and contiguous:
 *       q, k, g : [tokens, H, d_k]   v, o : [tokens, H, d_v]   beta : [tokens, H]
 *       states  : [sequences, H, d_k, d_v]  (row-major d_k x d_v per head)
 *   - g is the natural-log decay.  Results are defined for g in [-5, 0] (the
 *     range of -5*sigmoid(x)); values below -5 may overflow the in-chunk
 *     factorisation.  Inputs must be finite.  Neither is checked.
 *   - The caller owns every buffer, including the workspace; the library never
 *     allocates device memory (kda_chunk_fwd_noalloc uses a static device array
 *     of the library instead of a workspace).  All work is enqueued asynchronously
 *     on `stream` (a hipStream_t passed as void*; NULL = the default stream).
 *   - Errors are returned synchronously as kda_status.  Argument validation is
 *     pure host code and runs before any launch; a failed launch returns
 *     KDA_ERR_DEVICE.  Faults during execution surface at the caller's next
 *     synchronisation.
 *   - A call only enqueues kernels (no allocation, copy or memset), so calls
 *     may be captured into a HIP graph.  Calls from several host threads are
 *     safe; the library's only global state is a per-device compute-unit
 *     count read once, and the per-device address of kda_chunk_fwd_noalloc's
 *     array.  Calls that share a workspace or an output must be ordered by the
 *     caller (same stream, or events).
 *   - Supported: d_k == d_v in {64, 128}; chunk_size 32 or 64; in_dtype
 *     KDA_F32 or KDA_BF16.  Other values -> KDA_ERR_UNSUPPORTED.
 *   - Paged state pool (ABI v2; the digest's inference paragraph: a pool of
 *     recurrent states with prefix reuse at 512-token boundaries): a pool is
 *     fp32 [num_slots, H, d_k, d_v]; an index array maps each sequence (or
 *     checkpoint) to a slot.  Index -1 means "no slot"; an index outside
 *     [-1, num_slots) is treated as -1.  The kernels check the range; the
 *     caller guarantees that the slots written in one call are distinct and
 *     are not also read in that call.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7u

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,
    KDA_ERR_UNSUPPORTED = 2,
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_DEVICE = 4
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* What kda_fwd_args.g and .beta hold. */
typedef enum {
    KDA_GATE_LOG_DECAY = 0,      /* g: fp32 log-decay [T,H,dk]; beta: fp32 [T,H] */
    KDA_GATE_PREACTIVATION = 1   /* g: bf16 pre-activations a [T,H,dk] (raw 16-bit words); beta: fp32
                                    pre-activations b [T,H]; the operator uses g = -5*sigmoid(a) and
                                    beta = sigmoid(b) (skill card quick facts: lower-bounded scaled
                                    sigmoid, g_min = -5) */
} kda_gate_mode;

/*
 * Chunked prefill over packed variable-length sequences.
 *
 * Sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]) of the packed token
 * axis.  Each sequence is cut into chunks of `chunk_size` tokens aligned to its
 * own start (the last may be partial; no chunk spans two sequences) and
 * starts from its own initial state.
 *
 * Fields:
 *   struct_size      sizeof(kda_fwd_args) as compiled by the caller.
 *   num_seqs         N >= 0.  total_tokens: T >= 0, must equal cu_seqlens[N].
 *   num_heads        H >= 1.   dk, dv: head dims.
 *   chunk_size       32 or 64: the token block of the chunked form.  32 runs the
 *                    software-pipelined kernel (the fast path); 64 runs a simpler
 *                    one-phase-at-a-time kernel.  Both compute the same operator
 *                    (results differ by rounding only).
 *   in_dtype         element type of q, k, v (bf16 = raw 16-bit bf16 words).
 *   scale            multiplies every output (o = scale * S^T q).
 *   q, k, v, g, beta see layouts above; 16-byte aligned.
 *   cu_seqlens       device int32 [N+1]; cu_seqlens_host: a host copy of the
 *                    same values (validation and launch sizing without a device
 *                    read).  The library does not check that they agree.
 *   initial_state    NULL => zeros; else fp32 [N, H, dk, dv].
 *   final_state      NULL => not written; else fp32 [N, H, dk, dv].  May alias
 *                    initial_state (each (n,h) slice is read before it is written).
 *   checkpoint_every 0 => none; else a positive multiple of chunk_size.  The state
 *                    after in-sequence positions every*m, m = 1..floor(L_n/every),
 *                    is written to `checkpoints`.
 *   checkpoints      fp32 [sum_n floor(L_n/every), H, dk, dv], sequence-major then
 *                    position.  Required iff checkpoint_every > 0.
 *   o                fp32 [T, H, dv]; must not alias any input.
 *   initial_state_indices  NULL => initial_state as above.  Else device int32 [N]:
 *                    initial_state is a pool of num_slots states and sequence n
 *                    starts from slot initial_state_indices[n] (-1: zeros).
 *   checkpoint_indices     NULL => checkpoints as above.  Else device int32
 *                    [sum_n floor(L_n/every)] (checkpoint m in the order above):
 *                    checkpoints is a pool of num_slots states and checkpoint m is
 *                    written to slot checkpoint_indices[m] (-1: not written).
 *   num_slots        >= 1 when either index array is set; else ignored.
 *                    final_state stays [N, H, dk, dv] either way.
 *   gate_mode        kda_gate_mode: KDA_GATE_PREACTIVATION fuses the gate
 *                    (g = -5 sigmoid(a), beta = sigmoid(b)) into the first stage, halving
 *                    the bytes of g.
 *   normalize_qk     1: q and k are L2-normalised per (token, head) over dk inside the
 *                    operator (a zero vector stays zero); `scale` still applies.  0: used
 *                    as given.
 *                    Either prologue needs bf16 inputs (else KDA_ERR_UNSUPPORTED).  With
 *                    chunk_size 32 and dk = 128 it is fused into the kernel's first stage;
 *                    otherwise it runs as a pass of its own whose outputs the workspace
 *                    holds (fp32 q / |q|, k / |k| and v with the normalisation, the rest
 *                    of the forward then computing on fp32 inputs; fp32 g and beta with
 *                    the gate), and kda_chunk_fwd_workspace_bytes includes them.
 *   segment_tokens   Context parallelism inside the GPU (chunk_size 32 only).  Over a stretch
 *                    of tokens the state is an affine function of the state it starts from,
 *                    S_t = M_t S_in + N_t, and so o_t = o0_t + S_in^T (scale M_t^T q_t) (the
 *                    t.iss.one DNSPODT digest of the K3 report, infrastructure paragraph: KDA's
 *                    context parallelism exchanges only the fixed-size state).  Each sequence
 *                    is cut into segments of segment_tokens tokens (from its start; the last
 *                    may be shorter) that run side by side: every segment from zero and, but a
 *                    sequence's first (which starts from its initial state), also from the
 *                    identity with v = 0; a short pass along each sequence then chains the
 *                    maps into every segment's initial state (and the final state, and
 *                    corrects the checkpoints), and a last pass adds S_in^T (scale M_t^T q_t)
 *                    to the later segments' outputs.  About twice the arithmetic, spread over
 *                    many more compute units: it pays for few, long sequences on few heads.
 *                    Results equal the uncut forward up to rounding.
 *                    0: the library decides (it cuts only when the (sequence, head) pairs
 *                    leave most compute units idle and the longest sequence spans at least
 *                    three segments).  -1: never cut.  > 0: cut at this length, a multiple
 *                    of 32 and of checkpoint_every (else KDA_ERR_INVALID_ARGUMENT); chunk_size
 *                    64 then gives KDA_ERR_UNSUPPORTED.  When cut, the workspace grows by
 *                    12 d_k d_v bytes per (segment, head), 4 d_k bytes per (token, head) and
 *                    4 d_k d_v bytes per (checkpoint, head).
 */
typedef struct {
    uint32_t struct_size;
    int32_t num_seqs;
    int32_t total_tokens;
    int32_t num_heads;
    int32_t dk;
    int32_t dv;
    int32_t chunk_size;
    kda_dtype in_dtype;
    float scale;
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *beta;
    const int32_t *cu_seqlens;
    const int32_t *cu_seqlens_host;
    const float *initial_state;
    float *final_state;
    int32_t checkpoint_every;
    float *checkpoints;
    float *o;
    const int32_t *initial_state_indices;
    const int32_t *checkpoint_indices;
    int32_t num_slots;
    int32_t gate_mode;
    int32_t normalize_qk;
    int32_t segment_tokens;
} kda_fwd_args;

/* Device workspace (bytes) that kda_chunk_fwd needs for `args` (host only; no
 * device access).  Returns 0 when args are invalid. */
size_t kda_chunk_fwd_workspace_bytes(const kda_fwd_args *args);

/* Enqueue the chunked forward.  `workspace` must hold at least
 * kda_chunk_fwd_workspace_bytes(args) bytes of device memory, 256-byte aligned;
 * it is scratch for the launch plan and is overwritten. */
kda_status kda_chunk_fwd(const kda_fwd_args *args, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same operator, arguments and
 * results as kda_chunk_fwd, with no workspace.  Its launch plan lives in a static device
 * array inside the library (768 KiB per GPU, held until the process ends); the call allocates
 * nothing and enqueues the same kernels on `stream`.
 *   - At most KDA_NOALLOC_MAX_SEQS sequences, else KDA_ERR_WORKSPACE_TOO_SMALL.
 *   - A prologue (gate_mode / normalize_qk) only where it is fused into the kernel (chunk_size
 *     32 and dk 128), else KDA_ERR_UNSUPPORTED: elsewhere its outputs would need a workspace.
 *   - Sequences are never cut into segments (segment_tokens 0 and -1 both run uncut; > 0
 *     gives KDA_ERR_UNSUPPORTED): the segments' states would need a workspace.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (different
 *     streams, no ordering between them) race.  Order them on one stream or with events.
 *   - The first call on a device looks the array's address up (no allocation); make that first
 *     call outside a graph capture.
 */
#define KDA_NOALLOC_MAX_SEQS 65536
kda_status kda_chunk_fwd_noalloc(const kda_fwd_args *args, void *stream);

/*
 * One decode step: for each of N independent sequences and each head, consume
 * one token and update that (sequence, head) state in place.
 *   q, k, g : [N, H, dk]    v : [N, H, dv]    beta : [N, H]
 *   state   : fp32 [N, H, dk, dv], read and overwritten in place; or, when
 *             state_indices is set, a pool fp32 [num_slots, H, dk, dv] in which
 *             sequence n uses slot state_indices[n] (device int32 [N]).  A
 *             sequence with slot -1 is inactive: its state is not touched and
 *             its o is 0.  Active slots must be distinct.
 *   o       : fp32 [N, H, dv]
 *   num_slots >= 1 when state_indices is set; else ignored.
 *   gate_mode, normalize_qk: the prologue, as in kda_fwd_args (g then holds the bf16
 *             pre-activations a and beta the fp32 pre-activations b; q and k are
 *             normalised over dk inside); either needs bf16 inputs (else
 *             KDA_ERR_UNSUPPORTED).
 */
typedef struct {
    uint32_t struct_size;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t dk;
    int32_t dv;
    kda_dtype in_dtype;
    float scale;
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *beta;
    float *state;
    const int32_t *state_indices;
    float *o;
    int32_t num_slots;
    int32_t gate_mode;
    int32_t normalize_qk;
} kda_decode_args;

kda_status kda_decode_step(const kda_decode_args *args, void *stream);

/*
 * Backward of the chunked prefill (the scripod shownote of the K3 report
 * reading lists a KDA kernel under pre-training, section 5.1.1; training needs
 * the operator's gradients): for the scalar
 *
 *     L = sum(d_o * o) + sum(d_final_state * final_state)
 *
 * of the forward over the same inputs (dense initial states, no pool; the fused
 * prologue is optional, see gate_mode and normalize_qk below), write dL/dq,
 * dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS_0.  Per token,
 * walking each sequence backwards with dS = dL/dS_t, the adjoint of the
 * recurrence is
 *     dS += scale q_t d_o_t^T;  dq_t = scale S_t d_o_t;  du = dS^T k_t;
 *     dv_t = beta_t du;  dbeta_t = <du, v_t - p_t>;  dp = -beta_t du;
 *     dk_t = dS u_t + St~ dp;  dg_t = alpha_t * rowsum((dS + k_t dp^T) * S_{t-1});
 *     dS <- Diag(alpha_t) (dS + k_t dp^T)
 * with St~ = Diag(alpha_t) S_{t-1}, p_t = St~^T k_t, u_t = beta_t (v_t - p_t).
 * The library evaluates it chunk by chunk (32 tokens): it recomputes the states
 * at chunk boundaries with the forward, runs the state gradient backwards over
 * the chunks, then forms every chunk's gradients in parallel.
 *
 * Fields (layouts, sizes and alignment as for kda_fwd_args):
 *   struct_size, num_seqs, total_tokens, num_heads, dk, dv, in_dtype, scale,
 *   q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state
 *                    as in kda_fwd_args (initial_state NULL => zeros).
 *   d_o              fp32 [T, H, dv]: dL/do.
 *   d_final_state    NULL => zeros; else fp32 [N, H, dk, dv].
 *   dq, dk_out, dg   fp32 [T, H, dk];  dv_out fp32 [T, H, dv];  dbeta fp32 [T, H].
 *                    Written in full; none may alias another buffer of the call.
 *   d_initial_state  NULL => not written; else fp32 [N, H, dk, dv].
 *   gate_mode        as in kda_fwd_args.  KDA_GATE_PREACTIVATION: g holds the bf16
 *                    pre-activations a (raw 16-bit words) and beta the fp32 pre-activations
 *                    b; dg and dbeta are then dL/da and dL/db (through g = -5 sigmoid(a),
 *                    beta = sigmoid(b)).
 *   states           NULL: the states at every 32-token boundary are recomputed (into the
 *                    workspace).  Else fp32 [sum_n floor(L_n / 32), H, dk, dv]: exactly the
 *                    checkpoints kda_chunk_fwd writes for the same inputs and prologue with
 *                    checkpoint_every = 32, read instead of recomputed (the workspace is then
 *                    smaller by their size).  16-byte aligned; no output may alias it.
 *   normalize_qk     as in kda_fwd_args: 1 normalises q and k inside; dq and dk are then
 *                    the gradients with respect to the raw q and k (zero for a zero row).
 *                    Either prologue needs bf16 inputs (else KDA_ERR_UNSUPPORTED); unlike
 *                    the forward's, it is supported at d_k = 64 and 128.  The
 *                    prologue's outputs are materialised in the workspace: q / |q|, k / |k|
 *                    and v in fp32 (3 * T*H*dk*4 bytes; the unit vectors are not rounded to
 *                    bf16, as in the forward) and g, beta in fp32 (T*H*(dk + 1)*4 bytes).
 * Supported: d_k == d_v in {64, 128}; in_dtype KDA_F32 or KDA_BF16.  The
 * workspace (kda_chunk_bwd_workspace_bytes) holds the recomputed states, the
 * state gradients at every chunk boundary and per-chunk factors: about
 * (3 dk dv + 32 (2 dk + dv) + dk + 2 * 32^2) * 4 bytes per (32-token chunk,
 * head).  Results are fp32 and deterministic.
 */
typedef struct {
    uint32_t struct_size;
    int32_t num_seqs;
    int32_t total_tokens;
    int32_t num_heads;
    int32_t dk;
    int32_t dv;
    kda_dtype in_dtype;
    float scale;
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *beta;
    const int32_t *cu_seqlens;
    const int32_t *cu_seqlens_host;
    const float *initial_state;
    const float *d_o;
    const float *d_final_state;
    float *dq;
    float *dk_out;
    float *dv_out;
    float *dg;
    float *dbeta;
    float *d_initial_state;
    int32_t gate_mode;
    int32_t normalize_qk;
    const float *states;
} kda_bwd_args;

/* Device workspace (bytes) with which kda_chunk_bwd runs the whole batch at once (host only).
 * Returns 0 when args are invalid. */
size_t kda_chunk_bwd_workspace_bytes(const kda_bwd_args *args);

/* The least workspace kda_chunk_bwd accepts (host only): that of the batch's longest single
 * sequence run alone (at most kda_chunk_bwd_workspace_bytes).  Returns 0 when args are invalid. */
size_t kda_chunk_bwd_workspace_min_bytes(const kda_bwd_args *args);

/* Enqueue the backward.  `workspace`: device memory, 256-byte aligned, overwritten, of
 * workspace_bytes >= kda_chunk_bwd_workspace_min_bytes(args) (else
 * KDA_ERR_WORKSPACE_TOO_SMALL).  With less than kda_chunk_bwd_workspace_bytes(args) the batch
 * runs as consecutive groups of whole sequences, each group the most that fits, one after
 * the other on `stream` (the sequences are independent; each group performs the same
 * computation, so results differ from the one-pass run only where the forward recompute
 * chooses another split of its work: by rounding).  This bounds the memory of a large batch
 * (the workspace of a whole batch grows with its tokens times heads). */
kda_status kda_chunk_bwd(const kda_bwd_args *args, void *workspace, size_t workspace_bytes, void *stream);

/* Static string for a status code. */
const char *kda_status_str(kda_status status);

/* KDA_ABI_VERSION of the library. */
uint32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
