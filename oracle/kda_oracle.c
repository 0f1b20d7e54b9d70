/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for the Kimi Delta Attention
 * (KDA) recurrence, in IEEE fp64.  Only the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library; the product
 * path (libkda.so and its Python binding) never does, and shares no code,
 * header, table or helper with it.
 *
 * What is computed (per sequence n, per head h, tokens in order):
 *
 *     S <- Diag(exp(g_t)) S                 per-channel forget gate, applied first
 *     p  = S^T k_t                          the memory's prediction for k_t
 *     u  = beta_t (v_t - p)                 delta-rule residual
 *     S <- S + k_t u^T                      targeted overwrite with the residual
 *     o_t = scale * S^T q_t                 read-out from the post-update state
 *
 * which is the same map as S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 * + beta_t k_t v_t^T, o_t = S_t^T q_t with alpha_t = exp(g_t).
 *
 * Sources (pages on the Kimi K3 technical report):
 *   - "Attention->K3 30-day course, Day 21", section 5, quiz Q9: before the
 *     write, the old memory predicts the current value and only the residual
 *     between v_t and that prediction is written back (the delta rule).
 *   - same page, interview answer D19 and quiz Q8: a fixed-size d x d state
 *     formed as K^T V, with a per-channel decay gate.
 *   - skillsmp "kimi-k3-tech-report" skill card, quick-facts list: per-channel
 *     forget gate whose log-decay is a lower-bounded scaled sigmoid, g_min=-5.
 *   The explicit operator order (decay, then predict from the decayed state,
 *   then write; read-out after the write) is the equation the build targets;
 *   the pages state the rule only in words.
 *
 * Inputs arrive as fp32 arrays: that is exactly the set of values the GPU
 * receives (bf16 inputs are widened to fp32 without rounding), and each value
 * is converted to fp64 before any arithmetic.
 *
 * Layouts (row-major, token-major, heads interleaved):
 *   q, k, g : [T_total, H, dk]     v : [T_total, H, dv]     beta : [T_total, H]
 *   S0, S_final : [N, H, dk, dv]   o : [T_total, H, dv]
 *   checkpoints : [sum_n floor(L_n / every), H, dk, dv], sequence-major, then
 *                 position; entry m of sequence n is the state after in-sequence
 *                 position every*(m+1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_seqs, num_heads, dk, dv;
    const int64_t *cu_seqlens; /* [num_seqs + 1] */
    const float *q, *k, *v, *g, *beta;
    double scale;
    const float *S0;        /* NULL => zero initial state */
    double *o;              /* [T_total, H, dv] */
    double *S_final;        /* NULL => not written */
    int32_t ckpt_every;     /* 0 => no checkpoints */
    double *ckpt;           /* see header */
    int32_t n_threads;
} oracle_fwd_args;

/* One (sequence, head) chain of the recurrence.  S is dk*dv doubles. */
static void run_chain(const oracle_fwd_args *a, int n, int h, double *S,
                      double *alpha, double *p, double *u, int64_t ckpt_base) {
    const int H = a->num_heads, dk = a->dk, dv = a->dv;
    const int64_t start = a->cu_seqlens[n], end = a->cu_seqlens[n + 1];

    if (a->S0) {
        const float *src = a->S0 + ((int64_t)n * H + h) * dk * dv;
        for (int i = 0; i < dk * dv; ++i) S[i] = (double)src[i];
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }

    for (int64_t t = start; t < end; ++t) {
        const float *qt = a->q + (t * H + h) * dk;
        const float *kt = a->k + (t * H + h) * dk;
        const float *vt = a->v + (t * H + h) * dv;
        const float *gt = a->g + (t * H + h) * dk;
        const double bt = (double)a->beta[t * H + h];

        /* forget gate: S <- Diag(exp(g_t)) S */
        for (int i = 0; i < dk; ++i) alpha[i] = exp((double)gt[i]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[i * dv + j] *= alpha[i];

        /* prediction p = S^T k_t from the decayed state */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int j = 0; j < dv; ++j) p[j] += S[i * dv + j] * ki;
        }

        /* residual u = beta (v - p); write S <- S + k u^T */
        for (int j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int j = 0; j < dv; ++j) S[i * dv + j] += ki * u[j];
        }

        /* read-out from the post-update state: o_t = scale * S^T q_t */
        double *ot = a->o + (t * H + h) * dv;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = (double)qt[i];
            for (int j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qi;
        }
        for (int j = 0; j < dv; ++j) ot[j] *= a->scale;

        /* state snapshot after every `ckpt_every` tokens of this sequence */
        const int64_t pos = t - start + 1;
        if (a->ckpt_every > 0 && a->ckpt && pos % a->ckpt_every == 0) {
            const int64_t m = ckpt_base + pos / a->ckpt_every - 1;
            memcpy(a->ckpt + (m * H + h) * (int64_t)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        }
    }

    if (a->S_final)
        memcpy(a->S_final + ((int64_t)n * H + h) * (int64_t)dk * dv, S, sizeof(double) * (size_t)dk * dv);
}

/* ---- a small thread pool over (sequence, head) chains, longest first ---- */
typedef struct {
    const oracle_fwd_args *a;
    const int32_t *order;      /* chain ids, longest sequence first */
    const int64_t *ckpt_base;  /* per sequence */
    int32_t n_chains;
    int32_t next;
    pthread_mutex_t lock;
} pool_t;

static void *worker(void *arg) {
    pool_t *P = (pool_t *)arg;
    const oracle_fwd_args *a = P->a;
    double *S = (double *)malloc(sizeof(double) * (size_t)a->dk * a->dv);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)a->dk);
    double *p = (double *)malloc(sizeof(double) * (size_t)a->dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)a->dv);
    for (;;) {
        pthread_mutex_lock(&P->lock);
        const int32_t c = P->next < P->n_chains ? P->order[P->next++] : -1;
        pthread_mutex_unlock(&P->lock);
        if (c < 0) break;
        const int n = c / a->num_heads, h = c % a->num_heads;
        run_chain(a, n, h, S, alpha, p, u, P->ckpt_base[n]);
    }
    free(S); free(alpha); free(p); free(u);
    return NULL;
}

static const int64_t *g_len_for_sort;
static int32_t g_heads_for_sort;
static int cmp_longest_first(const void *x, const void *y) {
    const int32_t cx = *(const int32_t *)x, cy = *(const int32_t *)y;
    const int64_t lx = g_len_for_sort[cx / g_heads_for_sort], ly = g_len_for_sort[cy / g_heads_for_sort];
    if (lx != ly) return lx > ly ? -1 : 1;
    return cx < cy ? -1 : (cx > cy);
}

/* Returns 0 on success, -1 on bad arguments / allocation failure. */
int oracle_kda_forward(const oracle_fwd_args *a) {
    if (!a || a->num_seqs < 0 || a->num_heads <= 0 || a->dk <= 0 || a->dv <= 0) return -1;
    const int N = a->num_seqs, H = a->num_heads;
    int64_t *len = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
    int64_t *base = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * H + 1));
    if (!len || !base || !order) { free(len); free(base); free(order); return -1; }
    int64_t acc = 0;
    for (int n = 0; n < N; ++n) {
        len[n] = a->cu_seqlens[n + 1] - a->cu_seqlens[n];
        base[n] = acc;
        if (a->ckpt_every > 0) acc += len[n] / a->ckpt_every;
    }
    for (int c = 0; c < N * H; ++c) order[c] = c;
    g_len_for_sort = len; g_heads_for_sort = H;
    qsort(order, (size_t)N * H, sizeof(int32_t), cmp_longest_first);

    pool_t P;
    P.a = a; P.order = order; P.ckpt_base = base; P.n_chains = N * H; P.next = 0;
    pthread_mutex_init(&P.lock, NULL);
    int nt = a->n_threads > 0 ? a->n_threads : 1;
    if (nt > N * H) nt = N * H > 0 ? N * H : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, worker, &P);
    for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&P.lock);
    free(th); free(len); free(base); free(order);
    return 0;
}

/*
 * One decode step for N independent (sequence, head) states: the loop body
 * above with a single token, applied to a state given in fp32.
 *   q, k, g : [N, H, dk]   v : [N, H, dv]   beta : [N, H]
 *   S_in : [N, H, dk, dv] fp32     S_out : [N, H, dk, dv] fp64     o : [N, H, dv]
 */
int oracle_kda_decode(int32_t N, int32_t H, int32_t dk, int32_t dv, const float *q, const float *k,
                      const float *v, const float *g, const float *beta, double scale,
                      const float *S_in, double *S_out, double *o, int32_t n_threads) {
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    int64_t *cu = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
    if (!cu) return -1;
    for (int n = 0; n <= N; ++n) cu[n] = n;
    oracle_fwd_args a;
    memset(&a, 0, sizeof a);
    a.num_seqs = N; a.num_heads = H; a.dk = dk; a.dv = dv; a.cu_seqlens = cu;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.scale = scale;
    a.S0 = S_in; a.o = o; a.S_final = S_out; a.ckpt_every = 0; a.ckpt = NULL;
    a.n_threads = n_threads;
    const int rc = oracle_kda_forward(&a);
    free(cu);
    return rc;
}
