/* Host harness of libkda's C ABI for the sanitizer test (tests/test_host_sanitized.py): every
 * entry point is called with valid and invalid arguments built from fake device pointers and
 * exactly-sized host arrays (so that AddressSanitizer sees any read past them), including ragged
 * and empty sequences and a 3000-sequence batch.  With no GPU visible, a call that passes
 * validation fails at its first launch (KDA_ERR_DEVICE); the harness checks every status
 * against the expected one.  It refuses to run when a GPU is visible: its pointers are fake. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

static int failures = 0;
static void expect(const char *what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d (%s), expected %d (%s)\n", what, got, kda_status_str((kda_status)got), want,
                kda_status_str((kda_status)want));
        ++failures;
    }
}
#define FAKE(i) ((void *)(uintptr_t)(0x100000ull * (i)))

static int32_t *cu_from(const int *lens, int n) {   /* exactly n + 1 entries, on the heap */
    int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n + 1));
    cu[0] = 0;
    for (int i = 0; i < n; ++i) cu[i + 1] = cu[i] + lens[i];
    return cu;
}

static kda_fwd_args fwd(const int32_t *cu, int n, int dk, int chunk, kda_dtype dt) {
    kda_fwd_args a;
    memset(&a, 0, sizeof a);
    a.struct_size = sizeof a;
    a.num_seqs = n;
    a.total_tokens = cu[n];
    a.num_heads = 3;
    a.dk = a.dv = dk;
    a.chunk_size = chunk;
    a.in_dtype = dt;
    a.scale = 1.0f;
    a.q = FAKE(1); a.k = FAKE(2); a.v = FAKE(3); a.g = (const float *)FAKE(4); a.beta = (const float *)FAKE(5);
    a.o = (float *)FAKE(6);
    a.cu_seqlens = (const int32_t *)FAKE(7);
    a.cu_seqlens_host = cu;
    return a;
}

static kda_bwd_args bwd(const int32_t *cu, int n, int dk, kda_dtype dt) {
    kda_bwd_args a;
    memset(&a, 0, sizeof a);
    a.struct_size = sizeof a;
    a.num_seqs = n;
    a.total_tokens = cu[n];
    a.num_heads = 2;
    a.dk = a.dv = dk;
    a.in_dtype = dt;
    a.scale = 1.0f;
    a.q = FAKE(1); a.k = FAKE(2); a.v = FAKE(3); a.g = (const float *)FAKE(4); a.beta = (const float *)FAKE(5);
    a.cu_seqlens = (const int32_t *)FAKE(7);
    a.cu_seqlens_host = cu;
    a.d_o = (const float *)FAKE(8);
    a.dq = (float *)FAKE(9); a.dk_out = (float *)FAKE(10); a.dv_out = (float *)FAKE(11); a.dg = (float *)FAKE(12);
    a.dbeta = (float *)FAKE(13);
    return a;
}

static void fwd_case(const char *what, kda_fwd_args a, int want) {
    const size_t ws = kda_chunk_fwd_workspace_bytes(&a);
    expect(what, kda_chunk_fwd(&a, FAKE(64), ws ? ws : 256, NULL), want);
    if (want == KDA_ERR_INVALID_ARGUMENT || want == KDA_ERR_UNSUPPORTED) expect(what, ws == 0 ? want : -1, want);
}

int main(void) {
    int devices = 0;
    if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
        fprintf(stderr, "a GPU is visible: this harness passes fake device pointers and must not launch\n");
        return 77;
    }
    expect("abi version", (int)kda_abi_version(), (int)KDA_ABI_VERSION);
    for (int s = 0; s <= 5; ++s) (void)kda_status_str((kda_status)s);

    /* ragged sequences with empty ones; 3000 sequences (lengths 0..70) */
    const int lens[] = {70, 0, 32, 29, 33, 1, 0, 513};
    const int nl = (int)(sizeof lens / sizeof lens[0]);
    int32_t *cu = cu_from(lens, nl);
    int *many = (int *)malloc(sizeof(int) * 3000);
    for (int i = 0; i < 3000; ++i) many[i] = (i * 37) % 71;
    int32_t *cu_many = cu_from(many, 3000);
    int32_t *cu_empty = cu_from(lens, 0);

    for (int chunk = 32; chunk <= 64; chunk += 32)
        for (int dk = 64; dk <= 128; dk += 64)
            for (int dt = 0; dt <= 1; ++dt) {
                fwd_case("fwd ragged", fwd(cu, nl, dk, chunk, (kda_dtype)dt), KDA_ERR_DEVICE);
                fwd_case("fwd 3000 sequences", fwd(cu_many, 3000, dk, chunk, (kda_dtype)dt), KDA_ERR_DEVICE);
                kda_fwd_args a = fwd(cu, nl, dk, chunk, (kda_dtype)dt);
                a.checkpoint_every = 2 * chunk;
                a.checkpoints = (float *)FAKE(20);
                a.initial_state = (const float *)FAKE(21);
                a.final_state = (float *)FAKE(21);
                fwd_case("fwd checkpoints, aliased states", a, KDA_ERR_DEVICE);
                a.initial_state_indices = (const int32_t *)FAKE(22);
                a.checkpoint_indices = (const int32_t *)FAKE(23);
                a.num_slots = 9;
                fwd_case("fwd pool", a, KDA_ERR_DEVICE);
                a = fwd(cu, nl, dk, chunk, (kda_dtype)dt);
                a.gate_mode = KDA_GATE_PREACTIVATION;
                a.normalize_qk = 1;
                fwd_case("fwd prologue", a, dt == KDA_BF16 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED);
                expect("fwd noalloc", kda_chunk_fwd_noalloc(&a, NULL),
                       dt != KDA_BF16 ? KDA_ERR_UNSUPPORTED
                                      : (chunk == 32 && dk == 128 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED));
                /* sequences cut into segments: plain, with checkpoints and a pool, auto on 3000 */
                a = fwd(cu, nl, dk, chunk, (kda_dtype)dt);
                a.segment_tokens = 64;
                fwd_case("fwd segments", a, chunk == 32 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED);
                expect("fwd noalloc segments", kda_chunk_fwd_noalloc(&a, NULL), KDA_ERR_UNSUPPORTED);
                a.checkpoint_every = 32;
                a.checkpoints = (float *)FAKE(20);
                a.initial_state = (const float *)FAKE(21);
                a.final_state = (float *)FAKE(21);
                a.initial_state_indices = (const int32_t *)FAKE(22);
                a.checkpoint_indices = (const int32_t *)FAKE(23);
                a.num_slots = 9;
                fwd_case("fwd segments, checkpoints, pool", a,
                         chunk == 32 ? KDA_ERR_DEVICE : KDA_ERR_INVALID_ARGUMENT);
                a.segment_tokens = 96;
                a.checkpoint_every = 64;
                fwd_case("fwd segment not a checkpoint multiple", a, KDA_ERR_INVALID_ARGUMENT);
                a = fwd(cu, nl, dk, chunk, (kda_dtype)dt);
                a.segment_tokens = 48;
                fwd_case("fwd segment not a chunk multiple", a, KDA_ERR_INVALID_ARGUMENT);
                a.segment_tokens = -2;
                fwd_case("fwd segment -2", a, KDA_ERR_INVALID_ARGUMENT);
                a.segment_tokens = -1;
                fwd_case("fwd segments off", a, KDA_ERR_DEVICE);
                a = fwd(cu_many, 3000, dk, chunk, (kda_dtype)dt);
                a.segment_tokens = 32;
                fwd_case("fwd 3000 sequences in segments", a, chunk == 32 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED);
            }
    kda_fwd_args a = fwd(cu, nl, 128, 32, KDA_BF16);
    fwd_case("fwd empty batch", fwd(cu_empty, 0, 128, 32, KDA_BF16), KDA_OK);
    a.total_tokens -= 1;
    fwd_case("fwd wrong total", a, KDA_ERR_INVALID_ARGUMENT);
    a = fwd(cu, nl, 128, 32, KDA_BF16);
    a.checkpoint_every = 48;
    fwd_case("fwd checkpoint not a chunk multiple", a, KDA_ERR_INVALID_ARGUMENT);
    a = fwd(cu, nl, 128, 32, KDA_BF16);
    a.q = NULL;
    fwd_case("fwd no q", a, KDA_ERR_INVALID_ARGUMENT);
    a = fwd(cu, nl, 96, 32, KDA_BF16);
    fwd_case("fwd d 96", a, KDA_ERR_UNSUPPORTED);
    a = fwd(cu, nl, 128, 32, KDA_BF16);
    expect("fwd small workspace", kda_chunk_fwd(&a, FAKE(64), 16, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
    expect("fwd misaligned workspace", kda_chunk_fwd(&a, (void *)((uintptr_t)FAKE(64) + 16), 1 << 20, NULL),
           KDA_ERR_INVALID_ARGUMENT);
    expect("fwd null args", kda_chunk_fwd(NULL, FAKE(64), 1 << 20, NULL), KDA_ERR_INVALID_ARGUMENT);
    expect("fwd noalloc null args", kda_chunk_fwd_noalloc(NULL, NULL), KDA_ERR_INVALID_ARGUMENT);
    {   /* more sequences than the allocation-free forward's array holds */
        int *zeros = (int *)calloc(KDA_NOALLOC_MAX_SEQS + 1, sizeof(int));
        int32_t *cu_big = cu_from(zeros, KDA_NOALLOC_MAX_SEQS + 1);
        kda_fwd_args b = fwd(cu_big, KDA_NOALLOC_MAX_SEQS + 1, 128, 32, KDA_BF16);
        expect("fwd noalloc too many", kda_chunk_fwd_noalloc(&b, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
        free(cu_big);
        free(zeros);
    }
    {   /* non-monotone offsets */
        int32_t *bad = cu_from(lens, nl);
        bad[3] = bad[2] - 1;
        kda_fwd_args b = fwd(bad, nl, 128, 32, KDA_BF16);
        b.total_tokens = bad[nl];
        fwd_case("fwd decreasing cu_seqlens", b, KDA_ERR_INVALID_ARGUMENT);
        free(bad);
    }

    /* backward */
    for (int dk = 64; dk <= 128; dk += 64)
        for (int dt = 0; dt <= 1; ++dt) {
            kda_bwd_args b = bwd(cu, nl, dk, (kda_dtype)dt);
            size_t ws = kda_chunk_bwd_workspace_bytes(&b);
            expect("bwd ragged ws > 0", ws > 0, 1);
            expect("bwd ragged", kda_chunk_bwd(&b, FAKE(64), ws, NULL), KDA_ERR_DEVICE);
            b = bwd(cu_many, 3000, dk, (kda_dtype)dt);
            b.initial_state = (const float *)FAKE(21);
            b.d_final_state = (const float *)FAKE(24);
            b.d_initial_state = (float *)FAKE(25);
            b.states = (const float *)FAKE(26);
            ws = kda_chunk_bwd_workspace_bytes(&b);
            expect("bwd 3000 sequences", kda_chunk_bwd(&b, FAKE(64), ws, NULL), KDA_ERR_DEVICE);
            b.gate_mode = KDA_GATE_PREACTIVATION;
            b.normalize_qk = 1;
            ws = kda_chunk_bwd_workspace_bytes(&b);
            expect("bwd prologue", kda_chunk_bwd(&b, FAKE(64), ws ? ws : 256, NULL),
                   dt == KDA_BF16 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED);
            b = bwd(cu, nl, dk, (kda_dtype)dt);
            b.dg = b.dq;
            expect("bwd aliased outputs", kda_chunk_bwd(&b, FAKE(64), 1 << 20, NULL), KDA_ERR_INVALID_ARGUMENT);
            b = bwd(cu, nl, dk, (kda_dtype)dt);
            expect("bwd small workspace", kda_chunk_bwd(&b, FAKE(64), 64, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
            {   /* groups of sequences within a smaller workspace, with and without given states */
                b = bwd(cu, nl, dk, (kda_dtype)dt);
                const size_t full = kda_chunk_bwd_workspace_bytes(&b), least = kda_chunk_bwd_workspace_min_bytes(&b);
                expect("bwd min <= full", least <= full && least > 0, 1);
                expect("bwd groups", kda_chunk_bwd(&b, FAKE(64), least, NULL), KDA_ERR_DEVICE);
                expect("bwd below min", kda_chunk_bwd(&b, FAKE(64), least - 256, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
                b = bwd(cu_many, 3000, dk, (kda_dtype)dt);
                b.initial_state = (const float *)FAKE(21);
                b.d_final_state = (const float *)FAKE(24);
                b.d_initial_state = (float *)FAKE(25);
                b.states = (const float *)FAKE(26);
                b.gate_mode = dt == KDA_BF16 ? KDA_GATE_PREACTIVATION : KDA_GATE_LOG_DECAY;
                expect("bwd 3000 sequences in groups",
                       kda_chunk_bwd(&b, FAKE(64), kda_chunk_bwd_workspace_min_bytes(&b) * 7, NULL), KDA_ERR_DEVICE);
            }
        }
    {
        kda_bwd_args b = bwd(cu_empty, 0, 128, KDA_BF16);
        expect("bwd empty", kda_chunk_bwd(&b, NULL, 0, NULL), KDA_OK);
    }

    /* decode */
    for (int dk = 64; dk <= 128; dk += 64)
        for (int dt = 0; dt <= 1; ++dt) {
            kda_decode_args d;
            memset(&d, 0, sizeof d);
            d.struct_size = sizeof d;
            d.num_seqs = 256;
            d.num_heads = 96;
            d.dk = d.dv = dk;
            d.in_dtype = (kda_dtype)dt;
            d.scale = 1.0f;
            d.q = FAKE(1); d.k = FAKE(2); d.v = FAKE(3); d.g = (const float *)FAKE(4); d.beta = (const float *)FAKE(5);
            d.state = (float *)FAKE(6);
            d.o = (float *)FAKE(7);
            expect("decode", kda_decode_step(&d, NULL), KDA_ERR_DEVICE);
            d.state_indices = (const int32_t *)FAKE(8);
            d.num_slots = 300;
            expect("decode pool", kda_decode_step(&d, NULL), KDA_ERR_DEVICE);
            d.gate_mode = KDA_GATE_PREACTIVATION;
            expect("decode prologue", kda_decode_step(&d, NULL), dt == KDA_BF16 ? KDA_ERR_DEVICE : KDA_ERR_UNSUPPORTED);
            d.o = d.state;
            expect("decode o aliases state", kda_decode_step(&d, NULL),
                   dt == KDA_BF16 ? KDA_ERR_INVALID_ARGUMENT : KDA_ERR_UNSUPPORTED);
        }
    free(cu);
    free(cu_many);
    free(cu_empty);
    free(many);
    printf("host ABI harness: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
