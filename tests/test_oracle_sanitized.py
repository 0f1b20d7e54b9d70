"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc) and run
on a ragged varlen case with an empty and a one-token sequence, initial states, checkpoints and
four threads: no memory or undefined-behaviour error."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
/* Drive the C oracle under ASan/UBSan on a ragged varlen case with checkpoints and decode. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
typedef struct {
    int32_t num_seqs, num_heads, dk, dv;
    const int64_t *cu_seqlens;
    const float *q, *k, *v, *g, *beta;
    double scale;
    const float *S0;
    double *o;
    double *S_final;
    int32_t ckpt_every;
    double *ckpt;
    int32_t n_threads;
} oracle_fwd_args;
int oracle_kda_forward(const oracle_fwd_args *a);
static float *rnd(size_t n, float lo, float hi) {
    float *x = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * (float)rand() / (float)RAND_MAX;
    return x;
}
int main(void) {
    const int N = 5, H = 3, dk = 8, dv = 6;
    int64_t cu[6] = {0, 70, 70, 71, 103, 167};
    const int T = 167, every = 32;
    int64_t nck = 0;
    for (int n = 0; n < N; ++n) nck += (cu[n + 1] - cu[n]) / every;
    oracle_fwd_args a = {N, H, dk, dv, cu, rnd((size_t)T * H * dk, -1, 1), rnd((size_t)T * H * dk, -1, 1),
                         rnd((size_t)T * H * dv, -1, 1), rnd((size_t)T * H * dk, -5, 0), rnd((size_t)T * H, 0, 1),
                         0.7, rnd((size_t)N * H * dk * dv, -0.1f, 0.1f), malloc((size_t)T * H * dv * 8),
                         malloc((size_t)N * H * dk * dv * 8), every, malloc((size_t)(nck ? nck : 1) * H * dk * dv * 8), 4};
    int st = oracle_kda_forward(&a);
    printf("status %d, o[0] %.6f, checkpoints %lld\n", st, a.o[0], (long long)nck);
    return st;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_sanitizers(tmp_path):
    src = tmp_path / "drive.c"
    src.write_text(DRIVER)
    exe = tmp_path / "drive"
    r = subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-o", str(exe), str(src),
                        os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-lpthread"],
                       capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")   # the driver does not free its inputs
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "status 0" in run.stdout
