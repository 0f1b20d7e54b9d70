"""Mistakes planted in a copy of the oracle source (on the CPU) must fail at
least one pin of test_oracle_pins.py.  This checks that the pins constrain
every part of the recurrence: gate order, residual sign, beta, the post-update
read-out, orientation of S, and checkpoint indexing."""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("no_forget_gate", "for (int i = 0; i < dk; ++i) alpha[i] = exp((double)gt[i]);",
     "for (int i = 0; i < dk; ++i) alpha[i] = 1.0;"),
    ("residual_sign", "u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = bt * ((double)vt[j] + p[j]);"),
    ("no_beta", "u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = ((double)vt[j] - p[j]);"),
    ("no_delta", "u[j] = bt * ((double)vt[j] - p[j]);", "u[j] = bt * ((double)vt[j]);"),
    ("scale_dropped", "for (int j = 0; j < dv; ++j) ot[j] *= a->scale;", ";"),
    ("transposed_readout", "ot[j] += S[i * dv + j] * qi;", "ot[j] += S[(j % dk) * dv + (i % dv)] * qi;"),
    ("checkpoint_off_by_one", "const int64_t m = ckpt_base + pos / a->ckpt_every - 1;",
     "const int64_t m = ckpt_base + pos / a->ckpt_every - (pos / a->ckpt_every > 1 ? 2 : 1);"),
    ("gate_after_write",
     "        /* prediction p = S^T k_t from the decayed state */",
     "        for (int i = 0; i < dk; ++i) for (int j = 0; j < dv; ++j) S[i * dv + j] /= alpha[i];\n"
     "        /* prediction p = S^T k_t from the decayed state */"),
]

PINS = [P.test_hand_example, P.test_pure_decay_closed_form, P.test_exact_retrieval_and_overwrite,
        P.test_scalar_recurrence, P.test_chaining_and_checkpoint_resume, P.test_one_token_from_zero_state,
        lambda fwd: [P.test_brute_force_product_form(dk, dv, fwd=fwd) for dk, dv in [(1, 1), (2, 2), (4, 2)]]]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert orig in src, f"mutation anchor for {name} not found"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(orig, bad, 1))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-o", str(so), str(path), "-lm"])
    fwd = oracle.forward_from_library(str(so))
    failed = []
    for pin in PINS:
        try:
            pin(fwd=fwd)
        except AssertionError:
            failed.append(getattr(pin, "__name__", "brute"))
    assert failed, f"planted mistake {name} passed every pin"
