"""Mistakes planted in a copy of the oracle's adjoint (oracle/backward.py, on the CPU) must fail its
pin, central differences of L = sum(do * o) + sum(dS_T * S_T) (the loss evaluated by the unchanged
forward).  This checks that the pin constrains every term of the adjoint: the dropped-term, sign,
missing-decay and transposition mistakes below, and the chain rule through the prologue."""
import importlib.util
import os

import numpy as np
import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")

# (name, original text, planted mistake)
MUTANTS = [
    ("dk_drops_decayed_state_term", "dk_[tt, h] = dS @ u + St @ dp", "dk_[tt, h] = dS @ u"),
    ("dp_sign", "dp = -bt * du", "dp = bt * du"),
    ("dg_without_alpha", "dg_[tt, h] = al * np.sum(dSt * S_prev, axis=1)",
     "dg_[tt, h] = np.sum(dSt * S_prev, axis=1)"),
    ("carry_without_decay", "dS = al[:, None] * dSt", "dS = dSt"),
    ("dbeta_without_prediction", "db_[tt, h] = du @ (vt - p)", "db_[tt, h] = du @ vt"),
    ("dq_from_previous_state", "dq_[tt, h] = scale * (S_t @ do[tt, h])", "dq_[tt, h] = scale * (S_prev @ do[tt, h])"),
    ("rank_one_transposed", "dSt = dS + np.outer(kt, dp)", "dSt = dS + np.outer(dp[:len(kt)], kt[:len(dp)])"),
]
FUSED_MUTANTS = [
    ("gate_chain_sign", "da = dg * (-5.0) * s * (1.0 - s)", "da = dg * 5.0 * s * (1.0 - s)"),
    ("beta_chain_dropped", "db = dbeta * beta * (1.0 - beta)", "db = dbeta"),
    ("projection_dropped", "proj = dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)", "proj = dxn"),
]


def _load(text, tmp_path, tag):
    f = tmp_path / f"backward_{tag}.py"
    f.write_text(text)
    spec = importlib.util.spec_from_file_location(f"oracle._backward_{tag}", str(f))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _problem(seed=5, dk=3, dv=3):
    rng = np.random.default_rng(seed)
    T, H, cu = 5, 1, [0, 2, 5]
    x = dict(q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)) * 0.6,
             v=rng.standard_normal((T, H, dv)), a=rng.standard_normal((T, H, dk)),
             b=rng.standard_normal((T, H)), S0=rng.standard_normal((2, H, dk, dv)) * 0.5,
             do=rng.standard_normal((T, H, dv)), dSf=rng.standard_normal((2, H, dk, dv)))
    return x, cu


def _fd_error(grads, loss, args, eps=1e-6):
    worst = 0.0
    for which, (x, gx) in enumerate(zip(args, grads)):
        for idx in np.ndindex(*x.shape):
            xp = [y.copy() for y in args]
            xm = [y.copy() for y in args]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            fd = (loss(*xp) - loss(*xm)) / (2 * eps)
            worst = max(worst, abs(fd - gx[idx]) / max(1.0, abs(fd)))
    return worst


def _plain_error(mod):
    x, cu = _problem()
    g = -0.5 * np.abs(x["a"])
    beta = 1.0 / (1.0 + np.exp(-x["b"]))
    args = [x["q"], x["k"], x["v"], g, beta, x["S0"]]
    grads = mod.backward(*args[:5], cu, 0.8, args[5], x["do"], x["dSf"])

    def loss(q, k, v, g_, b_, S0):
        return P._loss(q, k, v, g_, b_, S0, x["do"], x["dSf"], 0.8, cu)
    return _fd_error(grads, loss, args)


def _fused_error(mod):
    x, cu = _problem(seed=6)
    args = [x["q"], x["k"], x["v"], x["a"], x["b"], x["S0"]]
    grads = mod.backward_fused(*args[:5], cu, 0.8, args[5], x["do"], x["dSf"], normalize=True, gate=True)

    def loss(q, k, v, a, b, S0):
        qn, kn, g, beta = oracle.prologue(q, k, a, b, True)
        return P._loss(qn, kn, v, g, beta, S0, x["do"], x["dSf"], 0.8, cu)
    return _fd_error(grads, loss, args)


def test_unchanged_copy_passes(tmp_path):
    mod = _load(open(SRC).read(), tmp_path, "copy")
    assert _plain_error(mod) <= 1e-7
    assert _fused_error(mod) <= 1e-7


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_in_the_adjoint_is_caught(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, name
    mod = _load(src.replace(orig, bad), tmp_path, name)
    try:
        err = _plain_error(mod)
    except Exception:   # a shape error is caught too
        return
    assert err > 1e-4, (name, err)


@pytest.mark.parametrize("name,orig,bad", FUSED_MUTANTS, ids=[m[0] for m in FUSED_MUTANTS])
def test_planted_mistake_in_the_prologue_chain_rule_is_caught(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, name
    mod = _load(src.replace(orig, bad), tmp_path, name)
    err = _fused_error(mod)
    assert err > 1e-4, (name, err)
