"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something it does not share code with:
a hand-worked example, closed forms, exact retrieval, explicit-matrix brute
force, a separately written chunked form, or an invariant of the recurrence.
test_oracle_mutants.py shows that plausible mistakes planted in the oracle's
source fail at least one of these pins.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.chunked import forward_chunked
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T, H, dk, dv, beta_hi=1.0, unit_k=True):
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    g = (-5.0 * rng.random((T, H, dk))).astype(np.float32)
    beta = (beta_hi * rng.random((T, H))).astype(np.float32)
    return q, k, v, g, beta


# ---------------------------------------------------------------------------------------------
def test_hand_example(fwd=None):
    """Hand-worked 3-token example (tests/golden/hand_example_d2.md)."""
    fwd = fwd or oracle.forward
    d = json.load(open(os.path.join(GOLDEN, "hand_example_d2.json")))
    q = np.array(d["q"], np.float32)[:, None, :]
    k = np.array(d["k"], np.float32)[:, None, :]
    v = np.array(d["v"], np.float32)[:, None, :]
    g = np.log(np.array(d["alpha"], np.float64)).astype(np.float32)[:, None, :]
    beta = np.array(d["beta"], np.float32)[:, None]
    o, S, _ = fwd(q, k, v, g, beta, scale=d["scale"])
    np.testing.assert_allclose(o[:, 0, :], np.array(d["expected_o"]), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(S[0, 0], np.array(d["expected_S"]), rtol=1e-6, atol=1e-6)
    o2, S2 = forward_chunked(q, k, v, g, beta, scale=d["scale"], chunk=2)
    np.testing.assert_allclose(o2[:, 0, :], np.array(d["expected_o"]), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(S2[0, 0], np.array(d["expected_S"]), rtol=1e-6, atol=1e-6)


def test_pure_decay_closed_form(fwd=None):
    """P-a: beta = 0 -> S_T = Diag(exp(sum g)) S0 and o_t = scale * S0^T (exp(G_t) * q_t)."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(1)
    lens = [13, 0, 40]
    T, H, dk, dv = sum(lens), 2, 5, 3
    q, k, v, g, _ = _rand_case(rng, T, H, dk, dv)
    g *= 0.1
    beta = np.zeros((T, H), np.float32)
    S0 = rng.standard_normal((3, H, dk, dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S, _ = fwd(q, k, v, g, beta, cu, 0.7, S0)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        G = np.cumsum(g[s:e].astype(np.float64), axis=0)                 # [L, H, dk]
        for h in range(H):
            S0d = S0[n, h].astype(np.float64)
            Gl = G[-1, h] if e > s else np.zeros(dk)
            np.testing.assert_allclose(S[n, h], np.exp(Gl)[:, None] * S0d, rtol=1e-12, atol=1e-13)
            for t in range(e - s):
                exp_o = 0.7 * S0d.T @ (np.exp(G[t, h]) * q[s + t, h].astype(np.float64))
                np.testing.assert_allclose(o[s + t, h], exp_o, rtol=1e-12, atol=1e-13)


def test_exact_retrieval_and_overwrite(fwd=None):
    """P-b: g = 0, beta = 1, orthonormal keys: the state becomes sum_i k_i v_i^T, a query
    k_j returns v_j, and rewriting k_j replaces v_j only (targeted overwrite)."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(2)
    dk, dv, m = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :m].T.astype(np.float32)                                 # m orthonormal keys
    vals = rng.standard_normal((m, dv)).astype(np.float32)
    vnew = rng.standard_normal(dv).astype(np.float32)
    j = 3
    # tokens: m writes, m reads, 1 overwrite of key j, m reads
    ks = np.concatenate([keys, keys, keys[j:j + 1], keys])
    qs = np.concatenate([keys, keys, keys[j:j + 1], keys])
    vs = np.concatenate([vals, np.zeros((m, dv)), vnew[None], np.zeros((m, dv))]).astype(np.float32)
    bs = np.concatenate([np.ones(m), np.zeros(m), np.ones(1), np.zeros(m)]).astype(np.float32)
    T = len(ks)
    g = np.zeros((T, 1, dk), np.float32)
    o, S, _ = fwd(qs[:, None], ks[:, None], vs[:, None], g, bs[:, None])
    # keys are orthonormal only to fp32 rounding: tolerance reflects that, not the oracle
    tol = dict(rtol=0, atol=2e-6)
    np.testing.assert_allclose(o[m:2 * m, 0], vals, **tol)
    expect = vals.copy()
    expect[j] = vnew
    np.testing.assert_allclose(o[2 * m + 1:, 0], expect, **tol)
    np.testing.assert_allclose(S[0, 0], keys.T.astype(np.float64) @ expect, **tol)


def _brute(q, k, v, g, beta, S0, scale):
    """Explicit product form: M_t = (I - beta k k^T) Diag(alpha); S_t = M_t S + beta k v^T."""
    T, dk = q.shape
    S = S0.astype(np.float64).copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        kt = k[t].astype(np.float64)[:, None]
        Mt = (np.eye(dk) - beta[t] * kt @ kt.T) @ np.diag(np.exp(g[t].astype(np.float64)))
        S = Mt @ S + beta[t] * kt @ v[t].astype(np.float64)[None, :]
        o[t] = scale * S.T @ q[t].astype(np.float64)
    return o, S


@pytest.mark.parametrize("dk,dv", [(1, 1), (1, 3), (2, 2), (3, 1), (4, 4), (4, 2)])
def test_brute_force_product_form(dk, dv, fwd=None):
    """P-c: tiny problems against the explicit matrix product form (unnormalised keys,
    beta up to 2)."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(10 * dk + dv)
    T, H = 6, 2
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv, beta_hi=2.0, unit_k=False)
    S0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    o, S, _ = fwd(q, k, v, g, beta, None, 1.3, S0)
    for h in range(H):
        ob, Sb = _brute(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h], 1.3)
        np.testing.assert_allclose(o[:, h], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sb, rtol=1e-12, atol=1e-12)


def test_scalar_recurrence(fwd=None):
    """P-c, d = 1: s_t = (1 - beta k^2) alpha s_{t-1} + beta k v, o_t = scale q s_t."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(3)
    q, k, v, g, beta = _rand_case(rng, 9, 1, 1, 1, unit_k=False)
    o, S, _ = fwd(q, k, v, g, beta, scale=0.5)
    s = 0.0
    for t in range(9):
        kk, bb = float(k[t, 0, 0]), float(beta[t, 0])
        s = (1 - bb * kk * kk) * np.exp(float(g[t, 0, 0])) * s + bb * kk * float(v[t, 0, 0])
        assert abs(o[t, 0, 0] - 0.5 * float(q[t, 0, 0]) * s) <= 1e-12 * max(1.0, abs(s))
    assert abs(S[0, 0, 0, 0] - s) <= 1e-12 * max(1.0, abs(s))


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_chunked_equals_recurrent(chunk):
    """P-d: the separately written chunked form agrees with the recurrence (varlen,
    partial chunks, random initial state)."""
    w = W.make_prefill([70, 1, 33, 64], H=2, dk=12, dv=6, dtype="f32", seed=4, s0_std=0.3)
    o, S, _ = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 0.9, w.s0)
    o2, S2 = forward_chunked(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 0.9, w.s0, chunk=chunk)
    assert W.rel_max_err(o2, o) < 1e-12
    assert W.rel_max_err(S2, S) < 1e-12


def test_scalar_gate_special_case():
    """P-j: a gate shared by all channels (the scalar-gate delta rule) runs through the
    same code; chunked and recurrent forms agree."""
    w = W.make_prefill([90], H=1, dk=8, dv=4, dtype="f32", seed=8, s0_std=0.2)
    g = np.repeat(w.g[:, :, :1], 8, axis=2)
    o, S, _ = oracle.forward(w.q, w.k, w.v, g, w.beta, w.cu_seqlens, 1.0, w.s0)
    o2, S2 = forward_chunked(w.q, w.k, w.v, g, w.beta, w.cu_seqlens, 1.0, w.s0, chunk=16)
    assert W.rel_max_err(o2, o) < 1e-12 and W.rel_max_err(S2, S) < 1e-12


def test_linearity_in_values_and_state(fwd=None):
    """P-e: for fixed q, k, g, beta the map (V, S0) -> (O, S_T) is linear."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(5)
    T, H, dk, dv = 30, 2, 6, 4
    q, k, _, g, beta = _rand_case(rng, T, H, dk, dv)
    V1, V2 = (rng.standard_normal((T, H, dv)).astype(np.float32) for _ in range(2))
    S1, S2 = (rng.standard_normal((1, H, dk, dv)).astype(np.float32) for _ in range(2))
    a, b = 0.75, -1.5   # exact in fp32, so a*V1 + b*V2 is formed exactly enough
    Va = (a * V1.astype(np.float64) + b * V2).astype(np.float32)
    Sa = (a * S1.astype(np.float64) + b * S2).astype(np.float32)
    oA, sA, _ = fwd(q, k, Va, g, beta, None, 1.0, Sa)
    o1, s1, _ = fwd(q, k, V1, g, beta, None, 1.0, S1)
    o2, s2, _ = fwd(q, k, V2, g, beta, None, 1.0, S2)
    # inputs Va, Sa are rounded to fp32; compare against the same rounding of the combination
    np.testing.assert_allclose(oA, a * o1 + b * o2, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(sA, a * s1 + b * s2, rtol=1e-6, atol=1e-6)


def test_value_column_separability(fwd=None):
    """P-f: columns of (V, S0) never mix: running column blocks separately gives the
    same columns of O and S_T (this is what lets the GPU split d_v across waves)."""
    fwd = fwd or oracle.forward
    w = W.make_prefill([50], H=2, dk=8, dv=8, dtype="f32", seed=9, s0_std=0.5)
    o, S, _ = fwd(w.q, w.k, w.v, w.g, w.beta, None, 1.0, w.s0)
    for c0, c1 in [(0, 3), (3, 8)]:
        ob, Sb, _ = fwd(w.q, w.k, w.v[:, :, c0:c1], w.g, w.beta, None, 1.0, w.s0[..., c0:c1])
        np.testing.assert_array_equal(ob, o[:, :, c0:c1])
        np.testing.assert_array_equal(Sb, S[..., c0:c1])


def test_chaining_and_checkpoint_resume(fwd=None):
    """P-g: run(x1 ++ x2, S0) == run(x2, run(x1, S0).final), and resuming from any
    checkpoint reproduces the tail."""
    fwd = fwd or oracle.forward
    w = W.make_prefill([160], H=2, dk=6, dv=5, dtype="f32", seed=11, s0_std=0.4)
    o, S, ck = fwd(w.q, w.k, w.v, w.g, w.beta, None, 1.0, w.s0, checkpoint_every=32)
    assert ck.shape[0] == 5
    for m in range(ck.shape[0]):
        p = 32 * (m + 1)
        sl = slice(p, None)
        ot, St, _ = fwd(w.q[sl], w.k[sl], w.v[sl], w.g[sl], w.beta[sl], None, 1.0, ck[m][None].astype(np.float32))
        np.testing.assert_allclose(ot, o[sl], rtol=1e-6, atol=1e-6)   # checkpoint rounded to fp32
        np.testing.assert_allclose(St, S, rtol=1e-6, atol=1e-6)
        # head = first p tokens; its final state is checkpoint m
        _, Sh, _ = fwd(w.q[:p], w.k[:p], w.v[:p], w.g[:p], w.beta[:p], None, 1.0, w.s0)
        np.testing.assert_array_equal(Sh[0], ck[m])
    # the last checkpoint of a sequence whose length is a multiple of `every` is the final state
    np.testing.assert_array_equal(ck[-1], S[0])


def test_packing_invariance(fwd=None):
    """P-h: a packed varlen batch equals separate per-sequence runs."""
    fwd = fwd or oracle.forward
    lens = [17, 0, 64, 5]
    w = W.make_prefill(lens, H=3, dk=4, dv=4, dtype="f32", seed=12, s0_std=0.3)
    cu = w.cu_seqlens
    o, S, ck = fwd(w.q, w.k, w.v, w.g, w.beta, cu, 1.0, w.s0, checkpoint_every=16)
    base = 0
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        on, Sn, ckn = fwd(w.q[sl], w.k[sl], w.v[sl], w.g[sl], w.beta[sl], None, 1.0, w.s0[n:n + 1],
                          checkpoint_every=16)
        np.testing.assert_array_equal(on, o[sl])
        np.testing.assert_array_equal(Sn[0], S[n])
        np.testing.assert_array_equal(ckn, ck[base:base + L // 16])
        base += L // 16


def test_decode_equals_prefill_of_one_token():
    """P-i: a decode step is the recurrence with T = 1 per sequence."""
    d = W.make_decode(5, 2, 8, 6, "f32", seed=13)
    od, Sd = oracle.decode(d.q, d.k, d.v, d.g, d.beta, d.s0, 0.8)
    cu = np.arange(6)
    op, Sp, _ = oracle.forward(d.q, d.k, d.v, d.g, d.beta, cu, 0.8, d.s0)
    np.testing.assert_array_equal(od, op)
    np.testing.assert_array_equal(Sd, Sp)


def test_one_token_from_zero_state(fwd=None):
    """P-l: S_1 = beta k v^T and o_1 = scale * beta (q.k) v."""
    fwd = fwd or oracle.forward
    rng = np.random.default_rng(14)
    q, k, v, g, beta = _rand_case(rng, 1, 3, 7, 5)
    o, S, _ = fwd(q, k, v, g, beta, None, 1.7)
    for h in range(3):
        kk, qq, vv, bb = (x.astype(np.float64) for x in (k[0, h], q[0, h], v[0, h], beta[0, h]))
        np.testing.assert_allclose(S[0, h], bb * np.outer(kk, vv), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o[0, h], 1.7 * bb * np.dot(qq, kk) * vv, rtol=1e-13, atol=1e-15)


def test_state_norm_bound():
    """Sanity bound: with |k| = 1, beta in [0,1], alpha <= 1,
    ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    w = W.make_prefill([1] * 40, H=2, dk=8, dv=8, dtype="f32", seed=15, s0_std=0.5)
    S = w.s0[:1].copy()
    for t in range(40):
        sl = slice(t, t + 1)
        _, Sn = oracle.decode(w.q[sl], w.k[sl], w.v[sl], w.g[sl], w.beta[sl], S)
        for h in range(2):
            lhs = np.linalg.norm(Sn[0, h])
            rhs = np.linalg.norm(S[0, h].astype(np.float64)) + w.beta[t, h] * np.linalg.norm(w.v[t, h])
            assert lhs <= rhs * (1 + 1e-12)
        S = Sn.astype(np.float32)


def test_workload_generator_properties():
    """The generator produces the documented distributions (unit-norm keys, q scaled
    by d_k^-1/2, g in (-5, 0), beta in (0, 1), bf16-exact values)."""
    w = W.make_prefill([300], H=2, dk=64, dv=64, dtype="bf16", seed=0, s0_std=0.1)
    assert np.allclose(np.linalg.norm(w.k.astype(np.float64), axis=-1), 1.0, atol=1e-2)
    assert np.allclose(np.linalg.norm(w.q.astype(np.float64), axis=-1), 64 ** -0.5, atol=1e-3)
    assert np.all(w.g < 0) and np.all(w.g > -5)
    assert np.all(w.beta > 0) and np.all(w.beta < 1)
    for x in (w.q, w.k, w.v):
        np.testing.assert_array_equal(W.round_bf16(x), x)
    assert abs(float(np.std(w.s0)) - 0.1) < 0.01
    L = W.varlen_lengths()
    assert len(L) == 64 and all(512 <= x <= 131072 and x % 512 == 0 for x in L)


# ---- paged state pool --------------------------------------------------------------------------
def test_decode_paged_is_decode_on_the_selected_slots():
    """The pool form of decode: identity slots reproduce decode; a permutation moves each result
    to its slot; a sequence with no slot (-1, or out of range) leaves the pool alone and reads 0."""
    d = W.make_decode(6, 2, 8, 6, "f32", seed=31)
    od, Sd = oracle.decode(d.q, d.k, d.v, d.g, d.beta, d.s0, 0.7)
    o1, p1 = oracle.decode_paged(d.q, d.k, d.v, d.g, d.beta, d.s0, np.arange(6), 0.7)
    np.testing.assert_array_equal(o1, od)
    np.testing.assert_array_equal(p1, Sd)
    # pool of 9 slots; sequence n lives in slot perm[n]; sequences 2 and 5 are inactive
    rng = np.random.default_rng(5)
    pool = rng.standard_normal((9, 2, 8, 6)).astype(np.float32)
    perm = np.array([7, 0, -1, 3, 8, 9])            # 9 is out of range: inactive too
    pool[perm[[0, 1, 3, 4]]] = d.s0[[0, 1, 3, 4]]
    o2, p2 = oracle.decode_paged(d.q, d.k, d.v, d.g, d.beta, pool, perm, 0.7)
    for n in (0, 1, 3, 4):
        np.testing.assert_array_equal(o2[n], od[n])
        np.testing.assert_array_equal(p2[perm[n]], Sd[n])
    for n in (2, 5):
        assert not o2[n].any()
    untouched = [s for s in range(9) if s not in (7, 0, 3, 8)]
    np.testing.assert_array_equal(p2[untouched], pool[untouched].astype(np.float64))


def test_forward_paged_prefix_reuse():
    """Prefix reuse through the pool: a run writes its 512-token-style checkpoints (here every
    16) into pool slots; a second run that starts from one of those slots over the remaining
    tokens reproduces the tail of running the whole sequence (P-g through the pool)."""
    w = W.make_prefill([80], H=2, dk=5, dv=4, dtype="f32", seed=32, s0_std=0.3)
    o, S, ck = oracle.forward(w.q, w.k, w.v, w.g, w.beta, None, 1.0, w.s0, checkpoint_every=16)
    pool = np.zeros((8, 2, 5, 4), dtype=np.float32)
    pool[6] = w.s0[0]
    cidx = np.array([1, -1, 4, 2, 0])                # checkpoint 1 is not kept
    o1, S1, pool1 = oracle.forward_paged(w.q, w.k, w.v, w.g, w.beta, None, 1.0, pool,
                                         initial_state_indices=np.array([6]), checkpoint_every=16,
                                         checkpoint_indices=cidx)
    np.testing.assert_array_equal(o1, o)
    np.testing.assert_array_equal(S1, S)
    for m, sl in enumerate(cidx):
        if sl >= 0:
            np.testing.assert_array_equal(pool1[sl], ck[m])
    np.testing.assert_array_equal(pool1[[3, 5, 6, 7]], pool[[3, 5, 6, 7]].astype(np.float64))
    # resume from the checkpoint after token 48 (checkpoint 2, slot 4) over tokens 48..79
    tail = slice(48, None)
    o2, S2, _ = oracle.forward_paged(w.q[tail], w.k[tail], w.v[tail], w.g[tail], w.beta[tail], None, 1.0,
                                     pool1.astype(np.float32), initial_state_indices=np.array([4]))
    np.testing.assert_allclose(o2, o[tail], rtol=1e-6, atol=1e-6)   # the slot holds fp32 values
    np.testing.assert_allclose(S2, S, rtol=1e-6, atol=1e-6)
    # a slot index of -1 starts from zeros
    o3, _, _ = oracle.forward_paged(w.q, w.k, w.v, w.g, w.beta, None, 1.0, pool,
                                    initial_state_indices=np.array([-1]))
    o0, _, _ = oracle.forward(w.q, w.k, w.v, w.g, w.beta, None, 1.0, None)
    np.testing.assert_array_equal(o3, o0)


# ---- fused prologue ------------------------------------------------------------------------------
def test_prologue_closed_values():
    """g = -5 sigmoid(a): -2.5 at a = 0, -> -5 and -> 0 at the tails; beta = sigmoid(b): 0.5 at 0;
    L2 normalisation: (3, 4) -> (0.6, 0.8), a zero vector stays zero."""
    a = np.array([[[0.0, 40.0, -40.0, 1.0]]])
    b = np.array([[0.0]])
    q = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    k = np.zeros((1, 1, 4))
    qn, kn, g, beta = oracle.prologue(q, k, a, b)
    assert g[0, 0, 0] == -2.5 and beta[0, 0] == 0.5
    assert abs(g[0, 0, 1] + 5.0) < 1e-15 and abs(g[0, 0, 2]) < 1e-15
    assert abs(g[0, 0, 3] + 5.0 / (1.0 + np.exp(-1.0))) < 1e-15
    np.testing.assert_allclose(qn[0, 0], [0.6, 0.8, 0.0, 0.0], rtol=0, atol=1e-16)
    assert not kn.any()


def test_fused_forward_is_invariant_to_the_scale_of_q_and_k():
    """With normalisation, rescaling each raw q and k row by positive factors leaves the output
    unchanged (up to the fp32 rounding of the normalised inputs), and equals forward() on the
    normalised, gated inputs."""
    w = W.make_prefill_raw([40, 17], H=2, dk=8, dv=6, seed=7, s0_std=0.2)
    o, S, _ = oracle.forward_fused(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 0.5, w.s0)
    rng = np.random.default_rng(3)
    cq = rng.uniform(0.1, 10.0, size=w.q.shape[:2] + (1,))
    ck = rng.uniform(0.1, 10.0, size=w.k.shape[:2] + (1,))
    o2, S2, _ = oracle.forward_fused(w.q * cq, w.k * ck, w.v, w.g, w.beta, w.cu_seqlens, 0.5, w.s0)
    np.testing.assert_allclose(o2, o, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(S2, S, rtol=1e-5, atol=1e-6)
    qn = w.q / np.linalg.norm(w.q.astype(np.float64), axis=-1, keepdims=True)
    kn = w.k / np.linalg.norm(w.k.astype(np.float64), axis=-1, keepdims=True)
    g = -5.0 * (1.0 / (1.0 + np.exp(-w.g.astype(np.float64))))
    beta = 1.0 / (1.0 + np.exp(-w.beta.astype(np.float64)))
    o3, S3, _ = oracle.forward(qn, kn, w.v, g, beta, w.cu_seqlens, 0.5, w.s0)
    np.testing.assert_array_equal(o3, o)
    np.testing.assert_array_equal(S3, S)


# ---- backward (adjoint) ----------------------------------------------------------------------------
def _loss(q, k, v, g, beta, S0, do, dSf, scale, cu=None):
    from oracle.backward import forward_states
    T, H, _ = q.shape
    cu = [0, T] if cu is None else cu
    L = 0.0
    for n in range(len(cu) - 1):
        for h in range(H):
            sl = slice(cu[n], cu[n + 1])
            st, o = forward_states(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], S0[n, h], scale)
            L += float(np.sum(do[sl, h] * o)) + float(np.sum(dSf[n, h] * st[-1]))
    return L


def test_backward_matches_finite_differences():
    """Central differences of L = sum(do*o) + sum(dS_T*S_T) against every gradient the adjoint
    returns (q, k, v, g, beta, S0), on two packed sequences of a small problem."""
    from oracle.backward import backward
    rng = np.random.default_rng(17)
    T, H, dk, dv, cu = 7, 2, 3, 4, [0, 4, 7]
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk)) * 0.6
    v = rng.standard_normal((T, H, dv))
    g = -rng.random((T, H, dk)) * 2.0
    beta = rng.random((T, H))
    S0 = rng.standard_normal((2, H, dk, dv)) * 0.5
    do = rng.standard_normal((T, H, dv))
    dSf = rng.standard_normal((2, H, dk, dv))
    scale = 0.7
    grads = backward(q, k, v, g, beta, cu, scale, S0, do, dSf)
    args = [q, k, v, g, beta, S0]
    eps = 1e-6
    for which, (x, gx) in enumerate(zip(args, grads)):
        for idx in np.ndindex(*x.shape):
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            fd = (_loss(*xp, do, dSf, scale, cu) - _loss(*xm, do, dSf, scale, cu)) / (2 * eps)
            assert abs(fd - gx[idx]) <= 1e-7 * max(1.0, abs(fd)), (which, idx, fd, gx[idx])


def test_backward_fused_prologue_matches_finite_differences():
    """Central differences of the same L, now a function of the raw q, k, the gate pre-activations
    a, b (g = -5 sigmoid(a), beta = sigmoid(b)) and v, S0, against backward_fused: gate and
    normalisation, the gate alone, the normalisation alone (then a, b are g and beta)."""
    import oracle
    from oracle.backward import backward_fused
    rng = np.random.default_rng(29)
    T, H, dk, dv, cu = 6, 2, 3, 4, [0, 2, 6]
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    a = rng.standard_normal((T, H, dk))
    b = rng.standard_normal((T, H))
    S0 = rng.standard_normal((2, H, dk, dv)) * 0.5
    do = rng.standard_normal((T, H, dv))
    dSf = rng.standard_normal((2, H, dk, dv))
    scale = 0.8
    for gate, normalize in ((True, True), (True, False), (False, True)):
        a_in, b_in = (a, b) if gate else (-0.5 * np.abs(a), 1.0 / (1.0 + np.exp(-b)))

        def loss(q_, k_, v_, a_, b_, S0_):
            qn, kn, g, beta = oracle.prologue(q_, k_, a_, b_, normalize)
            if not gate:
                g, beta = a_, b_
            return _loss(qn, kn, v_, g, beta, S0_, do, dSf, scale, cu)
        grads = backward_fused(q, k, v, a_in, b_in, cu, scale, S0, do, dSf, normalize, gate)
        args = [q, k, v, a_in, b_in, S0]
        eps = 1e-6
        for which, (x, gx) in enumerate(zip(args, grads)):
            for idx in np.ndindex(*x.shape):
                xp = [y.copy() for y in args]
                xm = [y.copy() for y in args]
                xp[which][idx] += eps
                xm[which][idx] -= eps
                fd = (loss(*xp) - loss(*xm)) / (2 * eps)
                assert abs(fd - gx[idx]) <= 1e-7 * max(1.0, abs(fd)), (gate, normalize, which, idx, fd, gx[idx])


def test_backward_pure_decay_closed_form():
    """beta = 0: o_t = scale S0^T (e^{G_t} * q_t) and S_T = Diag(e^{G_T}) S0, so
    dq_t = scale e^{G_t} * (S0 do_t), dv = dk = 0 (k and v enter only through u = 0), and
    dS0 = scale sum_t (e^{G_t} q_t) do_t^T + Diag(e^{G_T}) dS_T."""
    from oracle.backward import backward
    rng = np.random.default_rng(23)
    T, dk, dv = 6, 4, 3
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = -rng.random((T, 1, dk))
    beta = np.zeros((T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((T, 1, dv))
    dSf = rng.standard_normal((1, 1, dk, dv))
    dq, dk_, dv_, dg, db, dS0 = backward(q, k, v, g, beta, None, 0.5, S0, do, dSf)
    G = np.cumsum(g[:, 0], axis=0)                      # [T, dk]
    for t in range(T):
        np.testing.assert_allclose(dq[t, 0], 0.5 * np.exp(G[t]) * (S0[0, 0] @ do[t, 0]), rtol=1e-12)
    assert not dv_.any()
    ref = 0.5 * sum(np.outer(np.exp(G[t]) * q[t, 0], do[t, 0]) for t in range(T)) + np.exp(G[-1])[:, None] * dSf[0, 0]
    np.testing.assert_allclose(dS0[0, 0], ref, rtol=1e-12)
    assert not dk_.any() or np.allclose(dk_, 0.0)       # k enters only through u, which is 0


def test_backward_amplification_bounds_dg():
    """The amplification diagnostic sums the magnitudes of the terms of dg: amp >= |dg| always, with
    equality when the state has one value column (d_v = 1: a single term)."""
    from oracle import backward as OB
    for dv in (1, 3):
        rng = np.random.default_rng(11 + dv)
        T, H, dk = 9, 2, 3
        q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
        v, do = rng.standard_normal((T, H, dv)), rng.standard_normal((T, H, dv))
        g, beta = -rng.uniform(0, 2, (T, H, dk)), rng.uniform(0, 1, (T, H))
        s0, dsf = rng.standard_normal((1, H, dk, dv)), rng.standard_normal((1, H, dk, dv))
        *grads, amp = OB.backward(q, k, v, g, beta, [0, T], 0.7, s0, do, dsf, amplification=True)
        plain = OB.backward(q, k, v, g, beta, [0, T], 0.7, s0, do, dsf)
        for x, y in zip(grads, plain):
            np.testing.assert_array_equal(x, y)
        dg = grads[3]
        assert np.all(amp >= np.abs(dg) - 1e-15)
        if dv == 1:
            np.testing.assert_allclose(amp, np.abs(dg), rtol=1e-13, atol=1e-15)
        else:
            assert np.any(amp > np.abs(dg) * (1 + 1e-6))
