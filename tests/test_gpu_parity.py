"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Metric: max|gpu - oracle| / RMS(oracle) per output tensor, in fp64 over the
whole tensor (any non-finite value fails).  Bars: 1e-4 for the fp32 path
(fp32 inputs), 2e-2 for the bf16-input path (fp32 accumulation, fp32 o and S).
"""
import json
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev():
    return torch.device("cuda:0")


def to_dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev(), dt)


def in_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


CHUNKS = [32, 64]


def run_gpu(w, scale=1.0, s0=True, chunk=32):
    dt = in_dtype(w)
    o, sf, ck = kda.kda_chunk_fwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                                  to_dev(w.beta, torch.float32), list(w.cu_seqlens), scale,
                                  to_dev(w.s0, torch.float32) if (s0 and w.s0 is not None) else None,
                                  True, w.checkpoint_every, chunk_size=chunk)
    torch.cuda.synchronize()
    return o.cpu().numpy(), sf.cpu().numpy(), None if ck is None else ck.cpu().numpy()


def run_ref(w, scale=1.0, s0=True):
    return oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, scale, w.s0 if s0 else None,
                          w.checkpoint_every)


def compare(w, tol=None, scale=1.0, label="", chunk=32):
    tol = tol or TOL[w.dtype]
    o, sf, ck = run_gpu(w, scale, chunk=chunk)
    o_r, s_r, ck_r = run_ref(w, scale)
    errs = {"o": W.rel_max_err(o, o_r), "S": W.rel_max_err(sf, s_r)}
    if ck_r is not None and ck_r.size:
        errs["ckpt"] = W.rel_max_err(ck, ck_r)
    label = f"{label or w.name} C={chunk}"
    print(f"[parity] {label} seqlens={w.seqlens[:8]}{'...' if len(w.seqlens) > 8 else ''} "
          f"H={w.H} d={w.dk} {w.dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": label, "chunk": chunk, "H": w.H, "d": w.dk, "dtype": w.dtype,
                                "tokens": w.total_tokens, "tol": tol, **errs}) + "\n")
    for k_, v_ in errs.items():
        assert v_ <= tol, (k_, v_, tol)
    return errs


# ---- decode ----------------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(d, dtype):
    w = W.make_decode(6, 3, d, d, dtype, seed=21)
    dt = in_dtype(w)
    state = to_dev(w.s0, torch.float32).clone()
    o = kda.kda_decode_step(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                            to_dev(w.beta, torch.float32), state, 0.9)
    torch.cuda.synchronize()
    o_r, s_r = oracle.decode(w.q, w.k, w.v, w.g, w.beta, w.s0, 0.9)
    eo, es = W.rel_max_err(o.cpu().numpy(), o_r), W.rel_max_err(state.cpu().numpy(), s_r)
    print(f"[parity] decode N=6 H=3 d={d} {dtype}: o={eo:.2e} S={es:.2e}", flush=True)
    # decode runs in fp32 on exact inputs, so both paths meet the fp32 bar
    assert eo <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("gate,norm,d", [(True, True, 128), (True, False, 128), (False, True, 128),
                                         (True, True, 64)])
def test_decode_prologue(gate, norm, d):
    """Decode with the gate (g = -5 sigmoid(a) from bf16 a, beta = sigmoid(b)) and/or the L2
    normalisation of q and k inside, against the oracle's prologue + decode step; with the
    normalisation one q row and one k row are zero (they stay zero)."""
    N, H = 9, 3
    w = W.make_prefill_raw([1] * N, H=H, dk=d, dv=d, seed=63, s0_std=0.1)
    q, k = w.q.copy(), w.k.copy()
    if norm:
        q[2, 1] = 0.0
        k[4, 0] = 0.0
    else:
        q = W.round_bf16((q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32))
        k = W.round_bf16((k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32))
    qn, kn, g64, b64 = oracle.prologue(q, k, w.g, w.beta, normalize=norm)
    if gate:
        g_in, b_in, g_ref, b_ref = to_dev(w.g, torch.bfloat16), to_dev(w.beta, torch.float32), g64, b64
    else:
        g32, b32 = g64.astype(np.float32), b64.astype(np.float32)
        g_in, b_in, g_ref, b_ref = to_dev(g32, torch.float32), to_dev(b32, torch.float32), g32, b32
    state = to_dev(w.s0, torch.float32).clone()
    scale = d ** -0.5
    o = kda.kda_decode_step(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(w.v, torch.bfloat16),
                            g_in, b_in, state, scale, gate_preactivation=gate, normalize_qk=norm)
    torch.cuda.synchronize()
    o_r, s_r = oracle.decode(qn, kn, w.v, g_ref, b_ref, w.s0, scale)
    _log(f"decode prologue gate={gate} norm={norm} d={d}",
         {"o": W.rel_max_err(o.cpu().numpy(), o_r), "S": W.rel_max_err(state.cpu().numpy(), s_r)}, 1e-4)


# ---- prefill: small shapes and edge cases ------------------------------------------------------
@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_tiny_f32_T256_H2_d64(chunk):
    w = W.make_workload(0, seed=0)
    compare(w, label="tiny f32 T=256 H=2 d=64", chunk=chunk)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_varlen_ragged(d, dtype, chunk):
    """Several tiles and ragged tails: lengths that are not multiples of 64, an empty
    sequence, a single-token sequence; initial states; checkpoints every 64."""
    w = W.make_prefill([200, 64, 1, 0, 130, 333], H=3, dk=d, dv=d, dtype=dtype, seed=22, s0_std=0.1,
                       checkpoint_every=64)
    compare(w, label=f"varlen d={d} {dtype}", chunk=chunk)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_many_chains_one_workgroup_each(d, dtype):
    # 4 x 40 = 160 (sequence, head) chains: more than half the compute units, so the chunk-32
    # launch gives each chain a single workgroup (fewer chains split the value columns over two)
    w = W.make_prefill([100, 37, 64, 65], 40, d, d, dtype, seed=9, s0_std=0.1, checkpoint_every=64)
    compare(w, label=f"many chains d={d} {dtype}", chunk=32)


@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_more_sequences_than_one_plan_tile(chunk):
    """3000 sequences (lengths 0..70, some empty): the launch plan ranks them over several
    workgroups and LDS tiles of 1024 lengths, and the checkpoint bases are scanned over three
    tiles of 1024; initial states, checkpoints every 64."""
    rng = np.random.default_rng(61)
    lens = [int(x) for x in rng.integers(0, 71, size=3000)]
    w = W.make_prefill(lens, H=1, dk=64, dv=64, dtype="bf16", seed=61, s0_std=0.1, checkpoint_every=64)
    compare(w, label="3000 sequences", chunk=chunk)


@pytest.mark.parametrize("gate", ["min", "zero", "slow"])
@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_gate_extremes(gate, chunk):
    """g = -5 everywhere (the bound: the diagonal-tile factor reaches e^80), g = 0 (no
    decay: long-range accumulation), and slow decay (long memory)."""
    w = W.make_prefill([700], H=2, dk=128, dv=128, dtype="bf16", seed=23, s0_std=0.1, gate=gate)
    compare(w, label=f"gate={gate}", chunk=chunk)


@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_scalar_gate(chunk):
    """The gate shared by all channels (scalar-gate special case) through the same kernels."""
    w = W.make_prefill([300], H=2, dk=128, dv=128, dtype="bf16", seed=24, s0_std=0.1)
    w.g = np.repeat(w.g[:, :, :1], 128, axis=2).copy()
    compare(w, label="scalar gate", chunk=chunk)


@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_exact_retrieval_bf16(chunk):
    """g = 0, beta = 1, orthonormal keys written once each, then read back with beta = 0:
    the read-out returns the stored values (to the bf16-path bar)."""
    rng = np.random.default_rng(25)
    dk = dv = 128
    m = 100
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = W.round_bf16(Qm[:, :m].T.astype(np.float32))
    vals = W.round_bf16(rng.standard_normal((m, dv)).astype(np.float32))
    w = W.make_prefill([2 * m], H=1, dk=dk, dv=dv, dtype="bf16", seed=25, gate="zero")
    w.k[:, 0] = np.concatenate([keys, keys])
    w.q[:, 0] = np.concatenate([keys, keys])
    w.v[:, 0] = np.concatenate([vals, np.zeros_like(vals)])
    w.beta[:, 0] = np.concatenate([np.ones(m), np.zeros(m)]).astype(np.float32)
    errs = compare(w, label="retrieval", chunk=chunk)
    o, _, _ = run_gpu(w, chunk=chunk)
    # the recalled rows are close to the written values (keys are orthonormal only to bf16 rounding)
    assert np.max(np.abs(o[m:, 0] - vals)) / np.sqrt(np.mean(vals ** 2)) < 0.1


@pytest.mark.parametrize("chunk", CHUNKS)
def test_checkpoint_resume_on_gpu(chunk):
    """Resuming the GPU kernel from one of its own checkpoints reproduces the tail."""
    w = W.make_prefill([512], H=2, dk=128, dv=128, dtype="bf16", seed=26, s0_std=0.1, checkpoint_every=128)
    o, sf, ck = run_gpu(w, chunk=chunk)
    p = 256
    w2 = W.Workload("tail", [512 - p], 2, 128, 128, "bf16", w.q[p:], w.k[p:], w.v[p:], w.g[p:], w.beta[p:],
                    ck[1][None].astype(np.float32))
    o2, sf2, _ = run_gpu(w2, chunk=chunk)
    assert W.rel_max_err(o2, o[p:]) < 1e-5 and W.rel_max_err(sf2, sf) < 1e-5
    compare(w, label="ckpt", chunk=chunk)


def test_decode_equals_prefill_of_one_token():
    """A decode step and a prefill of one-token sequences compute the same map."""
    w = W.make_decode(16, 4, 128, 128, "bf16", seed=27)
    dt = torch.bfloat16
    state = to_dev(w.s0, torch.float32).clone()
    od = kda.kda_decode_step(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                             to_dev(w.beta, torch.float32), state, 1.0)
    op, sp, _ = kda.kda_chunk_fwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                                  to_dev(w.beta, torch.float32), list(range(17)), 1.0,
                                  to_dev(w.s0, torch.float32))
    torch.cuda.synchronize()
    # decode is fp32 arithmetic on exact inputs; the prefill is the bf16-operand path:
    # both meet their bar against the oracle, and agree with each other to the bf16 bar
    o_r, s_r = oracle.decode(w.q, w.k, w.v, w.g, w.beta, w.s0, 1.0)
    assert W.rel_max_err(od.cpu().numpy(), o_r) <= TOL["f32"]
    assert W.rel_max_err(state.cpu().numpy(), s_r) <= TOL["f32"]
    assert W.rel_max_err(op.cpu().numpy(), o_r) <= TOL["bf16"]
    assert W.rel_max_err(sp.cpu().numpy(), s_r) <= TOL["bf16"]
    assert W.rel_max_err(op.cpu().numpy(), od.cpu().numpy()) <= TOL["bf16"]
    assert W.rel_max_err(sp.cpu().numpy(), state.cpu().numpy()) <= TOL["bf16"]


@pytest.mark.parametrize("chunk", CHUNKS)
def test_bitwise_determinism_and_state_aliasing(chunk):
    """Two runs give bit-identical outputs; final_state may alias initial_state."""
    w = W.make_prefill([300, 77], H=2, dk=128, dv=128, dtype="bf16", seed=28, s0_std=0.1)
    a = run_gpu(w, chunk=chunk)
    b = run_gpu(w, chunk=chunk)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # in-place state: pass the same buffer as initial and final state
    dt = torch.bfloat16
    S = to_dev(w.s0, torch.float32).clone()
    args = [to_dev(x, dt) for x in (w.q, w.k, w.v)] + [to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32)]
    cu_h = torch.tensor(list(w.cu_seqlens), dtype=torch.int32)
    o = torch.empty((w.total_tokens, 2, 128), dtype=torch.float32, device=dev())
    cu_d = cu_h.to(dev())   # must stay alive until the launch has been enqueued
    A = kda.make_fwd_args(*args, cu_d, cu_h, 1.0, S, S, 0, None, o, chunk)
    ws = torch.empty(kda.lib().kda_chunk_fwd_workspace_bytes(kda.ctypes.byref(A)), dtype=torch.uint8, device=dev())
    st = kda.lib().kda_chunk_fwd(kda.ctypes.byref(A), kda.ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                 kda._stream(None))
    assert st == kda.KDA_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S.cpu().numpy(), a[1])
    np.testing.assert_array_equal(o.cpu().numpy(), a[0])


# ---- paged state pool ---------------------------------------------------------------------------
def _log(label, errs, tol):
    print(f"[parity] {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": label, "tol": tol, **errs}) + "\n")
    for k_, v_ in errs.items():
        assert v_ <= tol, (k_, v_, tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_paged_pool(dtype):
    """Decode on a pool of 2N+1 slots: distinct random slots, two inactive sequences (-1 and an
    index past the pool).  Active slots match the oracle; every other slot is bit-unchanged and
    inactive sequences read o = 0."""
    d = W.make_decode(12, 5, 128, 128, dtype, seed=41)
    N, P = 12, 25
    rng = np.random.default_rng(41)
    slots = rng.permutation(P)[:N].astype(np.int32)
    slots[3], slots[9] = -1, P + 4
    pool = (0.1 * rng.standard_normal((P, 5, 128, 128))).astype(np.float32)
    dt = in_dtype(d)
    pool_d = to_dev(pool, torch.float32)
    o = kda.kda_decode_step(to_dev(d.q, dt), to_dev(d.k, dt), to_dev(d.v, dt), to_dev(d.g, torch.float32),
                            to_dev(d.beta, torch.float32), pool_d, 0.9,
                            state_indices=to_dev(slots, torch.int32))
    torch.cuda.synchronize()
    o_r, pool_r = oracle.decode_paged(d.q, d.k, d.v, d.g, d.beta, pool, slots, 0.9)
    o, pool_g = o.cpu().numpy(), pool_d.cpu().numpy()
    act = [n for n in range(N) if 0 <= slots[n] < P]
    touched = slots[act]
    _log(f"decode paged {dtype}", {"o": W.rel_max_err(o[act], o_r[act]),
                                   "S": W.rel_max_err(pool_g[touched], pool_r[touched])}, 1e-4)
    assert not o[[3, 9]].any()
    rest = [s for s in range(P) if s not in set(touched.tolist())]
    np.testing.assert_array_equal(pool_g[rest], pool[rest])


@pytest.mark.parametrize("chunk", CHUNKS)
def test_prefill_paged_pool(chunk):
    """Prefill with initial states gathered from pool slots (one -1: zeros) and checkpoints
    scattered to pool slots (some -1: not kept), as for prefix reuse at checkpoint boundaries."""
    w = W.make_prefill([200, 64, 130, 333], H=3, dk=128, dv=128, dtype="bf16", seed=42, s0_std=0.1,
                       checkpoint_every=64)
    N, P = 4, 16
    M = sum(L // 64 for L in w.seqlens)                     # 3 + 1 + 2 + 5 = 11 checkpoints
    rng = np.random.default_rng(42)
    pool = (0.1 * rng.standard_normal((P, 3, 128, 128))).astype(np.float32)
    sidx = np.array([5, -1, 11, 2], dtype=np.int32)
    cidx = np.array([0, 1, -1, 3, 4, -1, 6, 7, 8, 9, 10], dtype=np.int32)[:M]   # slots 0..10 minus two
    assert not set(sidx[sidx >= 0]) & set(cidx[cidx >= 0])
    dt = in_dtype(w)
    pool_d = to_dev(pool, torch.float32)
    o, sf, _ = kda.kda_chunk_fwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                                 to_dev(w.beta, torch.float32), list(w.cu_seqlens), 1.0, None, True, 64,
                                 chunk_size=chunk, initial_state_indices=to_dev(sidx, torch.int32),
                                 state_pool=pool_d, checkpoint_indices=to_dev(cidx, torch.int32))
    torch.cuda.synchronize()
    o_r, sf_r, pool_r = oracle.forward_paged(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 1.0, pool, sidx, 64, cidx)
    pool_g = pool_d.cpu().numpy()
    written = cidx[cidx >= 0]
    _log(f"prefill paged C={chunk}", {"o": W.rel_max_err(o.cpu().numpy(), o_r),
                                      "S": W.rel_max_err(sf.cpu().numpy(), sf_r),
                                      "ckpt": W.rel_max_err(pool_g[written], pool_r[written])}, TOL["bf16"])
    rest = [s for s in range(P) if s not in set(written.tolist())]
    np.testing.assert_array_equal(pool_g[rest], pool[rest])


@pytest.mark.parametrize("chunk", CHUNKS)
def test_paged_pool_through_the_prologue(chunk):
    """The pool and the prologue together, as a serving loop would use them: a prefill with raw
    inputs (gate pre-activations, q and k normalised inside) whose initial states come from pool
    slots and whose checkpoints go to pool slots, then one decode step through the same prologue
    on slots the prefill wrote (and one inactive sequence), against the oracle's prologue +
    forward_paged + decode_paged."""
    w = W.make_prefill_raw([200, 64, 130, 333], H=3, dk=128, dv=128, seed=43, checkpoint_every=64)
    P, scale = 16, 128 ** -0.5
    M = sum(L // 64 for L in w.seqlens)
    rng = np.random.default_rng(43)
    pool = (0.1 * rng.standard_normal((P, 3, 128, 128))).astype(np.float32)
    sidx = np.array([5, -1, 11, 2], dtype=np.int32)
    cidx = np.array([0, 1, -1, 3, 4, -1, 6, 7, 8, 9, 10], dtype=np.int32)[:M]
    bf = torch.bfloat16
    pool_d = to_dev(pool, torch.float32)
    pro = dict(gate_preactivation=True, normalize_qk=True)
    o, sf, _ = kda.kda_chunk_fwd(to_dev(w.q, bf), to_dev(w.k, bf), to_dev(w.v, bf), to_dev(w.g, bf),
                                 to_dev(w.beta, torch.float32), list(w.cu_seqlens), scale, None, True, 64,
                                 chunk_size=chunk, initial_state_indices=to_dev(sidx, torch.int32),
                                 state_pool=pool_d, checkpoint_indices=to_dev(cidx, torch.int32), **pro)
    # decode: sequences on slots 3 and 10 (written above), 6, and one inactive
    wd = W.make_prefill_raw([1] * 4, H=3, dk=128, dv=128, seed=44)
    slots = np.array([3, 10, -1, 6], dtype=np.int32)
    od = kda.kda_decode_step(to_dev(wd.q, bf), to_dev(wd.k, bf), to_dev(wd.v, bf), to_dev(wd.g, bf),
                             to_dev(wd.beta, torch.float32), pool_d, scale,
                             state_indices=to_dev(slots, torch.int32), **pro)
    torch.cuda.synchronize()
    qn, kn, g64, b64 = oracle.prologue(w.q, w.k, w.g, w.beta, True)
    o_r, sf_r, pool_r = oracle.forward_paged(qn, kn, w.v, g64, b64, w.cu_seqlens, scale, pool, sidx, 64, cidx)
    qd, kd, gd, bd = oracle.prologue(wd.q, wd.k, wd.g, wd.beta, True)
    od_r, pool_r2 = oracle.decode_paged(qd, kd, wd.v, gd, bd, pool_r, slots, scale)
    pool_g = pool_d.cpu().numpy()
    touched = sorted(set(cidx[cidx >= 0].tolist()) | set(slots[slots >= 0].tolist()))
    _log(f"paged + prologue C={chunk}", {"o": W.rel_max_err(o.cpu().numpy(), o_r),
                                         "S": W.rel_max_err(sf.cpu().numpy(), sf_r),
                                         "pool": W.rel_max_err(pool_g[touched], pool_r2[touched]),
                                         "o_dec": W.rel_max_err(od.cpu().numpy(), od_r)}, TOL["bf16"])
    assert np.all(od.cpu().numpy()[2] == 0)
    rest = [s_ for s_ in range(P) if s_ not in touched]
    np.testing.assert_array_equal(pool_g[rest], pool[rest])


# ---- fused gate / normalisation prologue ---------------------------------------------------------
@pytest.mark.parametrize("gate,norm,d,chunk", [(True, True, 128, 32), (True, False, 128, 32),
                                              (False, True, 128, 32), (True, True, 64, 32),
                                              (True, True, 128, 64), (True, False, 64, 64),
                                              (False, True, 64, 64)])
def test_prefill_fused_prologue(gate, norm, d, chunk):
    """The gate (g = -5 sigmoid(a) from bf16 a, beta = sigmoid(b)) and/or the L2 normalisation
    of q, k, against the oracle's prologue + recurrence: fused into the first stage at chunk 32
    and d = 128, a pass of its own at the other shapes.  Ragged sequences, initial states,
    checkpoints every 64."""
    w = W.make_prefill_raw([200, 1, 0, 130, 333], H=3, dk=d, dv=d, seed=51, s0_std=0.1,
                           checkpoint_every=64)
    scale = d ** -0.5
    qn, kn, g64, b64 = oracle.prologue(w.q, w.k, w.g, w.beta, normalize=norm)
    if not norm:
        # unnormalised q, k would make the recurrence blow up: use unit rows (still bf16-exact)
        qn = W.round_bf16((w.q / np.linalg.norm(w.q, axis=-1, keepdims=True)).astype(np.float32))
        kn = W.round_bf16((w.k / np.linalg.norm(w.k, axis=-1, keepdims=True)).astype(np.float32))
    q_in, k_in = (w.q, w.k) if norm else (qn, kn)
    if gate:
        g_in, b_in = to_dev(w.g, torch.bfloat16), to_dev(w.beta, torch.float32)
        g_ref, b_ref = g64, b64
    else:
        g32, b32 = g64.astype(np.float32), b64.astype(np.float32)
        g_in, b_in = to_dev(g32, torch.float32), to_dev(b32, torch.float32)
        g_ref, b_ref = g32, b32
    o, sf, ck = kda.kda_chunk_fwd(to_dev(q_in, torch.bfloat16), to_dev(k_in, torch.bfloat16),
                                  to_dev(w.v, torch.bfloat16), g_in, b_in, list(w.cu_seqlens), scale,
                                  to_dev(w.s0, torch.float32), True, 64, chunk_size=chunk,
                                  gate_preactivation=gate, normalize_qk=norm)
    torch.cuda.synchronize()
    o_r, sf_r, ck_r = oracle.forward(qn, kn, w.v, g_ref, b_ref, w.cu_seqlens, scale, w.s0, checkpoint_every=64)
    _log(f"fused prologue gate={gate} norm={norm} d={d} C={chunk}",
         {"o": W.rel_max_err(o.cpu().numpy(), o_r), "S": W.rel_max_err(sf.cpu().numpy(), sf_r),
          "ckpt": W.rel_max_err(ck.cpu().numpy(), ck_r)}, TOL["bf16"])


def test_gate_decay_of_every_bf16_value():
    """The fused gate's decay alpha = exp(-5 sigmoid(a)) for every bf16 pre-activation a (NaNs aside):
    one token per chain with k = q = v = 0, beta = sigmoid(-1e30) = 0 and S0 = 1 leaves
    S_1 = Diag(alpha) S0, so the final state reads alpha out exactly.  With 128 chains the kernel
    runs two workgroups per chain, which look alpha up in a table in LDS; a second token per head in
    a second sequence makes 256 chains, one workgroup each, which form alpha arithmetically.  The two
    must agree bit for bit, and both lie within 1e-6 (8 ulp: three approximate fp32 transcendentals)
    of exp(-5 sigmoid(a)) in fp64 (the gate of the
    skill card's quick facts: scaled sigmoid, g >= -5)."""
    if torch.cuda.get_device_properties(0).multi_processor_count < 256:
        pytest.skip("the one- and two-workgroup kernels are chosen for a 256-CU device")
    bits = np.arange(1 << 16, dtype=np.uint32)
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    bits = bits[~((e == 0xFF) & (m != 0))].astype(np.uint16)
    H, D, blk = 128, 128, 128 * 128
    bits = np.concatenate([bits, bits[: (-len(bits)) % blk]])
    ref_all = -5.0 / (1.0 + np.exp(-(bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)))
    ref_all = np.exp(ref_all)
    z = torch.zeros((2, H, D), dtype=torch.bfloat16, device="cuda")
    b = torch.full((2, H), -1e30, dtype=torch.float32, device="cuda")
    s0 = torch.ones((2, H, D, D), dtype=torch.float32, device="cuda")
    worst = 0.0
    for i in range(0, len(bits), blk):
        a1 = torch.from_numpy(bits[i:i + blk].view(np.int16).copy()).view(torch.bfloat16).reshape(1, H, D).cuda()
        a2 = torch.cat([a1, a1])
        _, sf1, _ = kda.kda_chunk_fwd(z[:1], z[:1], z[:1], a1, b[:1], [0, 1], 1.0, s0[:1], gate_preactivation=True)
        _, sf2, _ = kda.kda_chunk_fwd(z, z, z, a2, b, [0, 1, 2], 1.0, s0, gate_preactivation=True)
        torch.cuda.synchronize()
        t1, t2 = sf1[0].cpu().numpy(), sf2[0].cpu().numpy()
        assert np.all(t1 == t1[..., :1]) and np.all(t2 == t2[..., :1]), "S_1 rows are alpha times ones"
        np.testing.assert_array_equal(t1[..., 0].ravel().view(np.uint32), t2[..., 0].ravel().view(np.uint32))
        ref = ref_all[i:i + blk]
        worst = max(worst, float(np.max(np.abs(t1[..., 0].ravel() - ref) / ref)))
    print(f"gate decay over {len(bits)} bf16 values: table == arithmetic, worst relative error {worst:.2e}",
          flush=True)
    assert worst <= 1e-6


@pytest.mark.parametrize("segment_tokens", [-1, 64])
def test_prefill_fused_normalisation_edge_rows(segment_tokens):
    """The fused normalisation (role waves: the rows' sums of squares from the diagonal of their Gram
    product) on edge rows: a zero q row and a zero k row (they stay zero), rows scaled by 2^-40 and
    2^40 (exact in bf16; their squares stay normal in fp32), in chunks 0, 1 and the ragged last one,
    uncut and cut into segments."""
    w = W.make_prefill_raw([150, 70], H=2, dk=128, dv=128, seed=57, s0_std=0.1)
    q, k = w.q.copy(), w.k.copy()
    q[3, 1] = 0.0
    k[40, 0] = 0.0
    q[33, 0] *= np.float32(2.0 ** -40)
    k[34, 1] *= np.float32(2.0 ** 40)
    k[149, 0] *= np.float32(2.0 ** -40)
    q[160, 1] *= np.float32(2.0 ** 40)
    k[219, 1] = 0.0
    scale = 128 ** -0.5
    qn, kn, g64, b64 = oracle.prologue(q, k, w.g, w.beta, normalize=True)
    o, sf, _ = kda.kda_chunk_fwd(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(w.v, torch.bfloat16),
                                 to_dev(w.g, torch.bfloat16), to_dev(w.beta, torch.float32), list(w.cu_seqlens),
                                 scale, to_dev(w.s0, torch.float32), True, chunk_size=32, gate_preactivation=True,
                                 normalize_qk=True, segment_tokens=segment_tokens)
    torch.cuda.synchronize()
    o_r, sf_r, _ = oracle.forward(qn, kn, w.v, g64, b64, w.cu_seqlens, scale, w.s0)
    o_g = o.cpu().numpy()
    assert np.all(o_g[3, 1] == 0.0)   # a zero query row reads nothing
    _log(f"fused normalisation edge rows seg={segment_tokens}",
         {"o": W.rel_max_err(o_g, o_r), "S": W.rel_max_err(sf.cpu().numpy(), sf_r)}, TOL["bf16"])


# ---- context parallelism: one GPU's share and the combine ----------------------------------------
def test_context_parallel_segments_combine():
    """One 512-token sequence cut into 4 segments, as 4 GPUs would hold it: each segment runs from
    S0 = 0 (outputs o0, final state N_p) and, with v = 0, from S0 = I (outputs oI = scale M_t^T q_t,
    final state M_p: the identity-column augmentation, d_v = d_k).  The states entering the
    segments follow S_in(p+1) = M_p S_in(p) + N_p (the exchange step) and o = o0 + S_in^T oI;
    the result must match the oracle on the unsplit sequence.  Slow decay, so the carried state
    matters."""
    P, Lseg, H, d = 4, 128, 2, 128
    w = W.make_prefill([P * Lseg], H=H, dk=d, dv=d, dtype="bf16", seed=81, s0_std=0.1, gate="slow")
    cu = [p * Lseg for p in range(P + 1)]
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    q, k, v = to_dev(w.q, bf), to_dev(w.k, bf), to_dev(w.v, bf)
    g, b = to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32)
    s0 = torch.zeros((P, H, d, d), dtype=torch.float32, device=dev)
    o0, n_p, _ = kda.kda_chunk_fwd(q, k, v, g, b, cu, 1.0, s0)
    eye = torch.eye(d, dtype=torch.float32, device=dev).expand(P, H, d, d).contiguous()
    oI, m_p, _ = kda.kda_chunk_fwd(q, k, torch.zeros_like(v), g, b, cu, 1.0, eye)
    torch.cuda.synchronize()
    o0, oI, n_p, m_p = (x.double().cpu() for x in (o0, oI, n_p, m_p))
    s_in = torch.from_numpy(w.s0[0]).double()                       # [H, d, d]
    o = torch.empty_like(o0)
    carried = 0.0
    for p in range(P):
        sl = slice(p * Lseg, (p + 1) * Lseg)
        corr = torch.einsum("thi,hij->thj", oI[sl], s_in)              # S_in^T oI per token
        o[sl] = o0[sl] + corr
        carried = max(carried, float(corr.abs().max() / o0[sl].abs().max()))
        s_in = torch.einsum("hij,hjk->hik", m_p[p], s_in) + n_p[p]
    o_r, s_r, _ = oracle.forward(w.q, w.k, w.v, w.g, w.beta, [0, P * Lseg], 1.0, w.s0)
    _log("context parallel, 4 segments x 128", {"o": W.rel_max_err(o.numpy(), o_r),
                                                "S": W.rel_max_err(s_in.numpy()[None], s_r)}, TOL["bf16"])
    assert carried > 0.05, carried   # the segments really depend on the state handed over


# ---- graph capture --------------------------------------------------------------------------------
def test_graph_capture_and_replay():
    """A prefill and a decode step through the C ABI captured into one HIP graph (arguments and
    buffers prepared before the capture, nothing allocated or cleared inside the calls), replayed
    three times with eager work and synchronisations between replays: every replay reproduces
    the eager result bit for bit."""
    import ctypes
    L = kda.lib()
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    w = W.make_prefill([300, 77], H=4, dk=128, dv=128, dtype="bf16", seed=91, s0_std=0.1)
    d = W.make_decode(16, 4, 128, 128, "bf16", seed=92)
    q, k, v = to_dev(w.q, bf), to_dev(w.k, bf), to_dev(w.v, bf)
    g, b, s0 = to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32), to_dev(w.s0, torch.float32)
    cu_h = torch.tensor(list(w.cu_seqlens), dtype=torch.int32)
    cu_d = cu_h.to(dev)
    o = torch.empty((w.total_tokens, 4, 128), dtype=torch.float32, device=dev)
    sf = torch.empty_like(s0)
    A = kda.make_fwd_args(q, k, v, g, b, cu_d, cu_h, 1.0, s0, sf, 0, None, o, 32)
    ws = torch.empty(max(256, L.kda_chunk_fwd_workspace_bytes(ctypes.byref(A))), dtype=torch.uint8, device=dev)
    dq, dk_, dv_ = to_dev(d.q, bf), to_dev(d.k, bf), to_dev(d.v, bf)
    dg, db = to_dev(d.g, torch.float32), to_dev(d.beta, torch.float32)
    state0 = to_dev(d.s0, torch.float32)
    state = state0.clone()
    od = torch.empty((16, 4, 128), dtype=torch.float32, device=dev)
    D = kda.make_decode_args(dq, dk_, dv_, dg, db, state, od, 1.0)

    def step(stream):
        sp = ctypes.c_void_p(stream.cuda_stream)
        assert L.kda_chunk_fwd(ctypes.byref(A), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), sp) == 0
        assert L.kda_decode_step(ctypes.byref(D), sp) == 0

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, sf, od, state)]
    graph = torch.cuda.CUDAGraph()
    state.copy_(state0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    for rep in range(3):
        o.zero_(); sf.zero_(); od.zero_()
        state.copy_(state0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("o", "final_state", "o_decode", "state"), (o, sf, od, state), ref):
            assert torch.equal(x, y), (rep, name)
    print("[graph] prefill + decode captured; 3 replays equal to the eager result", flush=True)
