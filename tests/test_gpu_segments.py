"""GPU parity of the forward with its sequences cut into segments that run side by side
(kda_fwd_args.segment_tokens): every segment runs from zero and, as a transition run, from the
identity with v = 0 (its affine map S_t = M_t S_in + N_t and the outputs' part scale M_t^T q_t), a
chain along each sequence gives every segment's initial state S_in, its checkpoints and the final
state, and the later segments' outputs are corrected by S_in^T (scale M_t^T q_t).  Same metric and
bars as the other parity tests (max|gpu - oracle| / RMS(oracle): 1e-4 fp32 inputs, 2e-2 bf16
inputs), against the fp64 oracle on the uncut sequences.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import oracle
import workloads as W
from test_gpu_parity import TOL, _log, in_dtype, to_dev

pytestmark = pytest.mark.gpu


def run(w, seg, scale=1.0, **kw):
    dt = in_dtype(w)
    o, sf, ck = kda.kda_chunk_fwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                                  to_dev(w.beta, torch.float32), list(w.cu_seqlens), scale,
                                  None if w.s0 is None else to_dev(w.s0, torch.float32), True, w.checkpoint_every,
                                  chunk_size=32, segment_tokens=seg, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), sf.cpu().numpy(), None if ck is None else ck.cpu().numpy()


def check(w, seg, label, scale=1.0):
    o, sf, ck = run(w, seg, scale)
    o_r, s_r, ck_r = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, scale, w.s0, w.checkpoint_every)
    errs = {"o": W.rel_max_err(o, o_r), "S": W.rel_max_err(sf, s_r)}
    if ck_r is not None and ck_r.size:
        errs["ckpt"] = W.rel_max_err(ck, ck_r)
    _log(f"segments {label} seg={seg} {w.dtype} d={w.dk}", errs, TOL[w.dtype])
    return o, sf, ck


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segments_ragged(d, dtype):
    """Ragged lengths (an empty sequence, a one-token one, a last segment shorter than the rest),
    initial states, checkpoints every 64 tokens: 128-token segments."""
    w = W.make_prefill([1000, 0, 1, 130, 700], H=3, dk=d, dv=d, dtype=dtype, seed=91, s0_std=0.1,
                       checkpoint_every=64)
    check(w, 128, "ragged")


def test_segments_slow_decay_long_chain():
    """Slow decay (the maps M stay close to the identity, the carried state matters over the
    whole sequence): 8192 tokens in 16 segments, fp32 inputs, the fp32 bar."""
    w = W.make_prefill([8192], H=2, dk=64, dv=64, dtype="f32", seed=92, s0_std=0.1, gate="slow")
    check(w, 512, "slow decay")


@pytest.mark.parametrize("gate", ["min", "zero"])
def test_segments_gate_extremes(gate):
    """g = -5 (every map nearly annihilates what it carries) and g = 0 (no decay: the maps are
    products of projections only)."""
    w = W.make_prefill([2000, 300], H=2, dk=128, dv=128, dtype="bf16", seed=93, s0_std=0.1, gate=gate)
    check(w, 256, f"gate={gate}")


def test_segments_one_segment_each():
    """A segment longer than every sequence gives one segment each: every sequence runs once, from
    its initial state, in the paired launch (one workgroup per run), its final state moved verbatim
    by the chain.  Against the oracle, and against the uncut forward (which may split each run over
    two workgroups: the same arithmetic in another order) within the fp32-input bar."""
    w = W.make_prefill([300, 700, 64], H=2, dk=128, dv=128, dtype="bf16", seed=94, s0_std=0.1, checkpoint_every=64)
    o1, s1, c1 = check(w, 1024, "one segment each")
    o0, s0, c0 = run(w, -1)
    errs = {"o": W.rel_max_err(o1, o0), "S": W.rel_max_err(s1, s0), "ckpt": W.rel_max_err(c1, c0)}
    _log("segments one each vs uncut", errs, TOL["f32"])


def test_segments_pool_and_prologue():
    """Initial states from pool slots (one -1: zeros), checkpoints to pool slots (some -1), and the
    fused prologue (gate pre-activations, q and k normalised inside), cut into 64-token segments."""
    w = W.make_prefill_raw([200, 64, 130, 333], H=3, dk=128, dv=128, seed=95, checkpoint_every=64)
    P, scale = 16, 128 ** -0.5
    M = sum(L // 64 for L in w.seqlens)
    rng = np.random.default_rng(95)
    pool = (0.1 * rng.standard_normal((P, 3, 128, 128))).astype(np.float32)
    sidx = np.array([5, -1, 11, 2], dtype=np.int32)
    cidx = np.array([0, 1, -1, 3, 4, -1, 6, 7, 8, 9, 10], dtype=np.int32)[:M]
    bf = torch.bfloat16
    pool_d = to_dev(pool, torch.float32)
    o, sf, _ = kda.kda_chunk_fwd(to_dev(w.q, bf), to_dev(w.k, bf), to_dev(w.v, bf), to_dev(w.g, bf),
                                 to_dev(w.beta, torch.float32), list(w.cu_seqlens), scale, None, True, 64,
                                 chunk_size=32, initial_state_indices=to_dev(sidx, torch.int32),
                                 state_pool=pool_d, checkpoint_indices=to_dev(cidx, torch.int32),
                                 gate_preactivation=True, normalize_qk=True, segment_tokens=64)
    torch.cuda.synchronize()
    qn, kn, g64, b64 = oracle.prologue(w.q, w.k, w.g, w.beta, True)
    o_r, sf_r, pool_r = oracle.forward_paged(qn, kn, w.v, g64, b64, w.cu_seqlens, scale, pool, sidx, 64, cidx)
    pool_g = pool_d.cpu().numpy()
    written = cidx[cidx >= 0]
    _log("segments pool + prologue seg=64", {"o": W.rel_max_err(o.cpu().numpy(), o_r),
                                             "S": W.rel_max_err(sf.cpu().numpy(), sf_r),
                                             "ckpt": W.rel_max_err(pool_g[written], pool_r[written])},
         TOL["bf16"])
    rest = [s for s in range(P) if s not in set(written.tolist())]
    np.testing.assert_array_equal(pool_g[rest], pool[rest])


def test_segments_aliased_state_and_determinism():
    """final_state may alias initial_state (every initial state is read before any final state is
    written); two runs give the same bits."""
    w = W.make_prefill([900, 250], H=2, dk=128, dv=128, dtype="bf16", seed=96, s0_std=0.1)
    dt = in_dtype(w)
    args = [to_dev(x, dt) for x in (w.q, w.k, w.v)] + [to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32)]
    o1, sf1, _ = kda.kda_chunk_fwd(*args, list(w.cu_seqlens), 1.0, to_dev(w.s0, torch.float32), True,
                                   segment_tokens=128)
    o2, sf2, _ = kda.kda_chunk_fwd(*args, list(w.cu_seqlens), 1.0, to_dev(w.s0, torch.float32), True,
                                   segment_tokens=128)
    # in place: the state buffer is both the initial and the final state
    st = to_dev(w.s0, torch.float32)
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32)
    o3 = torch.empty_like(o1)
    a = kda.make_fwd_args(*args, cu.to(st.device), cu, 1.0, st, st, 0, None, o3, segment_tokens=128)
    ws = torch.empty(max(int(kda.lib().kda_chunk_fwd_workspace_bytes(kda.ctypes.byref(a))), 256),
                     dtype=torch.uint8, device=st.device)
    kda._check(kda.lib().kda_chunk_fwd(kda.ctypes.byref(a), kda.ctypes.c_void_p(ws.data_ptr()),
                                       kda.ctypes.c_size_t(ws.numel()), None))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(sf1, sf2)
    assert torch.equal(o3, o1) and torch.equal(st, sf1)
    o_r, s_r, _ = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 1.0, w.s0)
    _log("segments aliased", {"o": W.rel_max_err(o1.cpu().numpy(), o_r),
                              "S": W.rel_max_err(sf1.cpu().numpy(), s_r)}, TOL["bf16"])


def test_segments_library_choice_at_4096_tokens_32_heads():
    """The chained prefill shape (one 4,096-token sequence, 32 heads, d = 128, bf16): the library
    cuts it by itself (segment_tokens 0; its workspace then holds the segments' states), and
    every head's o and final state match the oracle on two heads computed one by one; the uncut
    run matches too."""
    w = W.make_prefill([4096], H=32, dk=128, dv=128, dtype="bf16", seed=97, s0_std=0.1)
    dt = in_dtype(w)
    args = [to_dev(x, dt) for x in (w.q, w.k, w.v)] + [to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32)]
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32)

    def ws_bytes(seg):
        a = kda.make_fwd_args(*args, cu.to(args[0].device), cu, 1.0, None, None, 0, None,
                              torch.empty((4096, 32, 128), device=args[0].device), segment_tokens=seg)
        return int(kda.lib().kda_chunk_fwd_workspace_bytes(kda.ctypes.byref(a)))

    assert ws_bytes(0) > ws_bytes(-1) + 4 * 32 * 128 * 128 * 4   # the library cut the sequence
    res = {}
    for seg in (0, -1):
        o, sf, _ = kda.kda_chunk_fwd(*args, list(w.cu_seqlens), 1.0, to_dev(w.s0, torch.float32), True,
                                     segment_tokens=seg)
        torch.cuda.synchronize()
        res[seg] = (o.cpu().numpy(), sf.cpu().numpy())
    for h in (0, 31):
        sl = lambda x: np.ascontiguousarray(x[:, h:h + 1])
        o_r, s_r, _ = oracle.forward(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), w.cu_seqlens, 1.0,
                                     np.ascontiguousarray(w.s0[:, h:h + 1]))
        for seg, (o, sf) in res.items():
            _log(f"segments 4096x32 head {h} seg={seg}", {"o": W.rel_max_err(o[:, h:h + 1], o_r),
                                                          "S": W.rel_max_err(sf[:, h:h + 1], s_r)}, TOL["bf16"])
