"""GPU parity of the backward (kda_chunk_bwd through the C ABI) against the fp64 oracle adjoint
(oracle.backward.backward), per gradient: max|gpu - oracle| / RMS(oracle) over the whole tensor.
Bars as for the forward, 1e-4 with fp32 inputs and 2e-2 with bf16 inputs, except dg on the fp32
path, whose bar is derived per case: dg_t = alpha_t * rowsum(dS~ * S_{t-1}) sums d_v terms that
are much larger than the result, so a relative error eps in the fp32 states and state gradients
reaches dg as eps * amp, amp_t = alpha_t * rowsum(|dS~ * S_{t-1}|) (the oracle's amplification
output).  The bar is max(1e-4, 4 * EPS_STATE_F32 * max(amp) / RMS(dg)) with EPS_STATE_F32 =
2e-6, the fp32 forward's measured state error (max|diff| / RMS of the final states, <= 2e-6 in
the fp32 parity cases)."""
import json
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import oracle
import workloads as W
from oracle import backward as OB
from parity_helpers import identity_bar

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
EPS_STATE_F32 = 2e-6
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def to_dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.device("cuda:0"), dt)


def run_bwd(w, do, dsf, scale=1.0, s0=True, **kw):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    outs = kda.kda_chunk_bwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                             to_dev(w.beta, torch.float32), to_dev(do, torch.float32), list(w.cu_seqlens), scale,
                             to_dev(w.s0, torch.float32) if (s0 and w.s0 is not None) else None,
                             None if dsf is None else to_dev(dsf, torch.float32), **kw)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in outs]


def dg_bar(dtype, dg_ref, amp):
    """dg's bar for one case: the path's bar, or on the fp32 path the state error carried through
    the measured cancellation amplification max(amp) / RMS(dg) (see the module docstring)."""
    if dtype != "f32" or dg_ref.size == 0:
        return TOL[dtype], 0.0
    rms = float(np.sqrt(np.mean(np.asarray(dg_ref, dtype=np.float64) ** 2)))
    a = float(np.max(amp)) / rms if rms > 0 else 0.0
    return max(TOL["f32"], 4.0 * EPS_STATE_F32 * a), a


def check(w, do, dsf, scale=1.0, s0=True, label="", **kw):
    tol = TOL[w.dtype]
    got = run_bwd(w, do, dsf, scale, s0, **kw)
    *ref, amp = OB.backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, scale, w.s0 if s0 else None, do, dsf,
                            amplification=True)
    dg_tol, a = dg_bar(w.dtype, ref[3], amp)
    errs = {n: W.rel_max_err(a_, b) for n, a_, b in zip(NAMES, got, ref) if b.size}
    label = label or w.name
    print(f"[bwd parity] {label} seqlens={w.seqlens[:8]} H={w.H} d={w.dk} {w.dtype}: "
          + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
          + (f"  (dg bar {dg_tol:.2e} from amplification {a:.1f})" if w.dtype == "f32" else ""), flush=True)
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": "bwd " + label, "H": w.H, "d": w.dk, "dtype": w.dtype,
                                "tokens": w.total_tokens, "tol": tol, "dg_tol": dg_tol, "dg_amp": a, **errs}) + "\n")
    for k_, v_ in errs.items():
        assert v_ <= (dg_tol if k_ == "dg" else tol), (k_, v_)
    return got


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_varlen_ragged(d, dtype):
    # empty, one-token, exact-chunk, chunk - 3, chunk + 1 and multi-chunk sequences, initial and final states
    w = W.make_prefill([70, 0, 32, 29, 33, 1], H=2, dk=d, dv=d, dtype=dtype, seed=21, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=21)
    check(w, do, dsf, label=f"varlen d={d} {dtype}")


def test_backward_scale_no_states():
    w = W.make_prefill([45, 96], H=3, dk=64, dv=64, dtype="f32", seed=22)
    do, _ = W.make_cotangents(w, seed=22, d_final=False)
    check(w, do, None, scale=0.37, s0=False, label="scale 0.37, no S0 / dS_T")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_long_sequence(dtype):
    # 32 chunks through the reverse scan
    w = W.make_prefill([1000, 24], H=2, dk=128, dv=128, dtype=dtype, seed=23, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=23)
    check(w, do, dsf, label=f"long {dtype}")


def test_backward_many_chains():
    # 111 chains: the scan's workgroup-to-chain map has a partial last group of 8
    rng = np.random.default_rng(24)
    lens = [int(x) for x in rng.integers(1, 120, size=37)]
    w = W.make_prefill(lens, H=3, dk=64, dv=64, dtype="bf16", seed=24, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=24)
    check(w, do, dsf, label="37 seqs x 3 heads")


def test_backward_more_sequences_than_one_plan_tile():
    # 1500 sequences (lengths 0..70): the launch plan and the chunk bases span two tiles of 1024
    rng = np.random.default_rng(62)
    lens = [int(x) for x in rng.integers(0, 71, size=1500)]
    w = W.make_prefill(lens, H=1, dk=64, dv=64, dtype="bf16", seed=62, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=62)
    check(w, do, dsf, label="1500 sequences")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("given", [False, True])
def test_backward_in_groups_of_sequences(dtype, given):
    """With the least workspace the library accepts (the longest sequence's own), the batch runs as
    groups of whole sequences one after another: against the oracle at the usual bars, and
    bit-identical to the one-pass run (every chunk and chain takes the same arithmetic; both runs'
    forward recomputes split each chain over two workgroups, having fewer chains than half the
    compute units).  With given states, each group reads its own slice of them."""
    w = W.make_prefill([300, 0, 1000, 64, 33, 700], H=2, dk=128, dv=128, dtype=dtype, seed=29, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=29)
    kw = {}
    if given:
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        _, _, ck = kda.kda_chunk_fwd(to_dev(w.q, dt), to_dev(w.k, dt), to_dev(w.v, dt), to_dev(w.g, torch.float32),
                                     to_dev(w.beta, torch.float32), list(w.cu_seqlens), 1.0,
                                     to_dev(w.s0, torch.float32), False, 32, chunk_size=32, segment_tokens=-1)
        kw["states"] = ck
    got = check(w, do, dsf, label=f"groups {dtype} given={given}", workspace_cap=1, **kw)
    one = run_bwd(w, do, dsf, **kw)
    for n, a_, b_ in zip(NAMES, got, one):
        np.testing.assert_array_equal(a_, b_, err_msg=n)


@pytest.mark.parametrize("gate", ["min", "zero", "slow"])
def test_backward_gate_extremes(gate):
    w = W.make_prefill([100, 64], H=2, dk=128, dv=128, dtype="bf16", seed=25, s0_std=0.1, gate=gate)
    do, dsf = W.make_cotangents(w, seed=25)
    check(w, do, dsf, label=f"gate={gate}")


@pytest.mark.parametrize("lens", [[0, 5, 0], [0, 0]])
def test_backward_empty_sequences(lens):
    # an empty sequence passes its final-state gradient through: dS0 = dS_T
    w = W.make_prefill(lens, H=2, dk=64, dv=64, dtype="f32", seed=28, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=28)
    got = check(w, do, dsf, label=f"empty {lens}")
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(got[5][n], dsf[n])


@pytest.mark.parametrize("pro", [False, True])
def test_backward_from_the_forwards_states(pro):
    """The forward run with checkpoint_every = 32, its checkpoints passed to the backward instead
    of being recomputed: the same gradients as the recomputing backward (d = 128 bf16, ragged
    sequences, S0 and dS_T; with and without the fused prologue)."""
    lens = [200, 1, 0, 64, 95]
    if pro:
        w = W.make_prefill_raw(lens, H=3, dk=128, dv=128, seed=64, s0_std=0.1)
        g_in = to_dev(w.g, torch.bfloat16)
        scale = 128 ** -0.5
    else:
        w = W.make_prefill(lens, H=3, dk=128, dv=128, dtype="bf16", seed=64, s0_std=0.1)
        g_in = to_dev(w.g, torch.float32)
        scale = 1.0
    do, dsf = W.make_cotangents(w, seed=64)
    q, k, v = (to_dev(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    b, s0 = to_dev(w.beta, torch.float32), to_dev(w.s0, torch.float32)
    kw = dict(gate_preactivation=pro, normalize_qk=pro)
    _, _, ck = kda.kda_chunk_fwd(q, k, v, g_in, b, list(w.cu_seqlens), scale, s0, True, 32, chunk_size=32, **kw)
    assert ck.shape[0] == sum(L // 32 for L in lens)
    args = (q, k, v, g_in, b, to_dev(do, torch.float32), list(w.cu_seqlens), scale, s0, to_dev(dsf, torch.float32))
    ref = kda.kda_chunk_bwd(*args, **kw)
    got = kda.kda_chunk_bwd(*args, states=ck, **kw)
    torch.cuda.synchronize()
    errs = {n: W.rel_max_err(x.cpu().numpy(), y.cpu().numpy()) for n, x, y in zip(NAMES, got, ref)}
    print(f"[bwd parity] given states (prologue={pro}) vs recomputed: "
          + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    for k_, v_ in errs.items():
        assert v_ <= 1e-6, (k_, v_)


@pytest.mark.parametrize("given,lens", [(False, [150] * 4), (True, [150] * 4), (False, [150] * 4 + [0])])
def test_backward_one_workgroup_scan(given, lens):
    """A batch of equal-length sequences with enough chains to fill the chip (4 x 150 tokens, 24
    heads: 96 chains on 256 compute units, d = 128, bf16) takes the state-gradient scan with one
    workgroup per chain, which forms R = P^T dO itself (ragged last chunks, S0 and dS_T): against
    the oracle, and with the forward's states given, against the recomputing run.  That run
    recomputes the states beside the scan with one workgroup per chain (the forward took two) and
    hi/lo products for (Gamma K) S, whose R = V - (Gamma K) S it hands to the gradient kernel, so
    the two agree to the states' rounding, not bit for bit: the bar, 1e-4 of each gradient's RMS,
    is 200 times below the bf16 bar (wrong states would miss it by orders of magnitude).  With one more, empty sequence the batch still takes it (the longest is 5/4 of
    the mean): that chain's dS0 is its dS_T."""
    w = W.make_prefill(lens, H=24, dk=128, dv=128, dtype="bf16", seed=31, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=31)
    kw = {}
    if given:
        _, _, ck = kda.kda_chunk_fwd(to_dev(w.q, torch.bfloat16), to_dev(w.k, torch.bfloat16),
                                     to_dev(w.v, torch.bfloat16), to_dev(w.g, torch.float32),
                                     to_dev(w.beta, torch.float32), list(w.cu_seqlens), 1.0,
                                     to_dev(w.s0, torch.float32), False, 32, chunk_size=32)
        kw["states"] = ck
    got = check(w, do, dsf, label=f"one-workgroup scan given={given} seqs={len(lens)}", **kw)
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(got[5][n], dsf[n])
    if given:
        ref = run_bwd(w, do, dsf)
        errs = {n: W.rel_max_err(a_, b_) for n, a_, b_ in zip(NAMES, got, ref)}
        print("[bwd parity] given states vs recomputed beside the scan: "
              + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        for k_, v_ in errs.items():
            assert v_ <= 1e-4, (k_, v_)


def test_backward_one_workgroup_scan_fused_prologue():
    """The one-workgroup scan through the fused gate and normalisation (fp32 unit vectors, the
    bf16 error budget): 4 x 150 tokens, 24 heads, d = 128, against the oracle's backward through
    the same prologue."""
    w = W.make_prefill_raw([150] * 4, H=24, dk=128, dv=128, seed=53, s0_std=0.1)
    scale = 128 ** -0.5
    do, dsf = W.make_cotangents(w, seed=53)
    outs = kda.kda_chunk_bwd(to_dev(w.q, torch.bfloat16), to_dev(w.k, torch.bfloat16), to_dev(w.v, torch.bfloat16),
                             to_dev(w.g, torch.bfloat16), to_dev(w.beta, torch.float32), to_dev(do, torch.float32),
                             list(w.cu_seqlens), scale, to_dev(w.s0, torch.float32), to_dev(dsf, torch.float32),
                             gate_preactivation=True, normalize_qk=True)
    torch.cuda.synchronize()
    got = [x.cpu().numpy() for x in outs]
    ref = OB.backward_fused(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, scale, w.s0, do, dsf, normalize=True, gate=True)
    errs = {n: W.rel_max_err(x, y) for n, x, y in zip(NAMES, got, ref)}
    print("[bwd parity] one-workgroup scan, fused prologue: " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()),
          flush=True)
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], (k_, v_)


def test_backward_deterministic():
    w = W.make_prefill([150, 77], H=4, dk=128, dv=128, dtype="bf16", seed=26, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=26)
    a = run_bwd(w, do, dsf)
    b = run_bwd(w, do, dsf)
    for n, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), n


def test_backward_T4096_H32_sampled_heads_and_linearity():
    """Chunked-prefill workload (one sequence, T = 4096, H = 32, d = 128, bf16): two heads
    against the oracle, and over all heads the identity that holds because o and S_T are linear
    in (S_0, v) jointly: sum(dv * v) + sum(dS0 * S0) = sum(d_o * o) + sum(dS_T * S_T)."""
    w = W.make_workload(1)
    do, dsf = W.make_cotangents(w, seed=27)
    dq, dk, dv, dg, db, ds0 = run_bwd(w, do, dsf)
    for x in (dq, dk, dv, dg, db, ds0):
        assert np.all(np.isfinite(x))
    heads = [0, 17]
    ref = OB.backward(w.q[:, heads], w.k[:, heads], w.v[:, heads], w.g[:, heads], w.beta[:, heads],
                      w.cu_seqlens, 1.0, None, do[:, heads], dsf[:, heads])
    errs = {n: W.rel_max_err(a[:, heads], b) for n, a, b in zip(NAMES, (dq, dk, dv, dg, db, ds0), ref)}
    print("[bwd parity] T=4096 H=32 heads", heads, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], (k_, v_)
    o, sf, _ = kda.kda_chunk_fwd(to_dev(w.q, torch.bfloat16), to_dev(w.k, torch.bfloat16),
                                 to_dev(w.v, torch.bfloat16), to_dev(w.g, torch.float32),
                                 to_dev(w.beta, torch.float32), list(w.cu_seqlens), 1.0, None)
    torch.cuda.synchronize()
    o_h, sf_h = o.cpu().numpy(), sf.cpu().numpy()
    o_r, s_r, _ = oracle.forward(w.q[:, heads], w.k[:, heads], w.v[:, heads], w.g[:, heads], w.beta[:, heads],
                                 w.cu_seqlens, 1.0, None, 0)
    errs_f = {"o": W.rel_max_err(o_h[:, heads], o_r), "S": W.rel_max_err(sf_h[:, heads], s_r)}
    lhs = float(np.sum(dv.astype(np.float64) * w.v))
    rhs = float(np.sum(do.astype(np.float64) * o_h) + np.sum(dsf.astype(np.float64) * sf_h))
    bar = identity_bar([(dv, w.v, errs["dv"]), (o_h, do, errs_f["o"]), (sf_h, dsf, errs_f["S"])])
    print(f"[bwd identity] sum(dv v) = {lhs:.9e}  sum(do o) + sum(dST ST) = {rhs:.9e}  |diff| {abs(lhs - rhs):.3e}"
          f" <= bar {bar:.3e}", flush=True)
    assert abs(lhs - rhs) <= bar, (lhs, rhs, bar)


@pytest.mark.parametrize("gate,norm,d", [(True, True, 128), (True, False, 128), (False, True, 128), (True, True, 64)])
def test_backward_fused_prologue(gate, norm, d):
    """Gradients with respect to the raw inputs of the fused prologue (gate pre-activations a, b
    with g = -5 sigmoid(a), beta = sigmoid(b); raw q, k normalised over d_k) against the oracle's
    backward through the same prologue.  bf16 inputs, ragged sequences, initial and final states;
    with the normalisation one q row and one k row are zero (their gradients are zero)."""
    w = W.make_prefill_raw([200, 1, 0, 130, 77], H=3, dk=d, dv=d, seed=52, s0_std=0.1)
    scale = d ** -0.5
    q, k = w.q.copy(), w.k.copy()
    if norm:
        q[5, 0] = 0.0
        k[7, 1] = 0.0
    else:
        # unnormalised q, k would make the recurrence blow up: use unit rows (still bf16-exact)
        q = W.round_bf16((q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32))
        k = W.round_bf16((k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32))
    if gate:
        a_ref, b_ref = w.g, w.beta
        g_in, b_in = to_dev(w.g, torch.bfloat16), to_dev(w.beta, torch.float32)
    else:
        g64 = -5.0 / (1.0 + np.exp(-w.g.astype(np.float64)))
        b64 = 1.0 / (1.0 + np.exp(-w.beta.astype(np.float64)))
        a_ref, b_ref = g64.astype(np.float32), b64.astype(np.float32)
        g_in, b_in = to_dev(a_ref, torch.float32), to_dev(b_ref, torch.float32)
    do, dsf = W.make_cotangents(w, seed=52)
    outs = kda.kda_chunk_bwd(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(w.v, torch.bfloat16),
                             g_in, b_in, to_dev(do, torch.float32), list(w.cu_seqlens), scale,
                             to_dev(w.s0, torch.float32), to_dev(dsf, torch.float32),
                             gate_preactivation=gate, normalize_qk=norm)
    torch.cuda.synchronize()
    got = [x.cpu().numpy() for x in outs]
    ref = OB.backward_fused(q, k, w.v, a_ref, b_ref, w.cu_seqlens, scale, w.s0, do, dsf, normalize=norm, gate=gate)
    errs = {n: W.rel_max_err(x, y) for n, x, y in zip(NAMES, got, ref)}
    label = f"fused prologue gate={gate} norm={norm} d={d}"
    print(f"[bwd parity] {label}: " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": "bwd " + label, "H": w.H, "d": d, "dtype": "bf16",
                                "tokens": w.total_tokens, "tol": TOL["bf16"], **errs}) + "\n")
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], (k_, v_)
    if norm:
        assert np.all(got[0][5, 0] == 0) and np.all(got[1][7, 1] == 0)


def test_backward_graph_capture_and_replay():
    """The backward through the C ABI captured into a HIP graph (arguments, outputs and workspace
    prepared before the capture), replayed three times with eager work between: every replay
    equals the eager result bit for bit."""
    import ctypes
    L = kda.lib()
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    w = W.make_prefill([130, 64, 7], H=3, dk=128, dv=128, dtype="bf16", seed=93, s0_std=0.1)
    do, dsf = W.make_cotangents(w, seed=93)
    q, k, v = to_dev(w.q, bf), to_dev(w.k, bf), to_dev(w.v, bf)
    g, b, s0 = to_dev(w.g, torch.float32), to_dev(w.beta, torch.float32), to_dev(w.s0, torch.float32)
    do_d, dsf_d = to_dev(do, torch.float32), to_dev(dsf, torch.float32)
    cu_h = torch.tensor(list(w.cu_seqlens), dtype=torch.int32)
    cu_d = cu_h.to(dev)
    T, H, D, N = w.total_tokens, 3, 128, 3
    outs = [torch.empty((T, H, D), dtype=torch.float32, device=dev) for _ in range(4)]
    outs.insert(4, torch.empty((T, H), dtype=torch.float32, device=dev))
    outs.append(torch.empty((N, H, D, D), dtype=torch.float32, device=dev))
    dq, dk_, dv_, dg, db, ds0 = outs
    A = kda.make_bwd_args(q, k, v, g, b, cu_d, cu_h, 1.0, s0, do_d, dsf_d, dq, dk_, dv_, dg, db, ds0)
    ws = torch.empty(L.kda_chunk_bwd_workspace_bytes(ctypes.byref(A)), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()

    def step():
        assert L.kda_chunk_bwd(ctypes.byref(A), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                               ctypes.c_void_p(side.cuda_stream)) == 0

    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for rep in range(3):
        for x in outs:
            x.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, x, y in zip(NAMES, outs, ref):
            assert torch.equal(x, y), (rep, n)
    print("[graph] backward captured; 3 replays equal to the eager result", flush=True)
