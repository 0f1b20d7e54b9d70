"""GPU parity at the full sizes of the measured workloads, in the launch
configuration the benchmark times (bf16 q/k/v, chunk 32, the library's default).

The whole GPU problem runs at once; the fp64 oracle then recomputes a sample of
independent (sequence, head) chains -- whole chains, every token -- and the
sampled outputs, final states and checkpoints are compared element by element
with the bf16-path bar (max|diff| / RMS <= 2e-2).  Everything the oracle does not
recompute is checked for finiteness.  The decode workload (256 x 96 states) is
small enough for the oracle to cover completely.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
CHUNK = kda.DEFAULT_CHUNK


def dev():
    return torch.device("cuda:0")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def _report(label, errs):
    print(f"[fullsize] {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL_BF16, (label, k, v)


def _sub(w, heads):
    """The same problem restricted to a subset of heads (heads are independent)."""
    h = list(heads)
    return (np.ascontiguousarray(w.q[:, h]), np.ascontiguousarray(w.k[:, h]), np.ascontiguousarray(w.v[:, h]),
            np.ascontiguousarray(w.g[:, h]), np.ascontiguousarray(w.beta[:, h]),
            None if w.s0 is None else np.ascontiguousarray(w.s0[:, h]))


def _run_whole(w):
    d = dev()
    return kda.kda_chunk_fwd(_bf16(w.q).to(d), _bf16(w.k).to(d), _bf16(w.v).to(d), _f32(w.g).to(d),
                             _f32(w.beta).to(d), list(w.cu_seqlens), 1.0,
                             None if w.s0 is None else _f32(w.s0).to(d), True, w.checkpoint_every,
                             chunk_size=CHUNK)


def test_prefill_T4096_H32_every_head():
    w = W.make_workload(1)
    o, sf, _ = _run_whole(w)
    torch.cuda.synchronize()
    o_r, s_r, _ = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 1.0, w.s0, 0)
    _report("T=4096 H=32", {"o": W.rel_max_err(o.cpu().numpy(), o_r),
                                     "S": W.rel_max_err(sf.cpu().numpy(), s_r)})


def test_prefill_T65536_H96_sampled_heads():
    w = W.make_workload(2)
    o, sf, _ = _run_whole(w)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(sf).all())
    heads = [0, 41, 95]
    q, k, v, g, b, s0 = _sub(w, heads)
    o_r, s_r, _ = oracle.forward(q, k, v, g, b, w.cu_seqlens, 1.0, s0, 0)
    idx = torch.tensor(heads, device=o.device)
    o_s = o.index_select(1, idx).cpu().numpy()
    s_s = sf.index_select(1, idx).cpu().numpy()
    _report(f"T=65536 H=96 heads={heads}", {"o": W.rel_max_err(o_s, o_r), "S": W.rel_max_err(s_s, s_r)})


@pytest.mark.timeout(900)
def test_prefill_one_million_tokens_two_heads():
    """A 1,048,576-token context (the longest the pages speak of), two heads, bf16, initial state,
    checkpoints every 65536: every output, the final states and the checkpoints against the
    fp64 oracle over the whole chain (32,768 chunks through the recurrence)."""
    w = W.make_prefill([1 << 20], H=2, dk=128, dv=128, dtype="bf16", seed=71, s0_std=0.1,
                       checkpoint_every=1 << 16)
    o, sf, ck = _run_whole(w)
    torch.cuda.synchronize()
    o_r, s_r, ck_r = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 1.0, w.s0, 1 << 16)
    _report("T=1048576 H=2", {"o": W.rel_max_err(o.cpu().numpy(), o_r), "S": W.rel_max_err(sf.cpu().numpy(), s_r),
                              "ckpt": W.rel_max_err(ck.cpu().numpy(), ck_r)})


@pytest.mark.timeout(900)
def test_backward_T65536_H96_sampled_head_and_identity():
    """The backward at the benchmark's shape: every gradient finite; one whole head (65,536 tokens)
    against the fp64 oracle adjoint; and over all 96 heads the identity that holds because o and S_T
    are linear in (S_0, V) jointly: sum(dv v) + sum(dS0 S0) = sum(d_o o) + sum(dS_T S_T), with o and
    S_T from the forward."""
    from oracle import backward as OB
    w = W.make_workload(2)
    do, dsf = W.make_cotangents(w, seed=31)
    d = dev()
    q, k, v = _bf16(w.q).to(d), _bf16(w.k).to(d), _bf16(w.v).to(d)
    g, b, s0 = _f32(w.g).to(d), _f32(w.beta).to(d), _f32(w.s0).to(d)
    do_d, dsf_d = _f32(do).to(d), _f32(dsf).to(d)
    dq, dk, dv, dg, db, ds0 = kda.kda_chunk_bwd(q, k, v, g, b, do_d, list(w.cu_seqlens), 1.0, s0, dsf_d)
    o, sf, _ = kda.kda_chunk_fwd(q, k, v, g, b, list(w.cu_seqlens), 1.0, s0, True, 0, chunk_size=CHUNK)
    torch.cuda.synchronize()
    for x in (dq, dk, dv, dg, db, ds0):
        assert bool(torch.isfinite(x).all())
    lhs = float((dv.double() * v.double()).sum() + (ds0.double() * s0.double()).sum())
    rhs = float((do_d.double() * o.double()).sum() + (dsf_d.double() * sf.double()).sum())
    norm = float(torch.sqrt((dv.double() ** 2).sum() * (v.double() ** 2).sum()))
    print(f"[fullsize] T=65536 H=96 backward identity: {lhs:.6e} vs {rhs:.6e} (scale {norm:.3e})", flush=True)
    assert abs(lhs - rhs) <= 1e-3 * norm, (lhs, rhs, norm)
    del o, sf
    h = [41]
    qh, kh, vh, gh, bh, s0h = _sub(w, h)
    ref = OB.backward(qh, kh, vh, gh, bh, w.cu_seqlens, 1.0, s0h, np.ascontiguousarray(do[:, h]),
                      np.ascontiguousarray(dsf[:, h]))
    got = [x[:, h[0]:h[0] + 1].cpu().numpy() for x in (dq, dk, dv, dg, db, ds0)]
    _report(f"T=65536 H=96 backward head {h[0]}", {n: W.rel_max_err(a, r) for n, a, r in
                                              zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref)})


@pytest.mark.timeout(900)
def test_backward_prologue_T65536_H96_sampled_head_and_identity():
    """The backward through the fused gate / normalisation prologue at the benchmark's shape and in
    its launch configuration (`bench.py --backward --prologue`): raw bf16 q, k ~ N(0,1), bf16 gate
    pre-activations a ~ N(0,1), fp32 b ~ N(0,1), scale d^-1/2, drawn on the device with a seeded
    generator.  Every gradient finite; one whole head against the oracle's adjoint through the
    same prologue; over all 96 heads the linearity identity (the prologue touches neither v nor S_0)."""
    from oracle import backward as OB
    d = dev()
    T, H, D = 65536, 96, 128
    gen = torch.Generator(device=d)
    gen.manual_seed(33)

    def rn(*shape):
        return torch.randn(shape, generator=gen, device=d)

    bf = torch.bfloat16
    q, k, v, a = rn(T, H, D).to(bf), rn(T, H, D).to(bf), rn(T, H, D).to(bf), rn(T, H, D).to(bf)
    b = rn(T, H)
    s0, do, dsf = 0.1 * rn(1, H, D, D), rn(T, H, D), rn(1, H, D, D)
    scale = D ** -0.5
    pro = dict(gate_preactivation=True, normalize_qk=True)
    grads = kda.kda_chunk_bwd(q, k, v, a, b, do, [0, T], scale, s0, dsf, **pro)
    o, sf, _ = kda.kda_chunk_fwd(q, k, v, a, b, [0, T], scale, s0, True, 0, chunk_size=32, **pro)
    torch.cuda.synchronize()
    for x in grads:
        assert bool(torch.isfinite(x).all())
    dv, ds0 = grads[2], grads[5]
    lhs = float((dv.double() * v.double()).sum() + (ds0.double() * s0.double()).sum())
    rhs = float((do.double() * o.double()).sum() + (dsf.double() * sf.double()).sum())
    norm = float(torch.sqrt((dv.double() ** 2).sum() * (v.double() ** 2).sum()))
    print(f"[fullsize] T=65536 H=96 prologue backward identity: {lhs:.6e} vs {rhs:.6e} (scale {norm:.3e})",
          flush=True)
    assert abs(lhs - rhs) <= 1e-3 * norm, (lhs, rhs, norm)
    del o, sf
    h = 57

    def host(x):
        return x[:, h:h + 1].float().cpu().numpy().astype(np.float64)

    ref = OB.backward_fused(host(q), host(k), host(v), host(a), host(b), [0, T], scale, host(s0), host(do),
                            host(dsf), normalize=True, gate=True)
    got = [host(x) for x in grads]
    _report(f"T=65536 H=96 prologue backward head {h}",
            {n: W.rel_max_err(x, r) for n, x, r in zip(("dq", "dk", "dv", "da", "db", "dS0"), got, ref)})


def test_decode_N256_H96_every_state():
    w = W.make_workload(3)
    d = dev()
    state = _f32(w.s0).to(d)
    o = kda.kda_decode_step(_bf16(w.q).to(d), _bf16(w.k).to(d), _bf16(w.v).to(d), _f32(w.g).to(d),
                            _f32(w.beta).to(d), state, 1.0)
    torch.cuda.synchronize()
    o_r, s_r = oracle.decode(w.q, w.k, w.v, w.g, w.beta, w.s0, 1.0)
    _report("decode N=256 H=96", {"o": W.rel_max_err(o.cpu().numpy(), o_r),
                                          "S": W.rel_max_err(state.cpu().numpy(), s_r)})


@pytest.mark.timeout(600)
def test_varlen_64seq_1p85M_tokens_checkpoints_sampled():
    seqlens = W.varlen_lengths()
    c = W.WORKLOADS[4]
    H, dk, dv, every = c["H"], c["dk"], c["dv"], c["checkpoint_every"]
    T, N = sum(seqlens), len(seqlens)
    d = dev()
    q = torch.empty((T, H, dk), dtype=torch.bfloat16, device=d)
    k = torch.empty_like(q)
    v = torch.empty((T, H, dv), dtype=torch.bfloat16, device=d)
    g = torch.empty((T, H, dk), dtype=torch.float32, device=d)
    beta = torch.empty((T, H), dtype=torch.float32, device=d)
    s0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=d)
    for first, off, part in W.workload_parts(4):
        n = part.total_tokens
        q[off:off + n] = _bf16(part.q).to(d)
        k[off:off + n] = _bf16(part.k).to(d)
        v[off:off + n] = _bf16(part.v).to(d)
        g[off:off + n] = _f32(part.g).to(d)
        beta[off:off + n] = _f32(part.beta).to(d)
        s0[first:first + len(part.seqlens)] = _f32(part.s0).to(d)
        print(f"[fullsize] varlen generated sequences {first}..{first + len(part.seqlens) - 1}", flush=True)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    o, sf, ck = kda.kda_chunk_fwd(q, k, v, g, beta, list(cu), 1.0, s0, True, every, chunk_size=CHUNK)
    torch.cuda.synchronize()
    assert ck.shape[0] == sum(L // every for L in seqlens)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(sf).all()) and bool(torch.isfinite(ck).all())
    del q, k, v, g, beta

    order = np.argsort(seqlens, kind="stable")
    sample = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0]), 7})
    heads = [0, 13, 31]
    ck_first = np.concatenate([[0], np.cumsum([L // every for L in seqlens])])
    idx = torch.tensor(heads, device=d)
    for s in sample:
        L = seqlens[s]
        w = W.make_prefill([L], H, dk, dv, c["dtype"], 0, c["s0_std"], "default", every, wid=4, seq_ids=[s])
        qs, ks, vs, gs, bs, s0s = _sub(w, heads)
        o_r, s_r, ck_r = oracle.forward(qs, ks, vs, gs, bs, w.cu_seqlens, 1.0, s0s, every)
        a = int(cu[s])
        errs = {"o": W.rel_max_err(o[a:a + L].index_select(1, idx).cpu().numpy(), o_r),
                "S": W.rel_max_err(sf[s:s + 1].index_select(1, idx).cpu().numpy(), s_r)}
        if L // every:
            errs["ckpt"] = W.rel_max_err(ck[ck_first[s]:ck_first[s + 1]].index_select(1, idx).cpu().numpy(), ck_r)
        _report(f"varlen seq {s} L={L} heads={heads}", errs)
