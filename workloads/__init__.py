"""Seeded synthetic inputs for the KDA operator, shared by the tests, the bench
and the smoke check.  This module holds none of the operator's arithmetic:
only random draws, the input normalisation the workloads prescribe, and bf16
rounding of inputs.

Distributions (the same for every workload, the "default" gate):
  q, k  ~ N(0, 1), L2-normalised per (token, head) over d_k; q is then scaled
          by d_k**-0.5 (so the operator itself runs with scale = 1).
  v     ~ N(0, 1)
  g     = -5 * sigmoid(N(0, 1))        [T, H, d_k] fp32, natural-log decay
  beta  = sigmoid(N(0, 1))             [T, H] fp32
  S0    ~ N(0, 0.01), read as variance 0.01 (std 0.1), when a workload has one.
Normalisation is done in fp32 with no epsilon; bf16 workloads round q, k, v
to bf16 (round-to-nearest-even) afterwards, and every consumer sees exactly
those rounded values.

Stress gates: "slow" g = -5*sigmoid(N(0,1) - 6) (mean g ~ -0.02, long memory);
"min" g = -5 everywhere (the bound); "zero" g = 0 (no decay).

Seeding: every tensor block is drawn from its own PCG64 stream,
SeedSequence([20261203, workload_id, seq, block, tensor_id, seed]), with
blocks of 4096 tokens inside each sequence, so any block can be regenerated
alone and generation parallelises over threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261203
BLOCK = 4096
_TID = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "s0": 5, "lengths": 6, "do": 7, "dsf": 8}


def _rng(wid, seq, block, tensor, seed):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([ROOT_SEED, wid, seq, block, _TID[tensor], seed])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-exact (uint16 array)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float32)))).astype(np.float32)


def _l2n(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / n).astype(np.float32)


@dataclass
class Workload:
    """A synthetic KDA problem.  Arrays are host numpy fp32 (bf16-exact where
    ``dtype == 'bf16'``)."""
    name: str
    seqlens: list
    H: int
    dk: int
    dv: int
    dtype: str                      # "f32" or "bf16": dtype of q, k, v
    q: np.ndarray = None
    k: np.ndarray = None
    v: np.ndarray = None
    g: np.ndarray = None
    beta: np.ndarray = None
    s0: np.ndarray = None           # [N, H, dk, dv] or None
    checkpoint_every: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int64)

    @property
    def total_tokens(self):
        return int(sum(self.seqlens))


def _gen_block(wid, seed, s, b, T0, Tb, H, dk, dv, dtype, gate, out):
    rq = _rng(wid, s, b, "q", seed)
    rk = _rng(wid, s, b, "k", seed)
    rv = _rng(wid, s, b, "v", seed)
    rg = _rng(wid, s, b, "g", seed)
    rb = _rng(wid, s, b, "beta", seed)
    q = _l2n(rq.standard_normal((Tb, H, dk), dtype=np.float32)) * np.float32(dk ** -0.5)
    k = _l2n(rk.standard_normal((Tb, H, dk), dtype=np.float32))
    v = rv.standard_normal((Tb, H, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    x = rg.standard_normal((Tb, H, dk), dtype=np.float32)
    if gate == "default":
        g = np.float32(-5.0) * _sigmoid(x)
    elif gate == "slow":
        g = np.float32(-5.0) * _sigmoid(x - np.float32(6.0))
    elif gate == "min":
        g = np.full((Tb, H, dk), -5.0, dtype=np.float32)
    elif gate == "zero":
        g = np.zeros((Tb, H, dk), dtype=np.float32)
    else:
        raise ValueError(gate)
    beta = _sigmoid(rb.standard_normal((Tb, H), dtype=np.float32))
    out["q"][T0:T0 + Tb] = q
    out["k"][T0:T0 + Tb] = k
    out["v"][T0:T0 + Tb] = v
    out["g"][T0:T0 + Tb] = g
    out["beta"][T0:T0 + Tb] = beta


def make_prefill(seqlens, H, dk=128, dv=128, dtype="bf16", seed=0, s0_std=0.0, gate="default",
                 checkpoint_every=0, wid=100, name=None, threads=None, seq_ids=None) -> Workload:
    """Packed varlen problem.  `seq_ids` (default 0..N-1) are the sequence
    indices the draws are keyed on: passing a subset of a larger workload's
    lengths with their original indices regenerates exactly those sequences."""
    seqlens = [int(x) for x in seqlens]
    seq_ids = list(range(len(seqlens))) if seq_ids is None else [int(x) for x in seq_ids]
    assert len(seq_ids) == len(seqlens)
    T = sum(seqlens)
    out = {n: np.empty((T, H, d), dtype=np.float32) for n, d in (("q", dk), ("k", dk), ("v", dv), ("g", dk))}
    out["beta"] = np.empty((T, H), dtype=np.float32)
    jobs = []
    off = 0
    for s, L in zip(seq_ids, seqlens):
        for b in range(0, max(1, math.ceil(L / BLOCK))):
            Tb = min(BLOCK, L - b * BLOCK)
            if Tb > 0:
                jobs.append((wid, seed, s, b, off + b * BLOCK, Tb, H, dk, dv, dtype, gate, out))
        off += L
    nt = threads or min(16, max(1, len(os.sched_getaffinity(0))))
    if len(jobs) > 1 and nt > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda j: _gen_block(*j), jobs))
    else:
        for j in jobs:
            _gen_block(*j)
    s0 = None
    if s0_std > 0:
        s0 = np.empty((len(seqlens), H, dk, dv), dtype=np.float32)
        for i, s in enumerate(seq_ids):
            s0[i] = _rng(wid, s, 0, "s0", seed).standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    return Workload(name or f"prefill_H{H}_d{dk}", seqlens, H, dk, dv, dtype, out["q"], out["k"], out["v"],
                    out["g"], out["beta"], s0, checkpoint_every, {"gate": gate, "seed": seed})


def make_prefill_raw(seqlens, H, dk=128, dv=128, seed=0, s0_std=0.0, checkpoint_every=0, wid=110,
                     name=None) -> Workload:
    """Inputs for the fused prologue: the same draws as the default distributions, before the
    gate and the normalisation.  q, k ~ N(0,1) unnormalised, v ~ N(0,1) (all bf16-exact),
    ``g`` holds the bf16-exact gate pre-activations a ~ N(0,1) [T,H,dk] and ``beta`` the fp32
    pre-activations b ~ N(0,1) [T,H].  (The operator then uses g = -5 sigmoid(a),
    beta = sigmoid(b) and L2-normalised q, k.)"""
    seqlens = [int(x) for x in seqlens]
    T = sum(seqlens)
    q = np.empty((T, H, dk), dtype=np.float32)
    k, a = np.empty_like(q), np.empty_like(q)
    v = np.empty((T, H, dv), dtype=np.float32)
    b = np.empty((T, H), dtype=np.float32)
    off = 0
    for s, L in enumerate(seqlens):
        for blk in range(0, max(1, math.ceil(L / BLOCK))):
            Tb = min(BLOCK, L - blk * BLOCK)
            if Tb <= 0:
                continue
            sl = slice(off + blk * BLOCK, off + blk * BLOCK + Tb)
            q[sl] = round_bf16(_rng(wid, s, blk, "q", seed).standard_normal((Tb, H, dk), dtype=np.float32))
            k[sl] = round_bf16(_rng(wid, s, blk, "k", seed).standard_normal((Tb, H, dk), dtype=np.float32))
            v[sl] = round_bf16(_rng(wid, s, blk, "v", seed).standard_normal((Tb, H, dv), dtype=np.float32))
            a[sl] = round_bf16(_rng(wid, s, blk, "g", seed).standard_normal((Tb, H, dk), dtype=np.float32))
            b[sl] = _rng(wid, s, blk, "beta", seed).standard_normal((Tb, H), dtype=np.float32)
        off += L
    s0 = None
    if s0_std > 0:
        s0 = np.empty((len(seqlens), H, dk, dv), dtype=np.float32)
        for i in range(len(seqlens)):
            s0[i] = _rng(wid, i, 0, "s0", seed).standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    return Workload(name or f"prefill_raw_H{H}_d{dk}", seqlens, H, dk, dv, "bf16", q, k, v, a, b, s0,
                    checkpoint_every, {"raw": True, "seed": seed})


def make_decode(N, H, dk=128, dv=128, dtype="bf16", seed=0, s0_std=0.1, gate="default", wid=103,
                name=None, threads=None) -> Workload:
    """N independent sequences, one new token each; the state is [N, H, dk, dv]."""
    w = make_prefill([1] * N, H, dk, dv, dtype, seed, 0.0, gate, 0, wid, name or f"decode_N{N}_H{H}", threads)
    # one independent state per sequence, drawn in parallel blocks of sequences
    s0 = np.empty((N, H, dk, dv), dtype=np.float32)

    def fill(s):
        s0[s] = _rng(wid, s, 0, "s0", seed).standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    nt = threads or min(16, max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(fill, range(N)))
    w.s0 = s0
    return w


def varlen_lengths(n=64, lo=512, hi=131072, step=512):
    """64 lengths, log-uniform on [lo, hi], rounded to the nearest multiple of
    `step` inside [lo, hi].  The total is whatever the draw gives (about 1.5M
    expected); it is reported, not rescaled."""
    r = _rng(4, 0, 0, "lengths", 0)
    x = np.exp(r.uniform(math.log(lo), math.log(hi), size=n))
    L = np.clip(np.rint(x / step) * step, lo, hi).astype(np.int64)
    return [int(v) for v in L]


# The five workloads the operator is measured and checked on.
WORKLOADS = {
    0: dict(name="tiny_f32_T256_H2_d64", kind="prefill", seqlens=[256], H=2, dk=64, dv=64, dtype="f32",
            s0_std=0.0, checkpoint_every=0),
    1: dict(name="prefill_T4096_H32_d128", kind="prefill", seqlens=[4096], H=32, dk=128, dv=128, dtype="bf16",
            s0_std=0.0, checkpoint_every=0),
    2: dict(name="prefill_T65536_H96_d128", kind="prefill", seqlens=[65536], H=96, dk=128, dv=128,
            dtype="bf16", s0_std=0.1, checkpoint_every=0),
    3: dict(name="decode_N256_H96_d128", kind="decode", N=256, H=96, dk=128, dv=128, dtype="bf16", s0_std=0.1),
    4: dict(name="varlen64_H32_d128_ckpt512", kind="prefill", seqlens=None, H=32, dk=128, dv=128, dtype="bf16",
            s0_std=0.1, checkpoint_every=512),
}


def make_workload(cid: int, seed: int = 0, gate: str = "default", threads=None) -> Workload:
    c = dict(WORKLOADS[cid])
    if c["kind"] == "decode":
        return make_decode(c["N"], c["H"], c["dk"], c["dv"], c["dtype"], seed, c["s0_std"], gate, wid=cid,
                           name=c["name"], threads=threads)
    seqlens = c["seqlens"] if c["seqlens"] is not None else varlen_lengths()
    return make_prefill(seqlens, c["H"], c["dk"], c["dv"], c["dtype"], seed, c["s0_std"], gate,
                        c["checkpoint_every"], wid=cid, name=c["name"], threads=threads)


def workload_parts(cid: int, max_tokens: int = 1 << 18, seed: int = 0, threads=None):
    """Yield (first_seq, token_offset, Workload) pieces that together make
    workload `cid`, each piece a run of whole sequences of at most about
    `max_tokens` tokens (a longer sequence is a piece of its own).  The values
    equal those of make_workload(cid), so a large workload can be streamed to a
    device without holding it on the host at once."""
    c = dict(WORKLOADS[cid])
    assert c["kind"] == "prefill"
    seqlens = c["seqlens"] if c["seqlens"] is not None else varlen_lengths()
    i, off = 0, 0
    while i < len(seqlens):
        j, n = i, 0
        while j < len(seqlens) and (j == i or n + seqlens[j] <= max_tokens):
            n += seqlens[j]
            j += 1
        yield i, off, make_prefill(seqlens[i:j], c["H"], c["dk"], c["dv"], c["dtype"], seed, c["s0_std"],
                                   "default", c["checkpoint_every"], wid=cid, name=c["name"], threads=threads,
                                   seq_ids=range(i, j))
        i, off = j, off + n


def make_cotangents(w: Workload, seed=0, d_final=True, wid=120):
    """Seeded upstream gradients for the backward of workload `w`: d_o ~ N(0, 1) fp32 [T, H, dv]
    and (if d_final) dS_T ~ N(0, 1) fp32 [N, H, dk, dv]; drawn per sequence."""
    do = np.empty((w.total_tokens, w.H, w.dv), dtype=np.float32)
    cu = w.cu_seqlens
    for s, L in enumerate(w.seqlens):
        if L:
            do[cu[s]:cu[s + 1]] = _rng(wid, s, 0, "do", seed).standard_normal((L, w.H, w.dv), dtype=np.float32)
    dsf = None
    if d_final:
        dsf = np.stack([_rng(wid, s, 0, "dsf", seed).standard_normal((w.H, w.dk, w.dv), dtype=np.float32)
                        for s in range(len(w.seqlens))]) if w.seqlens else np.zeros((0, w.H, w.dk, w.dv), np.float32)
    return do, dsf


def rel_max_err(x, ref) -> float:
    """max |x - ref| / RMS(ref) over the whole tensor, in fp64; inf if x has a
    non-finite value.  The two arrays must have the same shape (no broadcasting).
    An empty ref gives 0; an all-zero ref gives 0 if x is all zero, else inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch: {x.shape} vs {ref.shape}")
    if not np.all(np.isfinite(x)):
        return float("inf")
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    d = float(np.max(np.abs(x - ref)))
    return d / rms if rms > 0 else (0.0 if d == 0 else float("inf"))


class ErrAccum:
    """rel_max_err over a tensor seen in pieces (for tensors too large to hold, or to
    recompute, at once): the global max |x - ref| and the global sum of ref^2 and element
    count are accumulated, so value() equals rel_max_err of the concatenated pieces."""

    def __init__(self):
        self.maxdiff = 0.0
        self.sumsq = 0.0
        self.count = 0
        self.finite = True

    def add(self, x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if x.shape != ref.shape:
            raise ValueError(f"shape mismatch: {x.shape} vs {ref.shape}")
        if ref.size == 0:
            return self
        if not np.all(np.isfinite(x)):
            self.finite = False
            return self
        self.maxdiff = max(self.maxdiff, float(np.max(np.abs(x - ref))))
        self.sumsq += float(np.sum(ref * ref))
        self.count += ref.size
        return self

    def value(self) -> float:
        if not self.finite:
            return float("inf")
        if self.count == 0:
            return 0.0
        rms = math.sqrt(self.sumsq / self.count)
        return self.maxdiff / rms if rms > 0 else (0.0 if self.maxdiff == 0 else float("inf"))
