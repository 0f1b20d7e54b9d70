"""CPU fp64 oracle for the Kimi Delta Attention (KDA) operator -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``libkda.so`` and the
``gated_delta_rule_49_amd`` binding) never imports, links or calls it, and the
two share no code: the only thing both sides use is the seeded input
generator in ``workloads``, which holds none of the operator's arithmetic.

Two independent formulations live here:

* ``forward`` / ``decode`` -- the token-by-token recurrence in plain C, fp64
  (``kda_oracle.c``), multi-threaded over (sequence, head) chains.
* ``chunked.forward_chunked`` -- a separately written chunk-parallel form in
  numpy fp64 (pairwise exponentials, explicit forward substitution), used to
  pin the recurrence and the chunk algebra against each other.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exact retrieval, explicit-matrix brute force, exact rational
hand example, invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_kda.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _FwdArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("scale", ctypes.c_double),
        ("S0", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("S_final", ctypes.c_void_p),
        ("ckpt_every", ctypes.c_int32),
        ("ckpt", ctypes.c_void_p),
        ("n_threads", ctypes.c_int32),
    ]


def _bind(path):
    lib = ctypes.CDLL(path)
    lib.oracle_kda_forward.argtypes = [ctypes.POINTER(_FwdArgs)]
    lib.oracle_kda_forward.restype = ctypes.c_int
    lib.oracle_kda_decode.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 5 + [
        ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    lib.oracle_kda_decode.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _bind(build())
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most 16
    (a fair share of a shared host; the oracle is a checker, not a product)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward(q, k, v, g, beta, cu_seqlens=None, scale=1.0, initial_state=None,
            checkpoint_every=0, n_threads=None, _lib_override=None):
    """Token-by-token KDA recurrence in fp64.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; inputs are taken as the
    exact fp32 values the device receives.  cu_seqlens: [N+1] token offsets
    (None => one sequence).  initial_state: [N, H, dk, dv] or None (zeros).

    Returns (o [T,H,dv], S_final [N,H,dk,dv], checkpoints [M,H,dk,dv] or None),
    all float64.
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert beta.shape == (T, H)
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    S0 = None if initial_state is None else _f32(initial_state)
    if S0 is not None:
        assert S0.shape == (N, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    ck = None
    if checkpoint_every:
        M = int(np.sum(np.diff(cu) // checkpoint_every))
        ck = np.zeros((M, H, dk, dv), dtype=np.float64)
    a = _FwdArgs(N, H, dk, dv, cu.ctypes.data, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                 float(scale), _ptr(S0), _ptr(o), _ptr(Sf), int(checkpoint_every or 0), _ptr(ck),
                 int(n_threads or default_threads()))
    rc = (_lib_override or _load()).oracle_kda_forward(ctypes.byref(a))
    if rc != 0:
        raise RuntimeError("oracle_kda_forward failed")
    return o, Sf, ck


def decode(q, k, v, g, beta, state, scale=1.0, n_threads=None):
    """One decode step per (sequence, head).  q,k,g: [N,H,dk]; v: [N,H,dv];
    beta: [N,H]; state: [N,H,dk,dv] (fp32 values).  Returns (o, new_state) fp64."""
    q, k, v, g, beta, S = map(_f32, (q, k, v, g, beta, state))
    N, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv), dtype=np.float64)
    Sn = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().oracle_kda_decode(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   float(scale), _ptr(S), _ptr(Sn), _ptr(o),
                                   int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_kda_decode failed")
    return o, Sn


# ---- fused prologue (the skill card's quick facts: the log-decay is a lower-bounded scaled
# sigmoid with g_min = -5; q and k are L2-normalised per token and head)

def prologue(q, k, g_pre, b_pre, normalize=True):
    """The operator's inputs from raw ones, in fp64: g = -5 sigmoid(a), beta = sigmoid(b), and
    q, k divided by their L2 norm over d_k (a zero vector stays zero)."""
    q, k, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, g_pre, b_pre))
    g = -5.0 / (1.0 + np.exp(-a))
    beta = 1.0 / (1.0 + np.exp(-b))
    if normalize:
        def unit(x):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            return np.divide(x, n, out=np.zeros_like(x), where=n > 0)
        q, k = unit(q), unit(k)
    return q, k, g, beta


def forward_fused(q, k, v, g_pre, b_pre, cu_seqlens=None, scale=1.0, initial_state=None,
                  checkpoint_every=0, normalize=True):
    """forward() on the prologue's outputs (the recurrence takes them rounded to fp32)."""
    qn, kn, g, beta = prologue(q, k, g_pre, b_pre, normalize)
    return forward(qn, kn, v, g, beta, cu_seqlens, scale, initial_state, checkpoint_every=checkpoint_every)


# ---- paged state pool (the digest's inference paragraph: a pool of recurrent states with prefix
# reuse at 512-token boundaries).  A pool is [P, H, dk, dv]; an index of -1, or any index outside
# [0, P), means "no slot".  These are plain gathers and scatters around forward / decode.

def _slot(idx, P):
    i = int(idx)
    return i if 0 <= i < P else -1


def forward_paged(q, k, v, g, beta, cu_seqlens, scale, pool, initial_state_indices=None,
                  checkpoint_every=0, checkpoint_indices=None):
    """forward() with the initial states gathered from pool slots (initial_state_indices [N];
    -1: zeros) and the checkpoints scattered into pool slots (checkpoint_indices [M]; -1: not
    kept).  Returns (o, final_state, new_pool) fp64; new_pool is a copy of `pool` with the
    checkpoint slots overwritten."""
    pool = np.asarray(pool, dtype=np.float64)
    P, H, dk, dv = pool.shape
    cu = np.asarray(cu_seqlens if cu_seqlens is not None else [0, np.asarray(q).shape[0]], dtype=np.int64)
    N = len(cu) - 1
    s0 = None
    if initial_state_indices is not None:
        s0 = np.zeros((N, H, dk, dv), dtype=np.float64)
        for n in range(N):
            sl = _slot(initial_state_indices[n], P)
            if sl >= 0:
                s0[n] = pool[sl]
    o, sf, ck = forward(q, k, v, g, beta, cu, scale, s0, checkpoint_every=checkpoint_every)
    new_pool = pool.copy()
    if checkpoint_indices is not None and ck is not None:
        for m in range(ck.shape[0]):
            sl = _slot(checkpoint_indices[m], P)
            if sl >= 0:
                new_pool[sl] = ck[m]
    return o, sf, new_pool


def decode_paged(q, k, v, g, beta, pool, state_indices, scale=1.0):
    """decode() on pool slots: sequence n updates slot state_indices[n]; a sequence with no slot
    is inactive (o = 0, pool untouched).  Returns (o, new_pool) fp64."""
    pool = np.asarray(pool, dtype=np.float64)
    P = pool.shape[0]
    N = np.asarray(q).shape[0]
    act = [n for n in range(N) if _slot(state_indices[n], P) >= 0]
    o = np.zeros((N,) + np.asarray(v).shape[1:], dtype=np.float64)
    new_pool = pool.copy()
    if act:
        sl = [_slot(state_indices[n], P) for n in act]
        sel = lambda x: np.asarray(x)[act]
        oa, sa = decode(sel(q), sel(k), sel(v), sel(g), sel(beta), pool[sl], scale)
        o[act] = oa
        new_pool[sl] = sa
    return o, new_pool


def forward_from_library(path):
    """A `forward` bound to another build of kda_oracle.c (used by the mutation
    test, which compiles deliberately broken copies of the oracle source)."""
    lib = _bind(path)

    def fwd(*args, **kw):
        kw["_lib_override"] = lib
        return forward(*args, **kw)
    return fwd
