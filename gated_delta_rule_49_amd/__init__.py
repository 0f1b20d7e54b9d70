"""gated_delta_rule_49_amd -- Python binding of libkda, an MI355X (gfx950)
implementation of the Kimi Delta Attention (KDA) operator.

This module only marshals arguments: it takes torch tensors for device memory
and the current HIP stream, and calls the C ABI declared in ``include/kda.h``
(same names: ``kda_chunk_fwd``, ``kda_chunk_bwd``, ``kda_decode_step``,
``kda_chunk_fwd_workspace_bytes``, ``kda_chunk_bwd_workspace_bytes``,
``kda_chunk_bwd_workspace_min_bytes``, ``kda_status_str``,
``kda_abi_version``).
Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind -- if ``libkda.so`` is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_DEVICE = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_LOG_DECAY, KDA_GATE_PREACTIVATION = 0, 1


class KdaFwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("checkpoint_every", ctypes.c_int32), ("checkpoints", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("initial_state_indices", ctypes.c_void_p), ("checkpoint_indices", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32), ("gate_mode", ctypes.c_int32), ("normalize_qk", ctypes.c_int32),
        ("segment_tokens", ctypes.c_int32),
    ]


class KdaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("state", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p), ("o", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
        ("gate_mode", ctypes.c_int32), ("normalize_qk", ctypes.c_int32),
    ]


class KdaBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("d_o", ctypes.c_void_p), ("d_final_state", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk_out", ctypes.c_void_p), ("dv_out", ctypes.c_void_p),
        ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("d_initial_state", ctypes.c_void_p),
        ("gate_mode", ctypes.c_int32), ("normalize_qk", ctypes.c_int32), ("states", ctypes.c_void_p),
    ]


EXPORTED = ["kda_chunk_fwd", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_noalloc", "kda_chunk_bwd",
            "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd_workspace_min_bytes", "kda_decode_step",
            "kda_status_str", "kda_abi_version"]
NOALLOC_MAX_SEQS = 65536   # KDA_NOALLOC_MAX_SEQS of include/kda.h

ABI_VERSION = 7   # KDA_ABI_VERSION of include/kda.h, whose struct layouts the ctypes classes above mirror
_lib = None
_lock = threading.Lock()


def lib():
    """Load libkda.so (once).  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                                   "g.build()'` (hipcc, gfx950) first")
            L = ctypes.CDLL(LIB_PATH)
            L.kda_chunk_fwd.argtypes = [ctypes.POINTER(KdaFwdArgs), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
            L.kda_chunk_fwd.restype = ctypes.c_int
            L.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(KdaFwdArgs), ctypes.c_void_p]
            L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
            L.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaFwdArgs)]
            L.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
            L.kda_chunk_bwd.argtypes = [ctypes.POINTER(KdaBwdArgs), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
            L.kda_chunk_bwd.restype = ctypes.c_int
            L.kda_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaBwdArgs)]
            L.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
            L.kda_chunk_bwd_workspace_min_bytes.argtypes = [ctypes.POINTER(KdaBwdArgs)]
            L.kda_chunk_bwd_workspace_min_bytes.restype = ctypes.c_size_t
            L.kda_decode_step.argtypes = [ctypes.POINTER(KdaDecodeArgs), ctypes.c_void_p]
            L.kda_decode_step.restype = ctypes.c_int
            L.kda_status_str.argtypes = [ctypes.c_int]
            L.kda_status_str.restype = ctypes.c_char_p
            L.kda_abi_version.argtypes = []
            L.kda_abi_version.restype = ctypes.c_uint32
            if L.kda_abi_version() != ABI_VERSION:
                raise RuntimeError(f"{LIB_PATH} has ABI version {L.kda_abi_version()}, this binding expects "
                                   f"{ABI_VERSION}: rebuild it (`python -c 'import __graft_entry__ as g; g.build()'`)")
            _lib = L
    return _lib


def kda_status_str(status: int) -> str:
    return lib().kda_status_str(int(status)).decode()


def kda_abi_version() -> int:
    return int(lib().kda_abi_version())


class KdaError(RuntimeError):
    def __init__(self, status):
        super().__init__(kda_status_str(status))
        self.status = status


def _check(status):
    if status != KDA_OK:
        raise KdaError(status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)



# ---- argument checks ---------------------------------------------------------------------------
# The C ABI receives raw device pointers and cannot see dtypes, shapes, devices or strides, so a
# wrong tensor would make the kernels read or write outside its buffer.  Every entry point below
# checks its tensors here first and raises ValueError on any mismatch (no library call is made).

def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _tensor(name, t, device, shape=None, dtypes=None, optional=False):
    if t is None:
        _need(optional, f"{name} is required")
        return
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.device == device, f"{name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtypes is not None:
        _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _inputs(q, k, v, g, beta, gate_preactivation, device):
    _need(isinstance(q, torch.Tensor) and q.dim() == 3, "q must be a [tokens, H, dk] tensor")
    T, H, dk = q.shape
    _need(isinstance(v, torch.Tensor) and v.dim() == 3, "v must be a [tokens, H, dv] tensor")
    dv = v.shape[2]
    io = (torch.bfloat16, torch.float32)
    _tensor("q", q, device, (T, H, dk), io)
    _tensor("k", k, device, (T, H, dk), (q.dtype,))
    _tensor("v", v, device, (T, H, dv), (q.dtype,))
    _tensor("g", g, device, (T, H, dk), (torch.bfloat16,) if gate_preactivation else (torch.float32,))
    _tensor("beta", beta, device, (T, H), (torch.float32,))
    return T, H, dk, dv


def validate_fwd(q, k, v, g, beta, cu_host, cu_dev=None, initial_state=None, final_state=None, checkpoints=None,
                 o=None, initial_state_indices=None, checkpoint_indices=None, state_pool_slots=0,
                 checkpoint_every=0, gate_preactivation=False, device=None):
    """Check the tensors of a chunked forward; raises ValueError.  cu_host: int32 CPU [N+1]."""
    device = q.device if device is None else device
    T, H, dk, dv = _inputs(q, k, v, g, beta, gate_preactivation, device)
    _need(isinstance(cu_host, torch.Tensor) and cu_host.device.type == "cpu" and cu_host.dtype == torch.int32
          and cu_host.dim() == 1 and cu_host.numel() >= 1 and cu_host.is_contiguous(),
          "cu_seqlens (host copy) must be a contiguous int32 CPU tensor [N+1]")
    N = cu_host.numel() - 1
    _tensor("cu_seqlens", cu_dev, device, (N + 1,), (torch.int32,), optional=True)
    st = (torch.float32,)
    if initial_state_indices is not None:
        _tensor("initial_state_indices", initial_state_indices, device, (N,), (torch.int32,))
        _tensor("state_pool", initial_state, device, (state_pool_slots, H, dk, dv), st)
    else:
        _tensor("initial_state", initial_state, device, (N, H, dk, dv), st, optional=True)
    _tensor("final_state", final_state, device, (N, H, dk, dv), st, optional=True)
    lens = cu_host[1:] - cu_host[:-1]
    M = int((lens // checkpoint_every).sum()) if checkpoint_every > 0 and N > 0 else 0
    if checkpoint_indices is not None:
        _tensor("checkpoint_indices", checkpoint_indices, device, (M,), (torch.int32,))
        _tensor("state_pool", checkpoints, device, (state_pool_slots, H, dk, dv), st)
    elif checkpoints is not None:
        _tensor("checkpoints", checkpoints, device, (M, H, dk, dv), st)
    _tensor("o", o, device, (T, H, dv), st, optional=True)


def validate_bwd(q, k, v, g, beta, d_o, cu_host, cu_dev=None, initial_state=None, d_final_state=None,
                 states=None, outs=(), gate_preactivation=False, device=None):
    """Check the tensors of a backward; raises ValueError.  outs: (dq, dk, dv, dg, dbeta, dS0)."""
    device = q.device if device is None else device
    T, H, dk, dv = _inputs(q, k, v, g, beta, gate_preactivation, device)
    _need(isinstance(cu_host, torch.Tensor) and cu_host.device.type == "cpu" and cu_host.dtype == torch.int32
          and cu_host.dim() == 1 and cu_host.numel() >= 1 and cu_host.is_contiguous(),
          "cu_seqlens (host copy) must be a contiguous int32 CPU tensor [N+1]")
    N = cu_host.numel() - 1
    f32 = (torch.float32,)
    _tensor("cu_seqlens", cu_dev, device, (N + 1,), (torch.int32,), optional=True)
    _tensor("d_o", d_o, device, (T, H, dv), f32)
    _tensor("initial_state", initial_state, device, (N, H, dk, dv), f32, optional=True)
    _tensor("d_final_state", d_final_state, device, (N, H, dk, dv), f32, optional=True)
    M32 = int(((cu_host[1:] - cu_host[:-1]) // 32).sum()) if N > 0 else 0
    _tensor("states", states, device, (M32, H, dk, dv), f32, optional=True)
    shapes = ((T, H, dk), (T, H, dk), (T, H, dv), (T, H, dk), (T, H), (N, H, dk, dv))
    for name, t, shp in zip(("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"), outs, shapes):
        _tensor(name, t, device, shp, f32, optional=name == "d_initial_state")


def validate_decode(q, k, v, g, beta, state, o=None, state_indices=None, gate_preactivation=False, device=None):
    """Check the tensors of a decode step; raises ValueError."""
    device = q.device if device is None else device
    N, H, dk, dv = _inputs(q, k, v, g, beta, gate_preactivation, device)
    f32 = (torch.float32,)
    _need(isinstance(state, torch.Tensor) and state.dim() == 4, "state must be [N or slots, H, dk, dv]")
    if state_indices is not None:
        _tensor("state_indices", state_indices, device, (N,), (torch.int32,))
        _need(state.shape[0] >= 1, "the state pool needs at least one slot")
        _tensor("state", state, device, (state.shape[0], H, dk, dv), f32)
    else:
        _tensor("state", state, device, (N, H, dk, dv), f32)
    _tensor("o", o, device, (N, H, dv), f32, optional=True)


def _require_device(q):
    _need(isinstance(q, torch.Tensor) and q.device.type == "cuda",
          "inputs must be CUDA (HIP) tensors: the operator runs only in libkda's GPU kernels")

DEFAULT_CHUNK = 32


def make_fwd_args(q, k, v, g, beta, cu_dev, cu_host, scale, initial_state, final_state, checkpoint_every,
                  checkpoints, o, chunk_size=DEFAULT_CHUNK, initial_state_indices=None, checkpoint_indices=None,
                  num_slots=0, gate_preactivation=False, normalize_qk=False, segment_tokens=0):
    validate_fwd(q, k, v, g, beta, cu_host, cu_dev, initial_state, final_state, checkpoints, o,
                 initial_state_indices, checkpoint_indices, num_slots, checkpoint_every, gate_preactivation)
    T, H, dk = q.shape
    a = KdaFwdArgs()
    a.struct_size = ctypes.sizeof(KdaFwdArgs)
    a.num_seqs = int(cu_host.numel() - 1)
    a.total_tokens = int(T)
    a.num_heads = int(H)
    a.dk = int(dk)
    a.dv = int(v.shape[2])
    a.chunk_size = int(chunk_size)
    a.in_dtype = _dtype_code(q)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.cu_seqlens = _ptr(cu_dev)
    a.cu_seqlens_host = cu_host.data_ptr()
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state)
    a.checkpoint_every = int(checkpoint_every)
    a.checkpoints = _ptr(checkpoints)
    a.o = _ptr(o)
    a.initial_state_indices = _ptr(initial_state_indices)
    a.checkpoint_indices = _ptr(checkpoint_indices)
    a.num_slots = int(num_slots)
    a.gate_mode = KDA_GATE_PREACTIVATION if gate_preactivation else KDA_GATE_LOG_DECAY
    a.normalize_qk = 1 if normalize_qk else 0
    a.segment_tokens = int(segment_tokens)
    return a


def kda_chunk_fwd(q, k, v, g, beta, cu_seqlens=None, scale=1.0, initial_state=None, output_final_state=True,
                  checkpoint_every=0, stream=None, chunk_size=DEFAULT_CHUNK, initial_state_indices=None,
                  state_pool=None, checkpoint_indices=None, gate_preactivation=False, normalize_qk=False,
                  noalloc=False, segment_tokens=0):
    """Chunked KDA prefill (packed varlen).

    q, k: [T, H, dk]; v: [T, H, dv] (bf16 or fp32, CUDA, contiguous); g: [T, H, dk] fp32;
    beta: [T, H] fp32; cu_seqlens: int sequence offsets [N+1] (list / CPU or CUDA tensor,
    None = one sequence); initial_state: fp32 [N, H, dk, dv] or None.
    chunk_size: token block of the chunked form, 32 (software-pipelined kernel) or 64.
    Paged state pool: with state_pool fp32 [P, H, dk, dv], initial_state_indices int32 [N]
    (CUDA; -1 = zeros) picks each sequence's initial state from the pool (initial_state is then
    ignored), and checkpoint_indices int32 [M] (CUDA; -1 = not written) writes checkpoint m
    into pool slot checkpoint_indices[m] instead of returning a checkpoint tensor.
    Prologue (bf16 inputs; fused into the kernel at chunk_size 32 and dk 128, a pass of its own
    otherwise): gate_preactivation=True takes g as bf16 pre-activations a and beta as fp32
    pre-activations b (g = -5 sigmoid(a), beta = sigmoid(b)); normalize_qk=True L2-normalises
    q and k per (token, head) inside the operator.
    noalloc=True calls kda_chunk_fwd_noalloc instead: no workspace (the library's static launch-plan
    array, at most NOALLOC_MAX_SEQS sequences); the outputs are still allocated here.
    segment_tokens: context parallelism inside the GPU (chunk_size 32): 0 lets the library cut
    few, long sequences into segments that run side by side, -1 never cuts, > 0 cuts every that
    many tokens (a multiple of 32 and of checkpoint_every).
    Returns (o [T,H,dv] fp32, final_state [N,H,dk,dv] fp32 or None, checkpoints or None).
    """
    _require_device(q)
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    if cu_seqlens is None:
        cu_host = torch.tensor([0, T], dtype=torch.int32)
    elif isinstance(cu_seqlens, torch.Tensor):
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    else:
        cu_host = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    cu_dev = cu_host.to(dev)
    N = cu_host.numel() - 1
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    ck = None
    if checkpoint_every and checkpoint_indices is None:
        M = int(((cu_host[1:] - cu_host[:-1]) // checkpoint_every).sum())
        ck = torch.empty((M, H, dk, dv), dtype=torch.float32, device=dev)
    s0 = state_pool if initial_state_indices is not None else initial_state
    ck_arg = state_pool if checkpoint_indices is not None else ck
    nslots = int(state_pool.shape[0]) if state_pool is not None else 0
    a = make_fwd_args(q, k, v, g, beta, cu_dev, cu_host, scale, s0, sf, checkpoint_every, ck_arg, o,
                      chunk_size, initial_state_indices, checkpoint_indices, nslots, gate_preactivation,
                      normalize_qk, segment_tokens)
    L = lib()
    if noalloc:
        _check(L.kda_chunk_fwd_noalloc(ctypes.byref(a), _stream(stream)))
        return o, sf, ck
    ws_bytes = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
    if ws_bytes == 0 and N > 0:
        # invalid arguments: let the entry point report the precise status
        _check(L.kda_chunk_fwd(ctypes.byref(a), None, 0, _stream(stream)))
    ws = torch.empty(max(int(ws_bytes), 256), dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_fwd(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                           _stream(stream)))
    return o, sf, ck


def _cu_host(cu_seqlens, T):
    if cu_seqlens is None:
        return torch.tensor([0, T], dtype=torch.int32)
    if isinstance(cu_seqlens, torch.Tensor):
        return cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    return torch.tensor(list(cu_seqlens), dtype=torch.int32)


def make_bwd_args(q, k, v, g, beta, cu_dev, cu_host, scale, initial_state, d_o, d_final_state, dq, dk, dv, dg,
                  dbeta, d_initial_state, gate_preactivation=False, normalize_qk=False, states=None):
    validate_bwd(q, k, v, g, beta, d_o, cu_host, cu_dev, initial_state, d_final_state, states,
                 (dq, dk, dv, dg, dbeta, d_initial_state), gate_preactivation)
    T, H, dk_ = q.shape
    a = KdaBwdArgs()
    a.struct_size = ctypes.sizeof(KdaBwdArgs)
    a.num_seqs = int(cu_host.numel() - 1)
    a.total_tokens = int(T)
    a.num_heads = int(H)
    a.dk = int(dk_)
    a.dv = int(v.shape[2])
    a.in_dtype = _dtype_code(q)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.cu_seqlens = _ptr(cu_dev)
    a.cu_seqlens_host = cu_host.data_ptr()
    a.initial_state = _ptr(initial_state)
    a.d_o = _ptr(d_o)
    a.d_final_state = _ptr(d_final_state)
    a.dq, a.dk_out, a.dv_out, a.dg, a.dbeta = (_ptr(x) for x in (dq, dk, dv, dg, dbeta))
    a.d_initial_state = _ptr(d_initial_state)
    a.gate_mode = KDA_GATE_PREACTIVATION if gate_preactivation else KDA_GATE_LOG_DECAY
    a.normalize_qk = 1 if normalize_qk else 0
    a.states = _ptr(states)
    return a


def kda_chunk_bwd(q, k, v, g, beta, d_o, cu_seqlens=None, scale=1.0, initial_state=None, d_final_state=None,
                  output_d_initial_state=True, stream=None, workspace=None, gate_preactivation=False,
                  normalize_qk=False, states=None, workspace_cap=None):
    """Backward of kda_chunk_fwd: gradients of L = sum(d_o * o) + sum(d_final_state * final_state).

    Inputs as for kda_chunk_fwd (with gate_preactivation / normalize_qk as there: g, beta are then
    the gate pre-activations and q, k the raw vectors, and the returned dg, dbeta, dq, dk are the
    gradients with respect to those); d_o: fp32 [T, H, dv]; d_final_state: fp32 [N, H, dk, dv] or
    None (zeros).  workspace: optional uint8 CUDA tensor of at least the queried size (reused by
    callers that run the backward repeatedly).  states: the forward's checkpoints with
    checkpoint_every=32 (fp32 [sum floor(L/32), H, dk, dv]) to read instead of recomputing them, or
    None.  A given workspace smaller than the library's minimum (the longest sequence's need) is
    replaced by one allocated here.  workspace_cap: when the workspace is allocated here, at most
    this many bytes (never less than that minimum): the library then runs the batch in groups of
    sequences that fit.  Returns (dq, dk, dv, dg, dbeta, d_initial_state or None), all fp32."""
    _require_device(q)
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    cu_host = _cu_host(cu_seqlens, T)
    cu_dev = cu_host.to(dev)
    N = cu_host.numel() - 1
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dkk, dg = (torch.empty((T, H, dk), **f32) for _ in range(3))
    dvv = torch.empty((T, H, dv), **f32)
    db = torch.empty((T, H), **f32)
    ds0 = torch.empty((N, H, dk, dv), **f32) if output_d_initial_state else None
    a = make_bwd_args(q, k, v, g, beta, cu_dev, cu_host, scale, initial_state, d_o, d_final_state, dq, dkk, dvv,
                      dg, db, ds0, gate_preactivation, normalize_qk, states)
    L = lib()
    ws_bytes = int(L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a)))
    if ws_bytes == 0 and N > 0:
        _check(L.kda_chunk_bwd(ctypes.byref(a), None, 0, _stream(stream)))
    if workspace is not None:
        _tensor("workspace", workspace, dev, None, (torch.uint8,))
    least = int(L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a)))
    if workspace is None or workspace.numel() < least:
        # (a given workspace of at least the minimum is used as it is: the library then runs the
        # batch in groups of sequences if it is below the whole batch's need)
        if workspace_cap is not None:
            ws_bytes = min(ws_bytes, max(int(workspace_cap), least))
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_bwd(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                           ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return dq, dkk, dvv, dg, db, ds0


def make_decode_args(q, k, v, g, beta, state, o, scale, state_indices=None, gate_preactivation=False,
                     normalize_qk=False):
    validate_decode(q, k, v, g, beta, state, o, state_indices, gate_preactivation)
    N, H, dk = q.shape
    a = KdaDecodeArgs()
    a.struct_size = ctypes.sizeof(KdaDecodeArgs)
    a.num_seqs = int(N)
    a.num_heads = int(H)
    a.dk = int(dk)
    a.dv = int(v.shape[2])
    a.in_dtype = _dtype_code(q)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.state = _ptr(state)
    a.state_indices = _ptr(state_indices)
    a.o = _ptr(o)
    a.num_slots = int(state.shape[0]) if state_indices is not None else 0
    a.gate_mode = KDA_GATE_PREACTIVATION if gate_preactivation else KDA_GATE_LOG_DECAY
    a.normalize_qk = 1 if normalize_qk else 0
    return a


def kda_decode_step(q, k, v, g, beta, state, scale=1.0, out=None, stream=None, state_indices=None,
                    gate_preactivation=False, normalize_qk=False):
    """One decode token per sequence; `state` [N,H,dk,dv] fp32 is updated in place.  With
    state_indices (int32 [N], CUDA), `state` is a pool [P,H,dk,dv] and sequence n uses slot
    state_indices[n] (-1: inactive, o = 0).  gate_preactivation / normalize_qk: the prologue,
    as in kda_chunk_fwd (bf16 inputs).  Returns o [N, H, dv] fp32."""
    _require_device(q)
    N, H, dk = q.shape
    o = out if out is not None else torch.empty((N, H, v.shape[2]), dtype=torch.float32, device=q.device)
    a = make_decode_args(q, k, v, g, beta, state, o, scale, state_indices, gate_preactivation, normalize_qk)
    _check(lib().kda_decode_step(ctypes.byref(a), _stream(stream)))
    return o
