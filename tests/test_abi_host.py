"""Host-side tests of the C ABI (no GPU): the library loads, exports every
symbol include/kda.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_49_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_49_amd import build
        build.build()
    return kda.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert kda.kda_abi_version() == 7 == kda.ABI_VERSION
    for code, name in enumerate(["KDA_OK", "KDA_ERR_INVALID_ARGUMENT", "KDA_ERR_UNSUPPORTED",
                                 "KDA_ERR_WORKSPACE_TOO_SMALL", "KDA_ERR_DEVICE"]):
        assert kda.kda_status_str(code) == name
    assert kda.kda_status_str(99) == "KDA_ERR_UNKNOWN"


STRUCTS = (("kda_fwd_args", kda.KdaFwdArgs), ("kda_decode_args", kda.KdaDecodeArgs),
           ("kda_bwd_args", kda.KdaBwdArgs))


def test_struct_layouts_match_header(tmp_path):
    """Every field offset and the size of each argument struct, as compiled from
    include/kda.h by the C compiler, equal the ctypes layouts of the binding."""
    import subprocess
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "kda.h"', "int main(void) {"]
    for cname, pyt in STRUCTS:
        prog.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in pyt._fields_:
            prog.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    prog.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, pyt in STRUCTS:
        assert got[(cname, "size")] == ctypes.sizeof(pyt)
        for f, _ in pyt._fields_:
            assert got[(cname, f)] == getattr(pyt, f).offset, (cname, f)


FAKE = 0x10000  # 64 KiB-aligned fake device address: never dereferenced by host validation


def fwd_args(**over):
    cu = over.pop("cu", [0, 100, 228])
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    a = kda.KdaFwdArgs()
    a.struct_size = ctypes.sizeof(kda.KdaFwdArgs)
    a.num_seqs = len(cu) - 1
    a.total_tokens = cu[-1]
    a.num_heads = 4
    a.dk = a.dv = 128
    a.chunk_size = 64
    a.in_dtype = kda.KDA_BF16
    a.scale = 1.0
    a.q, a.k, a.v, a.g, a.beta, a.o = (FAKE * (i + 1) for i in range(6))
    a.cu_seqlens = FAKE * 8
    a.cu_seqlens_host = ctypes.cast(cu_arr, ctypes.c_void_p).value
    a.checkpoint_every = 0
    for key, val in over.items():
        setattr(a, key, val)
    return a, cu_arr


def status(L, a, ws=FAKE * 16, ws_bytes=1 << 20):
    return L.kda_chunk_fwd(ctypes.byref(a), ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("field,value,expect", [
    ("struct_size", 8, kda.KDA_ERR_INVALID_ARGUMENT),
    ("num_heads", 0, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dk", 96, kda.KDA_ERR_UNSUPPORTED),
    ("dv", 64, kda.KDA_ERR_UNSUPPORTED),
    ("chunk_size", 16, kda.KDA_ERR_UNSUPPORTED),
    ("chunk_size", 128, kda.KDA_ERR_UNSUPPORTED),
    ("in_dtype", 7, kda.KDA_ERR_INVALID_ARGUMENT),
    ("q", None, kda.KDA_ERR_INVALID_ARGUMENT),
    ("g", FAKE + 4, kda.KDA_ERR_INVALID_ARGUMENT),          # misaligned
    ("o", FAKE * 1, kda.KDA_ERR_INVALID_ARGUMENT),          # aliases q
    ("checkpoint_every", 100, kda.KDA_ERR_INVALID_ARGUMENT),
    ("checkpoint_every", 96, kda.KDA_ERR_INVALID_ARGUMENT),   # not a multiple of chunk_size 64
    ("checkpoint_every", 64, kda.KDA_ERR_INVALID_ARGUMENT),  # checkpoints pointer missing
    ("total_tokens", 227, kda.KDA_ERR_INVALID_ARGUMENT),
    ("scale", float("nan"), kda.KDA_ERR_INVALID_ARGUMENT),
    ("initial_state_indices", FAKE * 9, kda.KDA_ERR_INVALID_ARGUMENT),   # no pool size, no pool
    ("checkpoint_indices", FAKE * 9, kda.KDA_ERR_INVALID_ARGUMENT),      # no pool size
])
def test_fwd_validation(L, field, value, expect):
    a, keep = fwd_args(**{field: value})
    assert status(L, a) == expect
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0


def test_pool_validation(L):
    # indices need a pool size, the initial-state indices need the pool, and checkpoint
    # indices need checkpoints
    a, keep = fwd_args(initial_state_indices=FAKE * 9, num_slots=4)
    assert status(L, a) == kda.KDA_ERR_INVALID_ARGUMENT            # initial_state (the pool) missing
    a, keep = fwd_args(checkpoint_indices=FAKE * 9, num_slots=4)
    assert status(L, a) == kda.KDA_ERR_INVALID_ARGUMENT            # checkpoint_every is 0
    a, keep = fwd_args(initial_state_indices=FAKE * 9, initial_state=FAKE * 10, num_slots=0)
    assert status(L, a) == kda.KDA_ERR_INVALID_ARGUMENT
    a, keep = fwd_args(initial_state_indices=FAKE * 9, initial_state=FAKE * 10, num_slots=4)
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) > 0   # valid


@pytest.mark.parametrize("cu", [[1, 100], [0, 50, 40], [0, 100, 90, 228]])
def test_bad_cu_seqlens(L, cu):
    a, keep = fwd_args(cu=cu)
    a.total_tokens = cu[-1]
    assert status(L, a) == kda.KDA_ERR_INVALID_ARGUMENT


def test_workspace_checks(L):
    a, keep = fwd_args()
    need = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
    assert need >= 2 * (4 + 8) and need % 256 == 0
    assert status(L, a, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert status(L, a, ws=0) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert status(L, a, ws=FAKE * 16 + 64, ws_bytes=need) == kda.KDA_ERR_INVALID_ARGUMENT  # unaligned
    # workspace grows with the number of sequences, not with tokens
    b, keep2 = fwd_args(cu=[0] + [10 * (i + 1) for i in range(300)])
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(b)) > need


@pytest.mark.parametrize("field", ["gate_mode", "normalize_qk"])
def test_fwd_prologue_needs_bf16(L, field):
    a, keep = fwd_args(**{field: 1, "in_dtype": kda.KDA_F32})
    assert status(L, a) == kda.KDA_ERR_UNSUPPORTED
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0


def test_fwd_prologue_workspace(L):
    """Fused into the kernel at chunk 32 and d_k = 128 (no extra workspace); at other shapes the
    prologue's outputs are materialised: fp32 q_n, k_n, v with the normalisation, g, beta with
    the gate."""
    rows = 228 * 4
    plain = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(fwd_args(chunk_size=32)[0]))
    both = dict(gate_mode=kda.KDA_GATE_PREACTIVATION, normalize_qk=1)
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(fwd_args(chunk_size=32, **both)[0])) == plain
    for over in (dict(chunk_size=64), dict(chunk_size=32, dk=64, dv=64)):
        d = over.get("dk", 128)
        base = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(fwd_args(**over)[0]))
        a, keep = fwd_args(**over, **both)
        need = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
        assert need >= base + rows * (3 * d * 4 + d * 4 + 4)
        assert status(L, a, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
        g = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(fwd_args(**over, gate_mode=1)[0]))
        n = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(fwd_args(**over, normalize_qk=1)[0]))
        assert base < g < need and base < n < need


def test_empty_batch_is_a_no_op(L):
    a, keep = fwd_args(cu=[0])
    a.num_seqs, a.total_tokens = 0, 0
    assert status(L, a, ws=0, ws_bytes=0) == kda.KDA_OK


def decode_args(**over):
    a = kda.KdaDecodeArgs()
    a.struct_size = ctypes.sizeof(kda.KdaDecodeArgs)
    a.num_seqs, a.num_heads, a.dk, a.dv = 8, 4, 128, 128
    a.in_dtype = kda.KDA_BF16
    a.scale = 1.0
    a.q, a.k, a.v, a.g, a.beta, a.state, a.o = (FAKE * (i + 1) for i in range(7))
    a.state_indices = None
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,expect", [
    ("struct_size", 4, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dk", 32, kda.KDA_ERR_UNSUPPORTED),
    ("state_indices", FAKE * 9, kda.KDA_ERR_INVALID_ARGUMENT),   # pool without num_slots
    ("state", None, kda.KDA_ERR_INVALID_ARGUMENT),
    ("state", FAKE + 8, kda.KDA_ERR_INVALID_ARGUMENT),
    ("o", FAKE * 6, kda.KDA_ERR_INVALID_ARGUMENT),          # aliases state
    ("num_heads", -1, kda.KDA_ERR_INVALID_ARGUMENT),
    ("gate_mode", 2, kda.KDA_ERR_INVALID_ARGUMENT),
    ("normalize_qk", -1, kda.KDA_ERR_INVALID_ARGUMENT),
])
def test_decode_validation(L, field, value, expect):
    a = decode_args(**{field: value})
    assert L.kda_decode_step(ctypes.byref(a), None) == expect


@pytest.mark.parametrize("field", ["gate_mode", "normalize_qk"])
def test_decode_prologue_needs_bf16(L, field):
    a = decode_args(**{field: 1, "in_dtype": kda.KDA_F32})
    assert L.kda_decode_step(ctypes.byref(a), None) == kda.KDA_ERR_UNSUPPORTED


def test_decode_empty_is_a_no_op(L):
    a = decode_args(num_seqs=0)
    assert L.kda_decode_step(ctypes.byref(a), None) == kda.KDA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        kda.lib()


def bwd_args(**over):
    cu = over.pop("cu", [0, 100, 228])
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    a = kda.KdaBwdArgs()
    a.struct_size = ctypes.sizeof(kda.KdaBwdArgs)
    a.num_seqs = len(cu) - 1
    a.total_tokens = cu[-1]
    a.num_heads = 4
    a.dk = a.dv = 128
    a.in_dtype = kda.KDA_BF16
    a.scale = 1.0
    a.q, a.k, a.v, a.g, a.beta, a.d_o = (FAKE * (i + 1) for i in range(6))
    a.dq, a.dk_out, a.dv_out, a.dg, a.dbeta = (FAKE * (i + 20) for i in range(5))
    a.cu_seqlens = FAKE * 8
    a.cu_seqlens_host = ctypes.cast(cu_arr, ctypes.c_void_p).value
    for key, val in over.items():
        setattr(a, key, val)
    return a, cu_arr


def bwd_status(L, a, ws=FAKE * 64, ws_bytes=1 << 40):
    return L.kda_chunk_bwd(ctypes.byref(a), ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("field,value,expect", [
    ("struct_size", 8, kda.KDA_ERR_INVALID_ARGUMENT),
    ("num_heads", 0, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dk", 96, kda.KDA_ERR_UNSUPPORTED),
    ("dv", 64, kda.KDA_ERR_UNSUPPORTED),
    ("in_dtype", 5, kda.KDA_ERR_INVALID_ARGUMENT),
    ("d_o", None, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dg", None, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dbeta", FAKE * 30 + 4, kda.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    ("dq", FAKE * 1, kda.KDA_ERR_INVALID_ARGUMENT),           # aliases q
    ("dv_out", FAKE * 20, kda.KDA_ERR_INVALID_ARGUMENT),      # aliases dq
    ("d_initial_state", FAKE * 6, kda.KDA_ERR_INVALID_ARGUMENT),   # aliases d_o
    ("total_tokens", 229, kda.KDA_ERR_INVALID_ARGUMENT),
    ("scale", float("nan"), kda.KDA_ERR_INVALID_ARGUMENT),
    ("gate_mode", 5, kda.KDA_ERR_INVALID_ARGUMENT),
    ("normalize_qk", 2, kda.KDA_ERR_INVALID_ARGUMENT),
    ("states", FAKE * 40 + 8, kda.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    ("states", FAKE * 21, kda.KDA_ERR_INVALID_ARGUMENT),       # aliases dk_out
])
def test_bwd_validation(L, field, value, expect):
    a, keep = bwd_args(**{field: value})
    assert bwd_status(L, a) == expect
    assert L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a)) == 0


@pytest.mark.parametrize("field", ["gate_mode", "normalize_qk"])
def test_bwd_prologue_needs_bf16(L, field):
    a, keep = bwd_args(**{field: 1, "in_dtype": kda.KDA_F32})
    assert bwd_status(L, a) == kda.KDA_ERR_UNSUPPORTED
    assert L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a)) == 0


def test_bwd_prologue_workspace(L):
    # the prologue's outputs are materialised: fp32 q_n, k_n and v with the normalisation, fp32 g
    # and beta with the gate
    base = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(bwd_args()[0]))
    a, keep = bwd_args(gate_mode=kda.KDA_GATE_PREACTIVATION, normalize_qk=1)
    need = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a))
    rows = 228 * 4
    assert need >= base + rows * (3 * 128 * 4 + 128 * 4 + 4)
    assert bwd_status(L, a, ws_bytes=need - 1) == kda.KDA_ERR_DEVICE   # groups of sequences
    assert bwd_status(L, a, ws_bytes=L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a)) - 1) == \
        kda.KDA_ERR_WORKSPACE_TOO_SMALL
    g, keep2 = bwd_args(gate_mode=kda.KDA_GATE_PREACTIVATION)
    n, keep3 = bwd_args(normalize_qk=1)
    assert base < L.kda_chunk_bwd_workspace_bytes(ctypes.byref(g)) < need
    assert base < L.kda_chunk_bwd_workspace_bytes(ctypes.byref(n)) < need


def test_bwd_given_states_workspace(L):
    # states passed in (the forward's checkpoints every 32 tokens): the workspace holds none
    base = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(bwd_args()[0]))
    a, keep = bwd_args(states=FAKE * 40)
    need = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a))
    n_ck = 100 // 32 + 128 // 32
    assert need <= base - n_ck * 4 * 128 * 128 * 4
    assert bwd_status(L, a, ws_bytes=L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a)) - 1) == \
        kda.KDA_ERR_WORKSPACE_TOO_SMALL


def test_bwd_workspace(L):
    # one sequence of 100 tokens (3 checkpoints, 4 chunks) and one of 128 (4 and 4), 4 heads, d = 128
    a, keep = bwd_args()
    need = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a))
    # checkpoints (7) and per chunk (8): D, W, E, A and T
    expect = (7 * 4 * 128 * 128 + 8 * 4 * (128 * 128 + 2 * 32 * 128 + 2 * 32 * 32)) * 4
    assert need % 256 == 0 and need >= expect
    assert bwd_status(L, a, ws_bytes=L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a)) - 1) == \
        kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert bwd_status(L, a, ws=0, ws_bytes=need) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert bwd_status(L, a, ws=FAKE * 64 + 128, ws_bytes=need) == kda.KDA_ERR_INVALID_ARGUMENT
    b, keep2 = bwd_args(cu=[0])
    b.num_seqs, b.total_tokens = 0, 0
    assert bwd_status(L, b, ws=0, ws_bytes=0) == kda.KDA_OK


# ---- the allocation-free forward (host-side refusals; no launch) ----------------------------
@pytest.mark.parametrize("field,value,expect", [
    ("struct_size", 8, kda.KDA_ERR_INVALID_ARGUMENT),
    ("dk", 96, kda.KDA_ERR_UNSUPPORTED),
    ("q", None, kda.KDA_ERR_INVALID_ARGUMENT),
    ("total_tokens", 227, kda.KDA_ERR_INVALID_ARGUMENT),
])
def test_noalloc_validates_like_the_workspace_entry_point(L, field, value, expect):
    a, keep = fwd_args(**{field: value})
    assert L.kda_chunk_fwd_noalloc(ctypes.byref(a), None) == expect == status(L, a)


def test_noalloc_refuses_more_sequences_than_its_array_holds(L):
    # an empty batch of NOALLOC_MAX_SEQS + 1 sequences: valid for kda_chunk_fwd, too many here
    cu = [0] * (kda.NOALLOC_MAX_SEQS + 2)
    a, keep = fwd_args(cu=cu)
    assert L.kda_chunk_fwd_noalloc(ctypes.byref(a), None) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) > 0


def test_noalloc_refuses_a_prologue_that_needs_a_workspace(L):
    # outside chunk 32 / d_k 128 the prologue runs as a pass whose outputs need caller memory
    for over in (dict(gate_mode=kda.KDA_GATE_PREACTIVATION), dict(normalize_qk=1),
                 dict(gate_mode=kda.KDA_GATE_PREACTIVATION, dk=64, dv=64, chunk_size=32)):
        a, keep = fwd_args(**over)
        assert L.kda_chunk_fwd_noalloc(ctypes.byref(a), None) == kda.KDA_ERR_UNSUPPORTED


def test_noalloc_empty_batch_is_a_no_op(L):
    a, keep = fwd_args(cu=[0])
    assert L.kda_chunk_fwd_noalloc(ctypes.byref(a), None) == kda.KDA_OK


def test_segment_choice(L):
    """The library cuts sequences into segments (segment_tokens 0) only when the (sequence, head)
    pairs leave most of the chip idle and the longest sequence spans at least 3 segments; the
    workspace then holds 3 states per (segment, head) (the two runs' final states, the entry state)
    and the transition runs' outputs (4 dk bytes per token and head) on top of the segments' plan.
    Without a GPU the library assumes 256 compute units."""
    state = 128 * 128 * 4

    def ws(cu, H, **over):
        a, keep = fwd_args(cu=cu, num_heads=H, chunk_size=32, **over)
        return L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))

    one = [0, 4096]
    # 4,096 tokens on 32 heads: 256 / (2 * 32) = 4 segments of 1,024 tokens
    assert ws(one, 32) >= ws(one, 32, segment_tokens=-1) + 4 * 32 * 3 * state + 4096 * 32 * 128 * 4
    assert ws(one, 32) == ws(one, 32, segment_tokens=1024)
    # 96 heads fill the chip with two workgroups per pair: no cut; nor for 64 sequences x 32 heads
    assert ws(one, 96) == ws(one, 96, segment_tokens=-1)
    many = list(range(0, 65 * 512, 512))
    assert ws(many, 32) == ws(many, 32, segment_tokens=-1)
    # too short to gain: 1,024 tokens would give 512-token segments, only 2 of them
    assert ws([0, 1024], 32) == ws([0, 1024], 32, segment_tokens=-1)
    # 1M tokens on 2 heads: 64 segments of 16,384 tokens
    big = [0, 1 << 20]
    assert ws(big, 2) == ws(big, 2, segment_tokens=16384) > ws(big, 2, segment_tokens=-1) + 64 * 2 * 3 * state
    # explicit cuts: the workspace grows with the number of segments
    assert ws(one, 32, segment_tokens=512) > ws(one, 32, segment_tokens=1024)
    # chunk 64 does not cut by itself, and refuses an explicit cut
    a, keep = fwd_args(cu=one, num_heads=32)
    b, keep2 = fwd_args(cu=one, num_heads=32, segment_tokens=-1)
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) == L.kda_chunk_fwd_workspace_bytes(ctypes.byref(b))
    a, keep = fwd_args(cu=one, num_heads=32, segment_tokens=1024)
    assert status(L, a) == kda.KDA_ERR_UNSUPPORTED


def test_bwd_workspace_groups(L):
    """A workspace below the whole batch's need, but at least the longest sequence's, is accepted:
    the batch then runs in groups of whole sequences (here the launch itself fails: no GPU).  The
    minimum is the longest sequence's own need, so it grows with that sequence, not the batch."""
    cu = [0, 100, 4196, 4228, 4228, 4356]   # lengths 100, 4096, 32, 0, 128
    a, keep = bwd_args(cu=cu)
    full = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a))
    least = L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a))
    b, keep2 = bwd_args(cu=[0, 4096])
    alone = L.kda_chunk_bwd_workspace_bytes(ctypes.byref(b))
    assert 0 < least < full
    assert alone <= least <= alone + 1024          # the 4096-token sequence alone (+ its offsets)
    assert bwd_status(L, a, ws_bytes=full) == kda.KDA_ERR_DEVICE
    assert bwd_status(L, a, ws_bytes=least) == kda.KDA_ERR_DEVICE
    assert bwd_status(L, a, ws_bytes=least - 256) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    # states given: the groups read their slices of them
    c, keep3 = bwd_args(cu=cu, states=FAKE * 40)
    assert bwd_status(L, c, ws_bytes=L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(c))) == kda.KDA_ERR_DEVICE
    # a single sequence: the minimum is the whole need
    assert L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(b)) == alone
    assert L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(bwd_args(num_heads=0)[0])) == 0   # invalid
