#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill of the long-context workload (T=65536 tokens,
H=96 heads, d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state, initial state) plus one
decode step of the decode workload (256 sequences x 96 heads, fp32 state
[256,96,128,128] updated in place).  Inputs are seeded synthetic data
(workloads.make_workload) resident in HBM before the timed region.

Prints ONE JSON line: value = prefill tokens/s; decode GB/s and the roofline
of the dominant kernel are reported beside it, and (each timed on its own after
the step) the prefill of the T=4096 and varlen workloads, the prefill through
the fused prologue and the backward on the prefill's shape; cpu_baseline times
the fp64 CPU oracle on a bounded sample of the prefill workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "KDA prefill tokens/s (H=96,d=128) + decode state-update HBM GB/s, 1 GPU"


def prefill_bytes(T, H, dk, dv, in_bytes=2, with_states=True):
    """Algorithmic HBM bytes of one prefill launch: read q,k,v,g,beta once, write o once,
    plus the initial/final states."""
    per_tok_head = in_bytes * (2 * dk + dv) + 4 * dk + 4 + 4 * dv
    return T * H * per_tok_head + (2 * H * dk * dv * 4 if with_states else 0)


def decode_bytes(N, H, dk, dv, in_bytes=2):
    """Algorithmic bytes of one decode step: state read + written once, token inputs, o."""
    return N * H * (2 * dk * dv * 4 + in_bytes * (2 * dk + dv) + 4 * dk + 4 + 4 * dv)


def prefill_flop_per_tokhead(C, dk, dv):
    """Algorithmic flops per token-head of the chunked form at chunk size C: the in-chunk Gram
    tiles, the triangular transform and the output assembly 2C(3 d_k + 2 d_v), plus the state
    read-outs and update 6 d_k d_v.  At C = 64 and d = 128 this is 180,224 (the count the
    roofline uses); at the kernel's C = 32 it is 139,264."""
    return 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv


ROOFLINE_CHUNK = 64   # the flop count of the roofline is the C = 64 one, whatever chunk the kernel runs


def roofline_bound(flop, nbytes):
    """The roofline that binds an algorithm of `flop` flops and `nbytes` HBM bytes on MI355X: HBM
    when its intensity is below the ridge point (peak bf16 flop/s over peak HBM bytes/s)."""
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return ("hbm" if flop / nbytes < ridge else "mfma"), flop / nbytes, ridge


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill (profiling runs)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the T=4096 H=32 and varlen timings that the default line carries")
    ap.add_argument("--chunk", type=int, default=32, choices=(32, 64), help="token block of the chunked form")
    ap.add_argument("--prologue", action="store_true",
                    help="with --workload 2 or --backward: fused gate/normalisation prologue (raw q, k, bf16 "
                         "gate pre-activations)")
    ap.add_argument("--workload", type=int, default=0, choices=(0, 1, 2, 4),
                    help="instead of the benchmark step, time the prefill of workload 1 (T=4096, H=32) or 4 "
                         "(64 packed sequences, H=32, checkpoints every 512) and print its own JSON line; with "
                         "--backward 4, the backward of workload 4 within a bounded workspace")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the benchmark step, time the backward (kda_chunk_bwd) on workload 2's shape "
                         "and print its own JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scales the HBM byte counters)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="only write the kernel-trace summaries under profiles/ from a rocprofv3 csv run of "
                         "bench.py and the JSON line that run printed")
    ap.add_argument("--summarize-backward-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="only write profiles/backward_T65536_H96_d128_kernel_trace.md from a rocprofv3 csv run of "
                         "bench.py --backward and the JSON line that run printed")
    ap.add_argument("--summarize-backward-counters", nargs=5, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE",
                                                                       "MFMA"),
                    help="only write profiles/backward_T65536_H96_d128_counters.md from five rocprofv3 --pmc "
                         "output folders of bench.py --backward (and the copy calibration)")
    ap.add_argument("--summarize-counters", nargs=7, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE", "MFMA",
                                                              "ISSUE", "STALL"),
                    help="only write the counter summaries of the prefill kernel and of the decode kernel under "
                         "profiles/ from seven rocprofv3 --pmc output folders (csv)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.chunk, *args.summarize_counters)
        summarize_decode_counters(*args.summarize_counters[:4])
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_backward_counters:
        summarize_backward_counters(*args.summarize_backward_counters)
        return
    if args.summarize_backward_trace:
        summarize_backward_trace(*args.summarize_backward_trace)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(the operator shards by head / sequence with no communication, "
                                   "but no multi-GPU path is built)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.backward and args.workload == 4:
        backward_varlen_workload(args.steps, args.warmup)
        return
    if args.backward:
        backward_workload(args.steps, args.warmup, args.prologue)
        return
    if args.workload:
        other_workload(args.workload, args.chunk, args.steps, args.warmup, args.prologue)
        return

    import gated_delta_rule_49_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    t_gen = time.time()
    wp = W.make_workload(2)
    wd = W.make_workload(3)
    gen_s = time.time() - t_gen

    def up(x, dt):
        return torch.from_numpy(x).to(dev, dt)

    bf = torch.bfloat16
    q, k, v = up(wp.q, bf), up(wp.k, bf), up(wp.v, bf)
    g, beta = up(wp.g, torch.float32), up(wp.beta, torch.float32)
    s0 = up(wp.s0, torch.float32)
    T, H, dk = wp.q.shape
    dv = wp.v.shape[2]
    cu_h = torch.tensor(list(wp.cu_seqlens), dtype=torch.int32)
    cu_d = cu_h.to(dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty_like(s0)
    A = kda.make_fwd_args(q, k, v, g, beta, cu_d, cu_h, 1.0, s0, sf, 0, None, o, args.chunk)
    L = kda.lib()
    ws_bytes = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(A))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    N, Hd, dkd = wd.q.shape
    dq, dk_, dvv = up(wd.q, bf), up(wd.k, bf), up(wd.v, bf)
    dg, db = up(wd.g, torch.float32), up(wd.beta, torch.float32)
    state = up(wd.s0, torch.float32)
    od = torch.empty((N, Hd, wd.v.shape[2]), dtype=torch.float32, device=dev)
    D = kda.make_decode_args(dq, dk_, dvv, dg, db, state, od, 1.0)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())

    def prefill():
        st = L.kda_chunk_fwd(ctypes.byref(A), wsp, wsn, sptr)
        if st != 0:
            raise RuntimeError(kda.kda_status_str(st))

    def decode():
        st = L.kda_decode_step(ctypes.byref(D), sptr)
        if st != 0:
            raise RuntimeError(kda.kda_status_str(st))

    for _ in range(args.warmup):
        prefill()
        if not args.prefill_only:
            decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        if not args.prefill_only:
            decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    pre_avg = float(np.mean(pre_ms))
    dec_avg = float(np.mean(dec_ms)) if not args.prefill_only else None

    tokens = T
    value = tokens / (pre_avg * 1e-3)
    pbytes = prefill_bytes(T, H, dk, dv)
    pflop = prefill_flop_per_tokhead(ROOFLINE_CHUNK, dk, dv) * T * H
    pflop_k = prefill_flop_per_tokhead(args.chunk, dk, dv) * T * H
    achieved_gbps = pbytes / (pre_avg * 1e-3) / 1e9
    bound, intensity, ridge = roofline_bound(pflop, pbytes)
    achieved_tflops = pflop / (pre_avg * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; workloads.make_workload 2 and 3)",
        "config": {"workload": "prefill T=65536 H=96 d_k=d_v=128 bf16 q/k/v, fp32 g/beta/state, initial state; "
                               "+ decode N=256 H=96 d=128 fp32 state in place",
                   "chunk": args.chunk, "tokens_per_step": T, "heads": H},
        "prefill": {"ms": round(pre_avg, 4), "ms_p10": round(float(np.percentile(pre_ms, 10)), 4),
                    "ms_p90": round(float(np.percentile(pre_ms, 90)), 4), "tokens_per_s": round(value, 1),
                    "alg_GBps": round(achieved_gbps, 1), "alg_bytes": pbytes,
                    "alg_flop_C64": pflop, "alg_TFLOPs_C64": round(achieved_tflops, 2),
                    f"alg_flop_C{args.chunk}": pflop_k,
                    f"alg_TFLOPs_C{args.chunk}": round(pflop_k / (pre_avg * 1e-3) / 1e12, 2),
                    "flop_note": "C64 = 180,224 flop per token-head (2C(3dk+2dv)+6dkdv at C=64, the roofline's "
                                 f"count); C{args.chunk} = the same formula at the chunk the kernel runs"},
        "roofline": {"kernel": KERNEL_NAME[args.chunk], "bound": bound,
                     "achieved": round(achieved_gbps if bound == "hbm" else achieved_tflops, 1),
                     "peak": HBM_PEAK_GBPS if bound == "hbm" else BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                     "frac": round(achieved_gbps / HBM_PEAK_GBPS if bound == "hbm" else
                                   achieved_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1)},
        "mfma": {"peak_TFLOPs": BF16_PEAK_TFLOPS, "alg_TFLOPs_C64": round(achieved_tflops, 2),
                 "alg_frac_of_peak": round(achieved_tflops / BF16_PEAK_TFLOPS, 4),
                 "busy_pct_executed": None, "executed_bf16_TFLOPs": None,
                 "note": "busy_pct_executed: rocprof SQ_VALU_MFMA_BUSY_CYCLES over all 1024 SIMDs (counts the "
                         "hi+lo split passes), from the committed counter summary while the kernel is unchanged"},
        "precision": "MFMA bf16 operands (hi+lo split pairs on all output-facing products), fp32 accumulate, "
                     "fp32 o and state",
        "gen_s": round(gen_s, 1),
    }
    if dec_avg is not None:
        dbytes = decode_bytes(N, Hd, dkd, dvv.shape[2])
        dgbps = dbytes / (dec_avg * 1e-3) / 1e9
        res["decode"] = {"ms": round(dec_avg, 4), "GBps": round(dgbps, 1), "alg_bytes": dbytes,
                         "frac_of_hbm_peak": round(dgbps / HBM_PEAK_GBPS, 4),
                         "ms_p10": round(float(np.percentile(dec_ms, 10)), 4),
                         "ms_p90": round(float(np.percentile(dec_ms, 90)), 4)}
        # the same decode through the paged pool: the state buffer as a pool of 256 slots,
        # sequence n in slot perm[n] (a seeded permutation); timed after the steps, not in them
        perm = torch.from_numpy(np.random.default_rng(3).permutation(N).astype(np.int32)).to(dev)
        Dp = kda.make_decode_args(dq, dk_, dvv, dg, db, state, od, 1.0, state_indices=perm)

        def decode_paged():
            st = L.kda_decode_step(ctypes.byref(Dp), sptr)
            if st != 0:
                raise RuntimeError(kda.kda_status_str(st))

        decode_paged()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            pev[i][0].record(stream)
            decode_paged()
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        pms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in pev]))
        res["decode"]["paged"] = {"ms": round(pms, 4), "GBps": round(dbytes / (pms * 1e-3) / 1e9, 1),
                                  "slots": "permutation of 256 pool slots"}
        # and through the prologue: bf16 gate pre-activations a, fp32 b (device draws), q and k
        # normalised inside; the g stream is 2 bytes per channel instead of 4
        gen = torch.Generator(device=dev)
        gen.manual_seed(4)
        a_pre = torch.randn(dg.shape, generator=gen, device=dev).to(torch.bfloat16)
        b_pre = torch.randn(db.shape, generator=gen, device=dev)
        Dq = kda.make_decode_args(dq, dk_, dvv, a_pre, b_pre, state, od, dkd ** -0.5, gate_preactivation=True,
                                  normalize_qk=True)

        def decode_prologue():
            st = L.kda_decode_step(ctypes.byref(Dq), sptr)
            if st != 0:
                raise RuntimeError(kda.kda_status_str(st))

        decode_prologue()
        qev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            qev[i][0].record(stream)
            decode_prologue()
            qev[i][1].record(stream)
        torch.cuda.synchronize()
        qms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in qev]))
        qbytes = dbytes - N * Hd * dkd * 2
        res["decode"]["prologue"] = {"ms": round(qms, 4), "GBps": round(qbytes / (qms * 1e-3) / 1e9, 1),
                                     "alg_bytes": qbytes,
                                     "inputs": "bf16 gate pre-activations, fp32 beta pre-activations, "
                                               "q and k normalised inside"}

    prof = measured_counters(args.chunk)
    if prof is not None:
        # HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE passes, scaled by the copy calibration;
        # only reported while the kernel sources still hash to what was profiled.
        res["roofline"]["traffic"] = prof["hbm_bytes_per_launch"]
        res["prefill"]["traffic_over_alg"] = round(prof["hbm_bytes_per_launch"] / pbytes, 3)
        for key in ("valu_busy_pct", "lds_busy_pct", "wait_any_over_wave_cycles"):
            if key in prof:
                res["prefill"][key] = prof[key]
        if "mfma_util_pct" in prof:
            res["mfma"]["busy_pct_executed"] = prof["mfma_util_pct"]
            res["mfma"]["executed_bf16_TFLOPs"] = round(prof["mfma_bf16_flop_per_launch"] / (pre_avg * 1e-3) / 1e12, 1)
        res["prefill"]["counters"] = prof["file"]

    if not args.prefill_only and not args.no_extra_workloads:
        # the other measured prefill workloads, each timed on its own after the step timing
        del q, k, v, g, beta, o, A, ws
        torch.cuda.empty_cache()
        for cid in (1, 4):
            r = other_workload(cid, args.chunk, max(5, min(K, 20)), 2, emit=False)
            res[f"workload_{cid}"] = {key: r[key] for key in ("workload", "tokens", "heads", "value", "unit", "ms",
                                                              "ms_p10", "ms_p90", "alg_GBps", "frac_of_hbm_peak",
                                                              "alg_bytes", "cache")}
            torch.cuda.empty_cache()
        if args.chunk == 32:
            # the prefill's shape through the fused prologue (raw q and k, bf16 gate pre-activations)
            r = other_workload(2, args.chunk, max(5, min(K, 20)), 2, prologue=True, emit=False)
            res["prefill"]["prologue"] = {"ms": r["ms"], "tokens_per_s": r["value"],
                                          "over_plain": round(r["ms"] / pre_avg, 4), "workload": r["workload"]}
            torch.cuda.empty_cache()
            # the backward (kda_chunk_bwd) on the prefill's shape, timed on its own
            r = backward_workload(max(3, min(K, 10)), 1, emit=False)
            res["backward"] = {key: r[key] for key in ("workload", "ms", "value", "unit", "alg_GBps",
                                                        "frac_of_hbm_peak", "workspace_GB")}
            res["backward"]["with_forward_states_ms"] = r["with_forward_states"]["ms"]
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wp, args.cpu_seconds, H, wd)
    print(json.dumps(res), flush=True)


KERNEL_NAME = {32: "chunk32_kernel<128,split2,bf16>", 64: "chunk_fwd_kernel<128,bf16>"}
KERNEL_SOURCES = {32: ["kda_chunk32.hip", "kda_frag.h", "kda_common.h"], 64: ["kda_chunk.hip", "kda_frag.h",
                                                                                  "kda_common.h"]}
COUNTER_FILE = {32: "chunk32_prefill_T65536_H96_d128_counters.json",
                64: "chunk64_prefill_T65536_H96_d128_counters.json"}


def kernel_digest(chunk):
    """Digest of the kernel's sources and of the compile flags they are built with."""
    import hashlib
    from gated_delta_rule_49_amd.build import SOURCE_FLAGS
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[chunk]:
        with open(os.path.join(ROOT, "gated_delta_rule_49_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
        h.update(repr(SOURCE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def measured_counters(chunk):
    """Counter figures for the prefill kernel from the committed profile summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", COUNTER_FILE[chunk])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != kernel_digest(chunk):
        return None
    d["file"] = "profiles/" + COUNTER_FILE[chunk]
    return d


def _counter_rows(folder, name_part, must=True):
    """Per-dispatch sums (over the whole chip) of each counter for kernels whose name contains
    name_part (none: an error, or with must=False an empty list)."""
    import csv
    import glob
    path = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not path:
        raise FileNotFoundError(f"no counter_collection.csv under {folder}")
    per = {}
    with open(path[0]) as f:
        for r in csv.DictReader(f):
            if name_part in r["Kernel_Name"]:
                d = per.setdefault(int(r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per and must:
        raise ValueError(f"no dispatch of a kernel matching {name_part!r} in {path[0]}")
    return list(per.values())


def _mean(rows, key):
    return sum(r[key] for r in rows) / len(rows)


COUNTER_STEP = "bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-extra-workloads"
ISSUE_COUNTERS = ("SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_INSTS_SALU SQ_WAVES "
                  "SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
STALL_COUNTERS = ("SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
                  "SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA "
                 "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def _copy_scales(cfetch_dir, cwrite_dir):
    """Bytes per counted byte of FETCH_SIZE and WRITE_SIZE (KiB per dispatch), from a plain copy that reads
    and writes `copy_bytes` per call (bench.py --copy-calibration 2048; its last three calls)."""
    copy_bytes = 2048 * (1 << 20)
    cf = _mean(_counter_rows(cfetch_dir, "elementwise_kernel")[-3:], "FETCH_SIZE")
    cw = _mean(_counter_rows(cwrite_dir, "elementwise_kernel")[-3:], "WRITE_SIZE")
    return copy_bytes, cf, cw, copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)


def summarize_counters(chunk, fetch_dir, write_dir, cfetch_dir, cwrite_dir, mfma_dir, issue_dir, stall_dir):
    """Write profiles/<kernel>_counters.json and .md for the prefill kernel: HBM bytes per launch from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for a plain
    copy of known size; MFMA busy and bf16 MOPS; VALU and LDS instruction counts and issue cycles; wait
    and LDS-conflict counters.  Busy fractions divide a per-SIMD cycle count by GRBM_GUI_ACTIVE (summed
    over the 8 XCDs, so / 8) times the 1024 SIMDs."""
    kname = {32: "chunk32_kernel<128, 2, false, unsigned short, 0>", 64: "chunk_fwd_kernel<128, false"}[chunk]
    fetch = _mean(_counter_rows(fetch_dir, kname), "FETCH_SIZE")
    write = _mean(_counter_rows(write_dir, kname), "WRITE_SIZE")
    copy_bytes, cf, cw, fs, ws = _copy_scales(cfetch_dir, cwrite_dir)
    xcd, simds = 8, 1024          # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs
    m = _counter_rows(mfma_dir, kname)
    gui = _mean(m, "GRBM_GUI_ACTIVE") / xcd
    busy, mops = _mean(m, "SQ_VALU_MFMA_BUSY_CYCLES"), _mean(m, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    iss = _counter_rows(issue_dir, kname)
    st = _counter_rows(stall_dir, kname)
    gi, gs = _mean(iss, "GRBM_GUI_ACTIVE") / xcd, _mean(st, "GRBM_GUI_ACTIVE") / xcd
    T, H = 65536, 96
    wg_chunks = T // 32 * H * 2 if chunk == 32 else T // 64 * H   # workgroup-chunks per launch (2 per chain)
    raw = {k: _mean(iss, k) for k in ISSUE_COUNTERS.split() if k != "GRBM_GUI_ACTIVE"}
    raw.update({k: _mean(st, k) for k in STALL_COUNTERS.split() if k != "GRBM_GUI_ACTIVE"})
    raw.update({"SQ_INSTS_MFMA": _mean(m, "SQ_INSTS_MFMA"), "SQ_VALU_MFMA_BUSY_CYCLES": busy,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops, "SQ_BUSY_CYCLES": _mean(m, "SQ_BUSY_CYCLES")})
    d = {
        "kernel": KERNEL_NAME[chunk],
        "workload": "prefill T=65536 H=96 d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state, initial state "
                    f"(bench.py prefill launch, chunk {chunk})",
        "source_digest": kernel_digest(chunk),
        "fetch_kib_per_launch": round(fetch, 1),
        "write_kib_per_launch": round(write, 1),
        "copy_calibration": {"bytes_read_and_written": copy_bytes, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
        "hbm_read_bytes_per_launch": round(fetch * 1024 * fs),
        "hbm_write_bytes_per_launch": round(write * 1024 * ws),
        "hbm_bytes_per_launch": round(fetch * 1024 * fs + write * 1024 * ws),
        "mfma_bf16_flop_per_launch": round(mops * 512),
        "mfma_busy_cycles": busy,
        "gui_active_cycles_per_xcd": gui,
        "mfma_util_pct": round(100.0 * busy / (gui * simds), 2),
        # SQ_ACTIVE_INST_* and SQ_WAVE_CYCLES / SQ_WAIT_* count 4-cycle units (one wave64 VALU
        # instruction issues in 4 cycles: ACTIVE_INST_VALU ~ INSTS_VALU); SQ_VALU_MFMA_BUSY_CYCLES counts cycles
        "valu_busy_pct": round(100.0 * 4 * raw["SQ_ACTIVE_INST_VALU"] / (gi * simds), 2),
        "lds_busy_pct": round(100.0 * 4 * raw["SQ_ACTIVE_INST_LDS"] / (gi * simds), 2),
        "issue_fraction_of_wave_time": round(raw["SQ_ACTIVE_INST_ANY"] / max(raw["SQ_WAVE_CYCLES"], 1), 4),
        "workgroup_chunks_per_launch": wg_chunks,
        "per_workgroup_chunk": {"valu_insts": round(raw["SQ_INSTS_VALU"] / wg_chunks, 1),
                                "lds_insts": round(raw["SQ_INSTS_LDS"] / wg_chunks, 1),
                                "salu_insts": round(raw["SQ_INSTS_SALU"] / wg_chunks, 1),
                                "mfma_insts": round(raw["SQ_INSTS_MFMA"] / wg_chunks, 1)},
        "lds_bank_conflict_per_lds_active": round(raw["SQ_LDS_BANK_CONFLICT"] / max(raw["SQ_LDS_IDX_ACTIVE"], 1), 4),
        "wait_inst_any_over_wave_cycles": round(raw["SQ_WAIT_INST_ANY"] / max(raw["SQ_WAVE_CYCLES"], 1), 4),
        "wait_any_over_wave_cycles": round(raw["SQ_WAIT_ANY"] / max(raw["SQ_WAVE_CYCLES"], 1), 4),
        "raw_counters_per_launch": {k: round(v) for k, v in raw.items()},
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- python3 {COUNTER_STEP}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 {COUNTER_STEP}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfetch_dir} -o run -- python3 bench.py "
            "--copy-calibration 2048",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwrite_dir} -o run -- python3 bench.py "
            "--copy-calibration 2048",
            f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d {mfma_dir} -o run -- python3 {COUNTER_STEP} "
            "--prefill-only",
            f"rocprofv3 --pmc {ISSUE_COUNTERS} --output-format csv -d {issue_dir} -o run -- python3 {COUNTER_STEP} "
            "--prefill-only",
            f"rocprofv3 --pmc {STALL_COUNTERS} --output-format csv -d {stall_dir} -o run -- python3 {COUNTER_STEP} "
            "--prefill-only",
            f"python3 bench.py --chunk {chunk} --summarize-counters {fetch_dir} {write_dir} {cfetch_dir} "
            f"{cwrite_dir} {mfma_dir} {issue_dir} {stall_dir}",
        ],
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    base = os.path.join(ROOT, "profiles", COUNTER_FILE[chunk])
    with open(base, "w") as f:
        json.dump(d, f, indent=1)
    alg = prefill_bytes(65536, 96, 128, 128)
    pw = d["per_workgroup_chunk"]
    with open(base[:-5] + ".md", "w") as f:
        f.write(f"# {d['kernel']}: HBM traffic, issue and MFMA counters\n\n")
        f.write(f"Workload: {d['workload']}.  Kernel source digest {d['source_digest']}.\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| FETCH_SIZE / WRITE_SIZE per launch | {d['fetch_kib_per_launch']} / {d['write_kib_per_launch']} KiB |\n")
        f.write(f"| copy calibration: FETCH_SIZE / WRITE_SIZE for {copy_bytes} B read + written | "
                f"{d['copy_calibration']['fetch_kib']} / {d['copy_calibration']['write_kib']} KiB |\n")
        f.write(f"| scale factors (bytes per counted byte) | fetch {fs:.4f}, write {ws:.4f} |\n")
        f.write(f"| HBM bytes read / written per launch | {d['hbm_read_bytes_per_launch']} / "
                f"{d['hbm_write_bytes_per_launch']} |\n")
        f.write(f"| algorithmic bytes per launch | {alg} |\n")
        f.write(f"| measured / algorithmic | {d['hbm_bytes_per_launch'] / alg:.3f} |\n")
        f.write(f"| MFMA bf16 flop per launch (MOPS x 512) | {d['mfma_bf16_flop_per_launch']:.4g} |\n")
        f.write(f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE/8 x 1024 SIMDs)) | {d['mfma_util_pct']} % |\n")
        f.write(f"| VALU busy (4 x SQ_ACTIVE_INST_VALU, 4-cycle units, same normalisation) | {d['valu_busy_pct']} % |\n")
        f.write(f"| LDS busy (4 x SQ_ACTIVE_INST_LDS, same normalisation) | {d['lds_busy_pct']} % |\n")
        f.write(f"| share of wave time issuing any instruction (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES) | "
                f"{d['issue_fraction_of_wave_time']} |\n")
        f.write(f"| per workgroup-chunk ({wg_chunks} per launch): VALU / LDS / SALU / MFMA instructions | "
                f"{pw['valu_insts']} / {pw['lds_insts']} / {pw['salu_insts']} / {pw['mfma_insts']} |\n")
        f.write(f"| LDS bank conflicts per LDS-active cycle | {d['lds_bank_conflict_per_lds_active']} |\n")
        f.write(f"| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waves waiting on a dependency) | "
                f"{d['wait_inst_any_over_wave_cycles']} |\n")
        f.write(f"| SQ_WAIT_ANY / SQ_WAVE_CYCLES (waves waiting on anything, barriers included) | "
                f"{d['wait_any_over_wave_cycles']} |\n\n")
        f.write("Raw counters per launch (sums over the chip, averaged over the profiled launches):\n\n")
        for k, v in d["raw_counters_per_launch"].items():
            f.write(f"    {k} = {v}\n")
        f.write("\nCommands (each counter group in its own run):\n\n")
        for c in d["commands"]:
            f.write(f"    {c}\n")
    print(json.dumps(d, indent=1))


def summarize_decode_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """Write profiles/decode_N256_H96_d128_counters.md: HBM bytes of the decode step (the timed launch of
    the plain path) from the same FETCH_SIZE / WRITE_SIZE passes as the prefill, calibrated as there."""
    kname = "decode_kernel<128, 128, unsigned short, 0>"
    fr, wr = _counter_rows(fetch_dir, kname), _counter_rows(write_dir, kname)
    fetch, write = _mean(fr, "FETCH_SIZE"), _mean(wr, "WRITE_SIZE")
    copy_bytes, cf, cw, fs, ws = _copy_scales(cfetch_dir, cwrite_dir)
    rd, wt = fetch * 1024 * fs, write * 1024 * ws
    alg = decode_bytes(256, 96, 128, 128)
    with open(os.path.join(ROOT, "profiles", "decode_N256_H96_d128_counters.md"), "w") as f:
        f.write(f"# {kname}: HBM traffic\n\n")
        f.write("Workload: decode step N=256 H=96 d_k=d_v=128 (bf16 q/k/v, fp32 g/beta, fp32 state [256,96,128,128] "
                f"in place).  Averaged over its {len(fr)} dispatches in the profiled run.\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| FETCH_SIZE / WRITE_SIZE per launch | {fetch:.1f} / {write:.1f} KiB |\n")
        f.write(f"| scale factors from a plain copy of {copy_bytes} B read + written | fetch {fs:.4f}, write {ws:.4f} |\n")
        f.write(f"| HBM bytes read / written per launch | {rd:.0f} / {wt:.0f} |\n")
        f.write(f"| algorithmic bytes per launch (state read + written once, token inputs, o) | {alg} |\n")
        f.write(f"| measured / algorithmic | {(rd + wt) / alg:.3f} |\n\n")
        f.write("Commands (the first two are the prefill summary's FETCH / WRITE passes; the step runs one prefill "
                "and one decode step per iteration):\n\n")
        for c in (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- python3 {COUNTER_STEP}",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 {COUNTER_STEP}",
                  f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfetch_dir} -o run -- python3 bench.py "
                  "--copy-calibration 2048",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwrite_dir} -o run -- python3 bench.py "
                  "--copy-calibration 2048",
                  f"python3 bench.py --summarize-counters {fetch_dir} {write_dir} {cfetch_dir} {cwrite_dir} ..."):
            f.write(f"    {c}\n")
    print(f"decode: read {rd:.4g} B, written {wt:.4g} B, measured/alg {(rd + wt) / alg:.3f}")


def summarize_backward_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir, mfma_dir):
    """Write profiles/backward_T65536_H96_d128_counters.md: per backward kernel, HBM bytes per launch
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size) and fp32 MFMA busy."""
    copy_bytes = 2048 * (1 << 20)
    cf = _mean(_counter_rows(cfetch_dir, "elementwise_kernel")[-3:], "FETCH_SIZE")
    cw = _mean(_counter_rows(cwrite_dir, "elementwise_kernel")[-3:], "WRITE_SIZE")
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    # (the recompute is the states-only variant of the chunk kernel, flag 4; the run's other
    # chunk32 launch is the forward that provides the states for the second timing)
    # (the state-gradient scan is whichever of its two forms the library chose for this batch)
    scan = "bwd_dscan_hl_kernel<128" if _counter_rows(fetch_dir, "bwd_dscan_hl_kernel<128", must=False) \
        else "bwd_dstate_kernel<128"
    # (the recompute takes one workgroup per chain when it runs beside the one-workgroup scan)
    rec = "chunk32_kernel<128, 1, false, unsigned short, 4" \
        if _counter_rows(fetch_dir, "chunk32_kernel<128, 1, false, unsigned short, 4", must=False) \
        else "chunk32_kernel<128, 2, false, unsigned short, 4"
    kernels = [(rec, "forward recompute (checkpoint every 32)"),
               ("bwd_prep_kernel<128", "prep"), (scan, "state-gradient scan"),
               ("bwd_grad_kernel<128", "gradients")]
    xcd, simds = 8, 1024
    lines = []
    for kn, role in kernels:
        f = _mean(_counter_rows(fetch_dir, kn), "FETCH_SIZE") * 1024 * fs
        w = _mean(_counter_rows(write_dir, kn), "WRITE_SIZE") * 1024 * ws
        m = _counter_rows(mfma_dir, kn)
        busy, gui = _mean(m, "SQ_VALU_MFMA_BUSY_CYCLES"), _mean(m, "GRBM_GUI_ACTIVE")
        lines.append(f"| `{kn}...>` ({role}) | {f / 1e9:.2f} | {w / 1e9:.2f} | "
                     f"{100.0 * busy / (gui / xcd * simds):.1f} % |\n")
    cmd = "python3 bench.py --backward --steps 1 --warmup 0"
    with open(os.path.join(ROOT, "profiles", "backward_T65536_H96_d128_counters.md"), "w") as f:
        f.write("# Backward (kda_chunk_bwd): HBM traffic and MFMA counters\n\n")
        f.write("Workload: backward of the prefill T=65536 H=96 d_k=d_v=128, bf16 q/k/v, fp32 g/beta, initial "
                "state, d_o and dS_T (one `bench.py --backward` call).  Per dispatch: prep, scan and gradient "
                "kernels also run once more reading the forward's states, with the same work.\n\n")
        f.write(f"HBM bytes = counter x scale, scales from a plain copy of {copy_bytes} B read + written: "
                f"fetch {fs:.4f}, write {ws:.4f}.  MFMA busy over all 1024 SIMDs (fp32 MFMA, and bf16 hi+lo "
                "products in the gradient kernel and the forward recompute).\n\n")
        f.write("| kernel | HBM read (GB) | HBM written (GB) | MFMA busy |\n|---|---|---|---|\n")
        for ln in lines:
            f.write(ln)
        f.write("\nCommands (each counter group in its own run):\n\n")
        for c in (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- {cmd}",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- {cmd}",
                  f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfetch_dir} -o run -- python3 bench.py "
                  "--copy-calibration 2048",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwrite_dir} -o run -- python3 bench.py "
                  "--copy-calibration 2048",
                  f"rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
                  f"GRBM_GUI_ACTIVE --output-format csv -d {mfma_dir} -o run -- {cmd}",
                  f"python3 bench.py --summarize-backward-counters {fetch_dir} {write_dir} {cfetch_dir} "
                  f"{cwrite_dir} {mfma_dir}"):
            f.write(f"    {c}\n")
    print("wrote profiles/backward_T65536_H96_d128_counters.md")


def summarize_trace(trace_dir, bench_json):
    """Write profiles/*_kernel_trace.md (one per hot kernel) from a rocprofv3 --kernel-trace --stats
    csv run of bench.py, next to the per-launch durations bench.py measured with HIP events."""
    import csv
    import glob
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    with open(path) as f:
        rows = list(csv.DictReader(f))
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- python3 bench.py "
           f"--steps {b['steps']} --warmup {b['warmup']} --no-cpu-baseline --no-extra-workloads "
           f"--chunk {b['config']['chunk']}")
    table = "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |\n|---|---|---|---|---|---|\n"
    for r in rows:
        table += (f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} % |\n")
    out = {
        "chunk32_prefill_T65536_H96_d128_kernel_trace.md": (
            "prefill T=65536 H=96 d_k=d_v=128 (bf16 q/k/v, fp32 g/beta/state, initial state)",
            "chunk32_kernel<128, 2, false, unsigned short, 0>", b["prefill"]["ms"]),
        "decode_N256_H96_d128_kernel_trace.md": (
            "decode step N=256 H=96 d_k=d_v=128 (bf16 q/k/v, fp32 g/beta, fp32 state in place)",
            "decode_kernel<128, 128, unsigned short, 0>", b.get("decode", {}).get("ms")),
    }
    # per-dispatch durations, in launch order, to average over the timed launches only (the
    # warm-up launches come first; the paged and prologue decode launches after the timed steps)
    tpath = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    disp = []
    if tpath:
        with open(tpath[0]) as f:
            disp = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                           for r in csv.DictReader(f)), key=lambda x: x[0])
    for fname, (wl, kname, ev_ms) in out.items():
        avg = [float(r["AverageNs"]) for r in rows if kname in r["Name"]]
        durs = [e - s_ for s_, e, n in disp if kname in n][b["warmup"]:b["warmup"] + b["steps"]]
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write(f"# {kname}: rocprofv3 kernel trace\n\nWorkload: {wl}.\n\n")
            if avg:
                f.write(f"rocprofv3 average duration of {kname} over all its dispatches: {avg[0] / 1e6:.4f} ms")
                if durs:
                    f.write(f"; over the {len(durs)} timed launches (warm-up excluded): "
                            f"{sum(durs) / len(durs) / 1e6:.4f} ms")
                f.write(f".  bench.py HIP-event average over the timed steps (same process): {ev_ms} ms.\n\n")
            f.write(f"Command:\n\n    {cmd}\n\nAll kernels of the run:\n\n{table}")
    print("wrote", ", ".join(out))


def summarize_backward_trace(trace_dir, bench_log):
    """Write profiles/backward[_prologue]_T65536_H96_d128_kernel_trace.md: per-kernel rocprofv3
    averages of a `bench.py --backward [--prologue]` run under --kernel-trace --stats, next to that
    run's event-timed total."""
    import csv
    import glob
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    # the backward's kernels: its own, the launch plan and the states-only recompute (flags >= 4);
    # the run's plain forward (which provides the states for the second timing) is left out
    def ours(name):
        if "kda" not in name:
            return False
        if "chunk32_kernel" in name:
            return int(name.split(">")[0].split(",")[-1]) >= 4
        return True
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if ours(r["Name"])]
    with open(bench_log) as f:
        b = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    fused = "fused" in b["workload"]
    name = "backward_prologue_T65536_H96_d128_kernel_trace.md" if fused else "backward_T65536_H96_d128_kernel_trace.md"
    total = sum(float(r["AverageNs"]) for r in rows) / 1e6
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("# Backward (kda_chunk_bwd" + (", fused gate / normalisation prologue" if fused else "")
                + "): rocprofv3 kernel trace\n\n")
        f.write(f"Workload: {b['workload']}.\n\n")
        f.write(f"bench.py HIP-event median of one backward (same process): {b['ms']} ms "
                f"({b['value']:.0f} tokens/s); sum of the per-kernel rocprof averages below: {total:.3f} ms (prep, scan and gradient kernels "
                "averaged over both timings, recomputing and reading the forward's states: the same work).  "
                "When the scan takes one workgroup per chain on few chains, the states-only recompute "
                "(`chunk32_kernel<..., 4>`) runs on a second stream beside the scan, so their times overlap "
                "and the sum exceeds the wall time.\n\n")
        f.write("Command:\n\n    rocprofv3 --kernel-trace --stats -d " + trace_dir + " -o run --output-format csv "
                "-- python -u bench.py --backward " + ("--prologue " if fused else "") + "--steps 5 --warmup 1\n\n")
        f.write("| kernel | calls | average (ms) | min (ms) | max (ms) |\n|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                    f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} |\n")
    print("wrote profiles/" + name)


def other_workload(cid, chunk, steps, warmup, prologue=False, emit=True):
    """Prefill tokens/s of workload 1 or 4 (one JSON line).  Workload 1 uses the seeded host
    generator; workload 4 (about 1.85M tokens x 32 heads, ~110 GB with o and checkpoints) is drawn
    on the device with torch's seeded generator from the same distributions (lengths from the
    seeded host draw), since only timing, not parity, is taken from it."""
    import numpy as np
    import torch
    import gated_delta_rule_49_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    pro = {}
    if cid == 2:
        # workload 2's shape with raw inputs for the fused prologue: q, k ~ N(0,1) unnormalised,
        # bf16 gate pre-activations a ~ N(0,1), fp32 b ~ N(0,1); drawn on the device
        T, H, dk, dv = 65536, 96, 128, 128
        seqlens = [T]
        gen = torch.Generator(device=dev)
        gen.manual_seed(20261203)
        q = torch.randn((T, H, dk), generator=gen, device=dev).to(bf)
        k = torch.randn((T, H, dk), generator=gen, device=dev).to(bf)
        v = torch.randn((T, H, dv), generator=gen, device=dev).to(bf)
        if prologue:
            g = torch.randn((T, H, dk), generator=gen, device=dev).to(bf)
            beta = torch.randn((T, H), generator=gen, device=dev)
            pro = dict(gate_preactivation=True, normalize_qk=True)
        else:
            q = (q.float() / q.float().norm(dim=-1, keepdim=True) * dk ** -0.5).to(bf)
            k = (k.float() / k.float().norm(dim=-1, keepdim=True)).to(bf)
            g = -5.0 * torch.sigmoid(torch.randn((T, H, dk), generator=gen, device=dev))
            beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=dev))
        s0 = 0.1 * torch.randn((1, H, dk, dv), generator=gen, device=dev)
        every = 0
        desc = ("prefill T=65536 H=96 d_k=d_v=128 bf16 q/k/v, initial state; " +
                ("fused prologue: bf16 gate pre-activations, fp32 beta pre-activations, q and k "
                 "normalised inside" if prologue else "fp32 g/beta, normalised q/k"))
    elif cid == 1:
        w = W.make_workload(1)
        up = lambda x, dt: torch.from_numpy(x).to(dev, dt)
        q, k, v = up(w.q, bf), up(w.k, bf), up(w.v, bf)
        g, beta = up(w.g, torch.float32), up(w.beta, torch.float32)
        seqlens = list(w.seqlens)
        H, dk, dv = w.H, w.dk, w.dv
        s0 = None
        every = 0
        desc = "prefill T=4096 H=32 d_k=d_v=128 bf16 q/k/v, fp32 g/beta, zero initial state"
    else:
        seqlens = W.varlen_lengths()
        H, dk, dv = 32, 128, 128
        T = int(sum(seqlens))
        gen = torch.Generator(device=dev)
        gen.manual_seed(20261203)
        q = torch.empty((T, H, dk), dtype=bf, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((T, H, dv), dtype=bf, device=dev)
        g = torch.empty((T, H, dk), dtype=torch.float32, device=dev)
        beta = torch.empty((T, H), dtype=torch.float32, device=dev)
        step = 1 << 16
        for a in range(0, T, step):
            b = min(T, a + step)
            x = torch.randn((b - a, H, dk), generator=gen, device=dev)
            q[a:b] = (x / x.norm(dim=-1, keepdim=True) * dk ** -0.5).to(bf)
            x = torch.randn((b - a, H, dk), generator=gen, device=dev)
            k[a:b] = (x / x.norm(dim=-1, keepdim=True)).to(bf)
            v[a:b] = torch.randn((b - a, H, dv), generator=gen, device=dev).to(bf)
            g[a:b] = -5.0 * torch.sigmoid(torch.randn((b - a, H, dk), generator=gen, device=dev))
            beta[a:b] = torch.sigmoid(torch.randn((b - a, H), generator=gen, device=dev))
        s0 = 0.1 * torch.randn((len(seqlens), H, dk, dv), generator=gen, device=dev)
        every = 512
        desc = (f"varlen prefill, {len(seqlens)} packed sequences (log-uniform 512..131072, T={T}), H=32, "
                "d_k=d_v=128 bf16 q/k/v, fp32 g/beta, per-sequence initial state, checkpoints every 512")
    T = int(sum(seqlens))
    cu_h = torch.tensor([0] + list(np.cumsum(seqlens)), dtype=torch.int32)
    cu_d = cu_h.to(dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty((len(seqlens), H, dk, dv), dtype=torch.float32, device=dev)
    n_ck = sum(L // every for L in seqlens) if every else 0
    ck = torch.empty((max(n_ck, 1), H, dk, dv), dtype=torch.float32, device=dev) if n_ck else None
    A = kda.make_fwd_args(q, k, v, g, beta, cu_d, cu_h, (dk ** -0.5) if pro else 1.0, s0, sf, every, ck, o,
                          chunk, **pro)
    L = kda.lib()
    ws = torch.empty(L.kda_chunk_fwd_workspace_bytes(ctypes.byref(A)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def prefill():
        st = L.kda_chunk_fwd(ctypes.byref(A), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), sptr)
        if st != 0:
            raise RuntimeError(kda.kda_status_str(st))

    for _ in range(warmup):
        prefill()
    torch.cuda.synchronize()
    # Workload 1's inputs and outputs (about 235 MB) fit in the 256 MB Infinity Cache: a 512 MB
    # buffer is written between timed calls (outside the events) so that each call starts cold.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cid == 1 else None
    ms = []
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        prefill()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = float(np.median(ms))
    nbytes = prefill_bytes(T, H, dk, dv, with_states=False) + len(seqlens) * H * dk * dv * 4 * (2 if s0 is not None else 1) \
        + n_ck * H * dk * dv * 4 - (T * H * dk * 2 if pro else 0)   # a bf16 gate stream: 2 B per channel less
    out = {
        "metric": "KDA prefill tokens/s", "workload": desc, "tokens": T, "heads": H, "chunk": chunk,
        "cache": "cold (512 MB written between calls)" if flush is not None else "inputs larger than the caches",
        "value": round(T / (med * 1e-3), 1), "unit": "tokens/s", "ms": round(med, 4),
        "ms_p10": round(float(np.percentile(ms, 10)), 4), "ms_p90": round(float(np.percentile(ms, 90)), 4),
        "alg_bytes": int(nbytes), "alg_GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "data": "synthetic (seeded)"}
    del q, k, v, g, beta, o, sf, ck, ws, A, flush
    if emit:
        print(json.dumps(out), flush=True)
    return out


def bwd_alg_bytes(T, H, dk, dv, N, fused=False, in_bytes=2):
    """Algorithmic HBM bytes of one backward: read q, k, v, g (bf16 pre-activations when fused),
    beta, d_o and the initial / final-state gradient inputs once, write dq, dk, dv, dg, dbeta and
    dS_0 once (fp32 gradients)."""
    per_tok_head = in_bytes * (2 * dk + dv) + (2 if fused else 4) * dk + 4 + 4 * dv + 4 * (3 * dk + dv + 1)
    return T * H * per_tok_head + 3 * N * H * dk * dv * 4


def backward_workload(steps, warmup, fused=False, emit=True):
    """Backward tokens/s on workload 2's shape (one sequence, T=65536, H=96, d=128, bf16 q/k/v,
    initial state, d_o and dS_T upstream gradients), inputs drawn on the device with torch's seeded
    generator from the workload distributions (timing only).  With fused, the inputs are the raw
    ones of the fused prologue (q, k ~ N(0,1) unnormalised, bf16 gate pre-activations a ~ N(0,1),
    b ~ N(0,1)) and the gradients are taken through the gate and the normalisation."""
    import numpy as np
    import torch
    import gated_delta_rule_49_amd as kda

    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    T, H, dk, dv = 65536, 96, 128, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    rn = lambda *shape: torch.randn(shape, generator=gen, device=dev)
    scale = 1.0
    if fused:
        q, k = rn(T, H, dk).to(bf), rn(T, H, dk).to(bf)
        v = rn(T, H, dv).to(bf)
        g, beta = rn(T, H, dk).to(bf), rn(T, H)
        scale = dk ** -0.5
    else:
        x = rn(T, H, dk)
        q = (x / x.norm(dim=-1, keepdim=True) * dk ** -0.5).to(bf)
        x = rn(T, H, dk)
        k = (x / x.norm(dim=-1, keepdim=True)).to(bf)
        del x
        v = rn(T, H, dv).to(bf)
        g = -5.0 * torch.sigmoid(rn(T, H, dk))
        beta = torch.sigmoid(rn(T, H))
    s0 = 0.1 * rn(1, H, dk, dv)
    do = rn(T, H, dv)
    dsf = rn(1, H, dk, dv)
    cu = [0, T]
    ws = torch.empty(0, dtype=torch.uint8, device=dev)
    out = None

    def run():
        nonlocal out, ws
        out = kda.kda_chunk_bwd(q, k, v, g, beta, do, cu, scale, s0, dsf, workspace=ws, gate_preactivation=fused,
                                normalize_qk=fused)

    run()
    torch.cuda.synchronize()
    # reuse one workspace (the binding allocates one per call when none is passed)
    ws = torch.empty(_bwd_ws_bytes(kda, q, k, v, g, beta, do, cu, s0, dsf, out, fused), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = float(np.median(ms))
    # the same backward reading the forward's states at every 32-token boundary (a forward run
    # with checkpoint_every = 32, untimed) instead of recomputing them
    _, _, states = kda.kda_chunk_fwd(q, k, v, g, beta, cu, scale, s0, False, 32, chunk_size=32,
                                     gate_preactivation=fused, normalize_qk=fused)
    ms_s = []
    for _ in range(max(1, steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.kda_chunk_bwd(q, k, v, g, beta, do, cu, scale, s0, dsf, workspace=ws, gate_preactivation=fused,
                          normalize_qk=fused, states=states)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_s.append(e0.elapsed_time(e1))
    med_s = float(np.median(ms_s))
    del states
    nbytes = bwd_alg_bytes(T, H, dk, dv, 1, fused)
    what = ("raw bf16 q/k/v, bf16 gate pre-activations a, fp32 b, gradients through the fused gate and "
            "q/k normalisation" if fused else "bf16 q/k/v, fp32 g/beta")
    r = {
        "metric": "KDA backward tokens/s", "workload": "backward of the prefill T=65536 H=96 d_k=d_v=128 "
                                                      + what + ", initial state, d_o and dS_T",
        "tokens": T, "heads": H, "value": round(T / (med * 1e-3), 1), "unit": "tokens/s", "ms": round(med, 4),
        "ms_p10": round(float(np.percentile(ms, 10)), 4), "ms_p90": round(float(np.percentile(ms, 90)), 4),
        "alg_bytes": int(nbytes), "alg_GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "workspace_GB": round(ws.numel() / 1e9, 2),
        "with_forward_states": {"ms": round(med_s, 4), "tokens_per_s": round(T / (med_s * 1e-3), 1),
                                "note": "the forward's checkpoints every 32 tokens passed in, not recomputed"},
        "data": "synthetic (seeded)"}
    if emit:
        print(json.dumps(r), flush=True)
    return r


BWD_VARLEN_CAP = 36 << 30   # workspace of the varlen backward: the library runs it in groups of sequences


def backward_varlen_workload(steps, warmup):
    """Backward tokens/s on workload 4's shape (64 packed sequences, 1,853,952 tokens, H=32, d=128,
    bf16 q/k/v, per-sequence initial states, d_o and dS_T) in one call within a 36 GiB workspace
    (the whole batch at once would need about ten times that): the library runs it in groups of
    whole sequences.  Inputs drawn on the device with torch's seeded generator (timing only)."""
    import numpy as np
    import torch
    import gated_delta_rule_49_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    lens = W.varlen_lengths()
    T, N, H, dk, dv = sum(lens), len(lens), 32, 128, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261204)
    rn = lambda *shape: torch.randn(shape, generator=gen, device=dev)
    q = torch.empty((T, H, dk), dtype=bf, device=dev)
    k = torch.empty_like(q)
    for dst, sc in ((q, dk ** -0.5), (k, 1.0)):
        for i in range(0, T, 1 << 17):   # in slices: the fp32 draw of the whole tensor is 30 GB
            x = rn(min(T - i, 1 << 17), H, dk)
            dst[i:i + x.shape[0]] = (x / x.norm(dim=-1, keepdim=True) * sc).to(bf)
    del x
    v = torch.empty((T, H, dv), dtype=bf, device=dev)
    for i in range(0, T, 1 << 17):
        v[i:i + (1 << 17)] = rn(min(T - i, 1 << 17), H, dv).to(bf)
    g = rn(T, H, dk)
    g.sigmoid_().mul_(-5.0)
    beta = torch.sigmoid(rn(T, H))
    s0 = 0.1 * rn(N, H, dk, dv)
    do = rn(T, H, dv)
    dsf = rn(N, H, dk, dv)
    cu = [0] + list(np.cumsum(lens))
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dkk, dg = (torch.empty((T, H, dk), **f32) for _ in range(3))
    dvv, db, ds0 = torch.empty((T, H, dv), **f32), torch.empty((T, H), **f32), torch.empty((N, H, dk, dv), **f32)
    cu_h = torch.tensor(cu, dtype=torch.int32)
    cu_d = cu_h.to(dev)
    a = kda.make_bwd_args(q, k, v, g, beta, cu_d, cu_h, 1.0, s0, do, dsf, dq, dkk, dvv, dg, db, ds0)
    L = kda.lib()
    full = int(L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a)))
    least = int(L.kda_chunk_bwd_workspace_min_bytes(ctypes.byref(a)))
    ws = torch.empty(max(least, min(full, BWD_VARLEN_CAP)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        kda._check(L.kda_chunk_bwd(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                   ctypes.c_void_p(stream.cuda_stream)))

    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = float(np.median(ms))
    nbytes = bwd_alg_bytes(T, H, dk, dv, N)
    print(json.dumps({
        "metric": "KDA backward tokens/s", "workload": "backward of the varlen prefill: 64 sequences, "
                                                      f"{T} tokens, H=32 d_k=d_v=128 bf16 q/k/v, fp32 g/beta, "
                                                      "per-sequence initial states, d_o and dS_T",
        "tokens": T, "heads": H, "value": round(T / (med * 1e-3), 1), "unit": "tokens/s", "ms": round(med, 4),
        "ms_min": round(min(ms), 4), "alg_bytes": int(nbytes), "alg_GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "workspace_GB": round(ws.numel() / 1e9, 2), "workspace_whole_batch_GB": round(full / 1e9, 2),
        "workspace_min_GB": round(least / 1e9, 2), "data": "synthetic (seeded)"}), flush=True)


def _bwd_ws_bytes(kda, q, k, v, g, beta, do, cu, s0, dsf, out, fused=False):
    import torch
    cu_h = torch.tensor(cu, dtype=torch.int32)
    a = kda.make_bwd_args(q, k, v, g, beta, cu_h.to(q.device), cu_h, 1.0, s0, do, dsf, *out,
                          gate_preactivation=fused, normalize_qk=fused)
    return int(kda.lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(a)))


def copy_calibration(mib):
    """A plain elementwise copy of known size (reads and writes `mib` MiB each call)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "calls": 3}), flush=True)


def cpu_baseline(wp, target_s, H_full, wd=None):
    """fp64 oracle on a bounded sample of the prefill workload: the first `Ts` tokens of `Hs`
    heads (one chain per thread), sized from a short calibration run to take about target_s
    seconds; when all tokens of `cores` heads are quicker than that, more heads (up to all of
    them), and when the whole workload is, whole-workload runs repeated.  Reported as
    equivalent tokens/s for all H_full heads.  With wd (the decode workload), also the oracle's
    decode step over all of its states, as algorithmic GB/s.  The oracle runs on
    oracle.default_threads() threads: the host CPUs this process may use, at most 16 (the CPU
    share of one GPU on a shared host); both counts are reported."""
    import numpy as np

    import oracle
    cores = oracle.default_threads()
    host_cpus = len(os.sched_getaffinity(0))
    T, H = wp.q.shape[0], wp.q.shape[1]

    def run(Ts, Hs, threads=cores):
        sl = (slice(0, Ts), slice(0, Hs))
        t = time.perf_counter()
        oracle.forward(wp.q[sl], wp.k[sl], wp.v[sl], wp.g[sl], wp.beta[sl], None, 1.0,
                       None if wp.s0 is None else wp.s0[:, :Hs], n_threads=threads)
        return time.perf_counter() - t

    # one chain on one thread, a fixed slice: the per-core rate
    one = min(T, 4096)
    single = one / run(one, 1, 1)

    Hs = min(cores, H)
    cal_T = 512
    cal = run(cal_T, Hs)
    while cal < 0.5 and cal_T < T:
        cal_T *= 2
        cal = run(cal_T, Hs)
    Ts = int(min(T, max(cal_T, cal_T * target_s / max(cal, 1e-3))))
    reps = 1
    if Ts == T:
        per_head_round = cal * T / cal_T          # all tokens of one round of `cores` heads
        rounds = max(1, min(-(-H // Hs), int(target_s / max(per_head_round, 1e-3))))
        Hs = min(H, Hs * rounds)
        if Hs == H:
            reps = max(1, int(target_s / max(per_head_round * -(-H // cores), 1e-3)))
    el = sum(run(Ts, Hs) for _ in range(reps))
    tokhead_per_s = reps * Ts * Hs / el
    out = {"value": round(tokhead_per_s / H_full, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "host_cpus_available": host_cpus,
           "threads_note": f"{cores} threads: the host CPUs available to this process ({host_cpus}), capped at 16, "
                           "the CPU share of one GPU",
           "single_thread_token_heads_per_s": round(single, 1),
           "sample": f"first {Ts} tokens x {Hs} heads of the T=65536 H=96 prefill (fp64 C recurrence, "
                     f"{Hs} chains on {cores} threads), {reps} run(s), {el:.1f} s; "
                     f"value = token-heads/s / 96; single thread: the first {one} tokens of head 0",
           "seconds": round(el, 2)}
    if wd is not None:
        N, Hd, dkd = wd.q.shape
        t = time.perf_counter()
        oracle.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.s0, 1.0, n_threads=cores)
        dt = time.perf_counter() - t
        nb = decode_bytes(N, Hd, dkd, wd.v.shape[2])
        out["decode"] = {"GBps": round(nb / dt / 1e9, 2), "seconds": round(dt, 2), "alg_bytes": nb,
                         "sample": f"one decode step of all {N} x {Hd} states (fp64 C, {cores} threads; the "
                                   "time includes the oracle's conversion of the fp32 inputs)"}
    return out


if __name__ == "__main__":
    main()
