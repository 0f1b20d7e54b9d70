"""Helpers shared by the GPU parity tests (not collected: no test_ prefix)."""
import math
import multiprocessing as mp

import numpy as np


def sum_sq(x, rows=1 << 16):
    """sum(x^2) of a torch tensor in fp64, a slice of the first axis at a time (the whole tensor
    in fp64 may not fit the device)."""
    return sum(float((x[i:i + rows].double() ** 2).sum()) for i in range(0, x.shape[0], rows)) if x.numel() else 0.0


def dot(a, b, rows=1 << 16):
    """sum(a * b) of two torch tensors of one shape in fp64, a slice of the first axis at a time."""
    assert a.shape == b.shape
    return sum(float((a[i:i + rows].double() * b[i:i + rows].double()).sum()) for i in range(0, a.shape[0], rows))


def identity_bar(terms, sigmas=6.0):
    """Bar for |sum_i <a_i, b_i> - sum_j <c_j, d_j>| when each GPU-computed tensor a carries an
    elementwise error of size at most e_a * RMS(a) (e_a: its measured max|diff| / RMS against the
    oracle) and the errors of different elements are independent: the error of <a, b> then has a
    standard deviation of at most e_a * RMS(a) * sqrt(sum b^2).  terms: [(a, b, e_a), ...] with
    numpy arrays or torch tensors (reduced in fp64 where they live); returns `sigmas` times the
    sum of those deviations."""
    tot = 0.0
    for a, b, e in terms:
        if a.size == 0 if isinstance(a, np.ndarray) else a.numel() == 0:
            continue
        if isinstance(a, np.ndarray):
            a64, b64 = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
            rms_a, l2_b = math.sqrt(float(np.mean(a64 * a64))), math.sqrt(float(np.sum(b64 * b64)))
        else:
            rms_a = math.sqrt(sum_sq(a) / a.numel())
            l2_b = math.sqrt(sum_sq(b))
        tot += e * rms_a * l2_b
    return sigmas * tot


def _one_head_backward(args):
    from oracle import backward as OB
    return OB.backward(*args)


def oracle_backward_heads(q, k, v, g, beta, cu, scale, s0, do, dsf, heads, workers=4):
    """oracle.backward on each listed head alone, in `workers` freshly spawned processes (the
    oracle keeps every state of a chain: about 8.6 GB per 65,536-token head at d = 128).
    Returns {head: (dq, dk, dv, dg, dbeta, dS0)} for that head, each with a head axis of 1."""
    def sl(x, h):
        return None if x is None else np.ascontiguousarray(x[:, h:h + 1])
    jobs = [(sl(q, h), sl(k, h), sl(v, h), sl(g, h), sl(beta, h), list(cu), scale, sl(s0, h), sl(do, h), sl(dsf, h))
            for h in heads]
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(workers, len(jobs))) as pool:
        res = pool.map(_one_head_backward, jobs)
    return dict(zip(heads, res))
