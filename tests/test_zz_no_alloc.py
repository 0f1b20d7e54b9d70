"""kda_chunk_fwd_noalloc, the forward that allocates nothing (its launch plan lives in the
library's static device array), through the C ABI: bit-identical to kda_chunk_fwd on the same
inputs, and within the bf16-path bar of the fp64 oracle, on two calls in a row, the second
with a smaller batch (the array keeps the first call's plan, which the second must overwrite)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def run(w, every, chunk, noalloc):
    dev = torch.device("cuda:0")
    to = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dev, dt)
    bf = torch.bfloat16
    out = kda.kda_chunk_fwd(to(w.q, bf), to(w.k, bf), to(w.v, bf), to(w.g, torch.float32),
                            to(w.beta, torch.float32), list(w.cu_seqlens), 1.0, to(w.s0, torch.float32), True, every,
                            chunk_size=chunk, noalloc=noalloc)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("chunk", [32, 64])
def test_noalloc_forward_equals_the_workspace_forward(chunk):
    every = 2 * chunk
    big = W.make_prefill([300, 64, 0, 129, 512, 33, 190], H=3, dk=128, dv=128, dtype="bf16", seed=81, s0_std=0.1)
    small = W.make_prefill([97, 256], H=3, dk=128, dv=128, dtype="bf16", seed=82, s0_std=0.1)
    for w in (big, small):
        print(f"[noalloc] chunk={chunk} seqlens={w.seqlens}", flush=True)
        got = run(w, every, chunk, noalloc=True)
        ref = run(w, every, chunk, noalloc=False)
        for name, a, b in zip(("o", "final_state", "checkpoints"), got, ref):
            assert torch.equal(a, b), name
        o_r, s_r, c_r = oracle.forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, 1.0, w.s0, every)
        errs = {"o": W.rel_max_err(got[0].cpu().numpy(), o_r), "S": W.rel_max_err(got[1].cpu().numpy(), s_r),
                "ckpt": W.rel_max_err(got[2].cpu().numpy(), c_r)}
        print(f"[noalloc] vs oracle: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        for k, v in errs.items():
            assert v <= 2e-2, (k, v)
