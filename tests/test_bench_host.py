"""Host-side logic of bench.py (no GPU): the one-GPU contract and the algorithmic byte counts
that the roofline figures divide by."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("dk,in_bytes,per_tok_head", [(128, 2, 1796), (64, 4, 1284)])
def test_prefill_bytes_per_token_head(dk, in_bytes, per_tok_head):
    # q, k, v (2 dk + dv) * in_bytes, g fp32 dk * 4 B, beta 4 B, o fp32 dv * 4 B: 1796 B for the
    # bf16 d = 128 workloads, 1284 B for the fp32 d = 64 one
    assert bench.prefill_bytes(1, 1, dk, dk, in_bytes=in_bytes, with_states=False) == per_tok_head
    # plus the initial and final states, once per (sequence, head)
    assert bench.prefill_bytes(65536, 96, dk, dk, in_bytes=in_bytes) == \
        65536 * 96 * per_tok_head + 2 * 96 * dk * dk * 4


def test_decode_bytes():
    # the state read and written once (2 * 128 * 128 * 4 B) plus one token's inputs and output
    assert bench.decode_bytes(1, 1, 128, 128) == 131072 + 1796
    assert bench.decode_bytes(256, 96, 128, 128) == 256 * 96 * 132868


def test_backward_bytes():
    # inputs as the forward's plus d_o (fp32), gradients dq, dk, dg (fp32 dk each), dv, dbeta;
    # d_final_state read, d_initial_state written and the initial state read once
    per = 2 * (2 * 128 + 128) + 4 * 128 + 4 + 4 * 128 + 4 * (3 * 128 + 128 + 1)
    assert bench.bwd_alg_bytes(1, 1, 128, 128, 0) == per
    assert bench.bwd_alg_bytes(65536, 96, 128, 128, 1) == 65536 * 96 * per + 3 * 96 * 128 * 128 * 4
    # a bf16 gate stream (pre-activations) is 2 bytes per channel cheaper
    assert bench.bwd_alg_bytes(1, 1, 128, 128, 0, fused=True) == per - 2 * 128


def test_flop_counts_and_roofline_bound():
    # 2C(3 dk + 2 dv) + 6 dk dv: 180,224 at C = 64, d = 128 (the roofline's count); 139,264 at C = 32
    assert bench.prefill_flop_per_tokhead(64, 128, 128) == 180224
    assert bench.prefill_flop_per_tokhead(32, 128, 128) == 139264
    # the prefill's intensity (about 100 flop/B) is below MI355X's ridge (2.5e15 / 8e12 = 312.5): HBM
    bound, inten, ridge = bench.roofline_bound(180224, 1796)
    assert bound == "hbm" and ridge == pytest.approx(312.5) and inten == pytest.approx(100.35, abs=0.01)
    assert bench.roofline_bound(400.0, 1.0)[0] == "mfma"
