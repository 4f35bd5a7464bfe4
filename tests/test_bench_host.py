"""bench.py's host-side contract, without a GPU: the run refuses more than
one GPU before touching any device, and the algorithmic byte counts behind
the roofline fraction are the sums of the operands each stage must move,
checked here against the layer workload's sizes worked out by hand
(2 x 2048 tokens, 24 heads x headdim 64, d_state 128, bf16, 4-chunk spans,
no initial state)."""
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ssd_inputs import by_name  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _Plan:
    def __init__(self, fused_pass, chunks_per_span=4):
        self.fused_pass = fused_pass
        self.chunks_per_span = chunks_per_span


def test_layer_algorithmic_bytes_by_hand():
    w = by_name("layer")
    assert (w.tokens, w.nheads, w.headdim, w.d_state, w.ngroups, w.dtype) == \
        (4096, 24, 64, 128, 1, "bf16")
    spans = bench.spans_used(w, _Plan(1))
    assert spans == 2 * (2048 // 64 // 4)  # 16 spans of 4 chunks
    x = 4096 * 24 * 64 * 2          # x, and y the same size
    d_raw = 4096 * 24 * 2
    bc = 4096 * 1 * 128 * 2         # B, and C the same size
    states = 16 * 24 * 128 * 64 * 2
    decays = 16 * 24 * 4
    final = 2 * 24 * 128 * 64 * 4
    plan1 = bench.stage_bytes(w, _Plan(1), spans)
    # plan 1: the state launch forms the first 7 spans of each sequence
    # (7/8 of the tokens); the scan reads those 14 span states
    formed = 14 * 24 * 128 * 64 * 2 + 14 * 24 * 4
    assert plan1["state"] == (x + d_raw + bc) * 7 // 8 + formed == 17605952
    assert plan1["scan"] == x + d_raw + 2 * bc + formed + final + x == 34538816
    plan0 = bench.stage_bytes(w, _Plan(0), spans)
    assert plan0["pass"] == 2 * states + decays + final
    assert plan0["scan"] == x + d_raw + 2 * bc + states + x
    fused = bench.stage_bytes(w, _Plan(2), spans)["fused"]
    assert fused == x + d_raw + 2 * bc + x + final + (16 - 2) * 24 * (128 * 64 * 2 + 4)


def test_layer_algorithmic_flops_by_hand():
    """Per token-head: 2NP for the chunk state, 2NP + 65P for the scan's
    inter- and intra-chunk products; 65N per token for the causal C B^T of
    the one B/C group; 2NP per span-head for the pair combine."""
    w = by_name("layer")
    spans = bench.spans_used(w, _Plan(1))
    th = 4096 * 24
    f = bench.stage_flops(w, _Plan(1), spans)
    # plan 1: 7/8 of the chunk states in the state launch, the last span's
    # in the scan; 14 span states combined
    assert f["state"] == th * 7 // 8 * 2 * 128 * 64
    assert f["scan"] == th * (2 * 128 * 64 + 65 * 64) + 4096 * 65 * 128 + 14 * 24 * 2 * 128 * 64 \
        + th // 8 * 2 * 128 * 64
    assert f["state"] + f["scan"] == bench.stage_flops(w, _Plan(2), spans)["fused"] - 2 * 24 * 2 * 128 * 64
    f0 = bench.stage_flops(w, _Plan(0), spans)
    assert f0["pass"] == 16 * 24 * 2 * 128 * 64
    assert f0["state"] + f0["pass"] + f0["scan"] == bench.stage_flops(w, _Plan(2), spans)["fused"]
