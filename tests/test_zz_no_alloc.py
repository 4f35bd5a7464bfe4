"""The allocation-free entry point ssd_fwd_noalloc (C ABI, through ctypes):
the same scan as ssd_fwd with the library's fixed per-GPU scratch in place
of a workspace.  Two calls in a row, the second on a smaller (packed)
input, each against ssd_fwd's output on the same inputs (bit for bit: the
same kernels and plan, only the scratch address differs) and the fp64
oracle."""
import pytest
import torch

from oracle import cref
from oracle import ssd_oracle as O
from ssd_inputs import WORKLOADS, make_inputs, random_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_ssd_chunked_02_amd as m
    m.library()
    return m


def _dev(p):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def test_noalloc_matches_ssd_fwd(ssd):
    big = make_inputs(WORKLOADS[2])                       # 2 x 2048 tokens, 24 heads
    small = random_problem(401, 1, 0, 4, 64, 128, dtype="bf16", init_scale=0.5,
                           lengths=[300, 1, 0, 90])       # packed, smaller
    probs = [_dev(big), _dev(small)]
    outs = []
    for d in probs:                                       # two no-alloc calls in a row
        b, L, H, P = d["x"].shape
        S = b if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
        y = torch.full((b, L, H, P), 5.0, dtype=d["x"].dtype, device=DEV)
        f = torch.full((S, H, d["B"].shape[3], P), 5.0, device=DEV)
        ssd.ssd_fwd_noalloc(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y, f,
                            init_state=d["init_state"], cu_seqlens=d["cu_seqlens"])
        outs.append((y, f))
    torch.cuda.synchronize()
    for p, d, (y, f) in zip((big, small), probs, outs):
        yw, fw = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                             init_state=d["init_state"], cu_seqlens=d["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(y, yw) and torch.equal(f, fw)
        yr, fr = cref.ssd_ref_seq_c(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"],
                                    p["init_state"], p["cu_seqlens"])
        ey, ef = O.rel_err(y.float().cpu(), yr), O.rel_err(f.cpu(), fr)
        print(f"noalloc y_err={ey:.3e} final_err={ef:.3e}", flush=True)
        assert ey <= 1e-2 and ef <= 1e-2
