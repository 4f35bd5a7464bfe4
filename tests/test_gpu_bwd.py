"""GPU parity of the backward pass: libssd's ssd_bwd (through its C ABI)
against the fp64 backward oracle (the adjoint of the recurrence, itself
pinned by finite differences in test_oracle_bwd_pins.py).

Bound per gradient (max|gpu - ref| / max|ref|): BWD_TOL for bf16 inputs
(fp32 accumulation; the operands of every product are rounded to bf16,
states included), 1e-5 for fp32 inputs.  The library does not read the
forward output y; the tests pass the GPU's own, as a caller would, or None.
dy and d_final are seeded Gaussians.
"""
import numpy as np
import pytest
import torch

from oracle import cref
from oracle import ssd_oracle as F
from oracle import ssd_oracle_bwd as O
from ssd_inputs import WORKLOADS, make_inputs, make_inputs_device, random_problem

pytestmark = pytest.mark.gpu

BWD_TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
DEV = "cuda:0"
KEYS = ("dx", "dd_raw", "dB", "dC", "dinit_state")


@pytest.fixture(scope="module")
def ssd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_ssd_chunked_02_amd as m
    m.library()
    return m


def _dev(t):
    return None if t is None else t.to(DEV)


def bwd_case(ssd, p, reverse=False, with_final=True, seed=0, label="", tuning=None):
    dt = p["x"].dtype
    tol = BWD_TOL[dt]
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    y, _ = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                       init_state=d["init_state"], cu_seqlens=d["cu_seqlens"], reverse=reverse)
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn(p["x"].shape, generator=g).to(dt)
    b, L, H, P = p["x"].shape
    N = p["B"].shape[3]
    S = b if p["cu_seqlens"] is None else p["cu_seqlens"].numel() - 1
    dfin = torch.randn((S, H, N, P), generator=g) if with_final else None
    got = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y, _dev(dy),
                      init_state=d["init_state"], cu_seqlens=d["cu_seqlens"], reverse=reverse,
                      d_final=_dev(dfin), tuning=tuning)
    torch.cuda.synchronize()
    ref = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                        init_state=p["init_state"], d_final=dfin, cu_seqlens=p["cu_seqlens"],
                        reverse=reverse)
    errs = {k: F.rel_err(got[k].float().cpu(), ref[k]) for k in KEYS}
    errs["dd_init"] = dd_init_err(float(got["dd_init"].cpu()), ref)
    print(f"{label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={tol}",
          flush=True)
    for k in KEYS:
        assert torch.isfinite(got[k].float()).all(), k
    for k, v in errs.items():
        assert v <= tol, (k, v)
    return got, ref


def dd_init_err(got, ref):
    """Error of the d_init gradient, a sum of every d d_raw entry.  Each
    summand carries the kernel's relative error, so the error of the sum is
    bounded by that error times the sum of the summands' magnitudes, not
    times the sum itself (the summands have both signs and largely cancel):
    the error is taken relative to sum |d d_raw|, the sum's condition scale."""
    return abs(got - ref["dd_init"]) / max(float(np.abs(ref["dd_raw"]).sum()), 1e-30)


SHAPES = [
    # (batch, seqlen, nheads, headdim, d_state, ngroups)
    (2, 200, 4, 64, 128, 1),
    (1, 130, 4, 32, 64, 2),
    (1, 64, 2, 16, 16, 1),
    (1, 65, 3, 48, 32, 1),
    (1, 1, 2, 64, 128, 1),
    (1, 150, 2, 192, 64, 1),    # three column groups (the bidirectional workload's headdim)
    (1, 100, 4, 80, 128, 2),    # a partial second column group
    (1, 257, 1, 512, 16, 1),    # the largest headdim: eight column groups
]


@pytest.mark.parametrize("chunks", [1, 4])
@pytest.mark.parametrize("rev", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes_bf16(ssd, shape, rev, chunks):
    """Every shape with both chunk-state plans (small problems default to
    one chunk per chunk-state workgroup)."""
    b, L, H, P, N, G = shape
    p = random_problem(301, b, L, H, P, N, ngroups=G, dtype="bf16", init_scale=0.5, d_init=-2.0)
    bwd_case(ssd, p, reverse=rev, label=f"bwd {shape} rev={rev} chunks={chunks}",
             tuning={"bwd_state_chunks": chunks})


@pytest.mark.parametrize("N", [16, 32])
def test_bwd_fp32(ssd, N):
    p = random_problem(307, 1, 256, 2, 16, N, dtype="f32", init_scale=0.5, d_init=-4.6)
    bwd_case(ssd, p, label=f"bwd fp32 N={N}")
    bwd_case(ssd, p, reverse=True, label=f"bwd fp32 N={N} rev")


def test_bwd_varlen(ssd):
    """Packed sequences with an empty one and ragged tails: every state pass
    restarts at a boundary, the empty sequence hands d_final straight to its
    initial-state gradient."""
    p = random_problem(311, 1, 0, 4, 64, 128, dtype="bf16", init_scale=0.5, d_init=-2.0,
                       lengths=[70, 0, 129, 64, 1])
    bwd_case(ssd, p, label="bwd varlen")
    bwd_case(ssd, p, reverse=True, label="bwd varlen rev")


def test_bwd_no_state_gradients(ssd):
    """No initial state and no final-state gradient."""
    p = random_problem(313, 2, 150, 2, 64, 64, dtype="bf16", d_init=-4.6)
    bwd_case(ssd, p, with_final=False, label="bwd no-state")


def test_bwd_head_subsets(ssd):
    """One head per workgroup (six partials of dB / dC added) and all heads
    in one workgroup give the same gradients within the bound."""
    p = random_problem(317, 1, 256, 6, 64, 128, dtype="bf16", init_scale=0.5, d_init=-2.0)
    for hs in (1, 6):
        bwd_case(ssd, p, label=f"bwd heads/wg={hs}", tuning={"bwd_heads": hs})


def test_bwd_layer_shape(ssd):
    """Layer-shaped problem (24 heads x headdim 64, d_state 128) at 512 tokens."""
    p = random_problem(331, 1, 512, 24, 64, 128, dtype="bf16", d_init=-4.6)
    bwd_case(ssd, p, with_final=False, label="bwd layer-shaped")


def test_bwd_bidir_shape_strided(ssd):
    """The bidirectional workload's head shape (headdim 192, d_state 64) in
    the reverse direction, with y and dy as the second halves of
    [b, L, H, 2P] buffers, on 300 tokens x 4 heads."""
    p = random_problem(341, 1, 300, 4, 192, 64, dtype="bf16", d_init=-4.6)
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    b, L, H, P = p["x"].shape
    ycat = torch.empty((b, L, H, 2 * P), dtype=torch.bfloat16, device=DEV)
    ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], reverse=True, y=ycat[..., P:])
    g = torch.Generator().manual_seed(9)
    dy = torch.randn((b, L, H, P), generator=g).to(torch.bfloat16)
    dycat = torch.zeros((b, L, H, 2 * P), dtype=torch.bfloat16)
    dycat[..., P:] = dy
    got = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], ycat[..., P:],
                      dycat.to(DEV)[..., P:], reverse=True)
    torch.cuda.synchronize()
    ref = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy, reverse=True)
    errs = {k: F.rel_err(got[k].float().cpu(), ref[k]) for k in KEYS}
    print("bwd bidir-shaped rev " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL[torch.bfloat16], (k, v)


def test_bwd_strided_dy_and_y(ssd):
    """dy and y as halves of a [b, L, H, 2P] buffer (the bidirectional layout)."""
    p = random_problem(337, 1, 100, 2, 32, 64, dtype="bf16", init_scale=0.5, d_init=-2.0)
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    b, L, H, P = p["x"].shape
    ycat = torch.empty((b, L, H, 2 * P), dtype=torch.bfloat16, device=DEV)
    ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"],
                y=ycat[..., P:])
    g = torch.Generator().manual_seed(5)
    dy = torch.randn((b, L, H, P), generator=g).to(torch.bfloat16)
    dycat = torch.zeros((b, L, H, 2 * P), dtype=torch.bfloat16)
    dycat[..., :P] = dy
    got = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], ycat[..., P:],
                      dycat.to(DEV)[..., :P], init_state=d["init_state"])
    ref = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                        init_state=p["init_state"])
    for k in KEYS:
        assert F.rel_err(got[k].float().cpu(), ref[k]) <= BWD_TOL[torch.bfloat16], k


@pytest.mark.parametrize("chunks", [1, 4])
def test_bwd_long_walks_weak_decay(ssd, chunks):
    """Both chunk-state passes over walks of 1 to 38 chunks (every position of
    the pass's two batches of eight in flight, walks past two batches), with
    weak decay so a state carried wrongly anywhere shows in the gradients of
    the sequence's first tokens and of the initial state; with one chunk per
    chunk-state workgroup, and with four-chunk spans whose states are carried
    (the last span of a sequence shorter, its last chunk ragged)."""
    t = {"bwd_state_chunks": chunks}
    lens = [64 * 37 + 5, 64 * 16, 1, 64 * 17 - 3, 64 * 9]
    p = random_problem(347, 1, 0, 2, 16, 16, dtype="f32", lengths=lens, d_init=-6.0,
                       init_scale=1.0)
    bwd_case(ssd, p, label="bwd long walks", tuning=t)
    bwd_case(ssd, p, reverse=True, label="bwd long walks rev", tuning=t)
    q = random_problem(349, 2, 64 * 37 + 5, 2, 16, 16, dtype="f32", d_init=-6.0,
                       init_scale=1.0)
    bwd_case(ssd, q, label="bwd long batch", tuning=t)
    bwd_case(ssd, q, reverse=True, label="bwd long batch rev", tuning=t)



@pytest.mark.parametrize("varlen", [False, True])
def test_bwd_chunk_state_plans_agree(ssd, varlen):
    """The two chunk-state plans: one workgroup per chunk with the pass walking
    every chunk, and four-chunk spans whose workgroups carry the state through
    the span (the pass then walks spans and each chunk's state is rebuilt from
    the span's entering state, the decay since the span start and the state
    gathered within the span).  Both match the oracle, and each other within
    the same bound; ragged spans and empty sequences included."""
    if varlen:
        p = random_problem(353, 1, 0, 3, 64, 64, dtype="bf16", d_init=-4.6, init_scale=0.5,
                           lengths=[64 * 9 + 7, 1, 64 * 4, 0, 200])
    else:
        p = random_problem(359, 2, 64 * 11 + 30, 3, 64, 64, dtype="bf16", d_init=-4.6,
                           init_scale=0.5)
    out = []
    for chunks in (4, 1):
        for reverse in (False, True):
            got, ref = bwd_case(ssd, p, reverse=reverse, seed=3, tuning={"bwd_state_chunks": chunks},
                                label=f"bwd plan chunks={chunks} rev={reverse}")
            out.append((got, ref))
    for i in range(2):
        a, b = out[i][0], out[i + 2][0]
        for k in KEYS:
            d = F.rel_err(a[k].float().cpu(), b[k].float().cpu())
            assert d <= BWD_TOL[torch.bfloat16], (k, d)


def test_bwd_layer_workload_full(ssd):
    """The layer workload at the size the benchmark times it (2 x 2048
    tokens, 24 heads x headdim 64, d_state 128), every gradient on full
    tensors against the C adjoint oracle, in the plan the benchmark runs:
    six heads per gradient workgroup, four head subsets of dB / dC partials,
    four-chunk chunk-state walks."""
    w = WORKLOADS[2]
    p = make_inputs(w)
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    info = ssd.ssd_fwd_plan(ssd.dims_for(d["x"], d["B"]))
    assert (info.bwd_heads_per_wg, info.bwd_head_subsets, info.bwd_state_chunks) == (6, 4, 4)
    y, _ = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"])
    g = torch.Generator().manual_seed(23)
    dy = torch.randn(p["x"].shape, generator=g).to(torch.bfloat16)
    dfin = torch.randn((2, 24, 128, 64), generator=g)
    got = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y, _dev(dy),
                      d_final=_dev(dfin))
    torch.cuda.synchronize()
    ref = cref.ssd_ref_bwd_c(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy, d_final=dfin,
                             col_block=64)
    errs = {k: F.rel_err(got[k].float().cpu(), ref[k]) for k in KEYS}
    errs["dd_init"] = dd_init_err(float(got["dd_init"].cpu()), ref)
    print("bwd layer full " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL[torch.bfloat16], (k, v)


@pytest.mark.parametrize("rev", [False, True])
def test_bwd_bidir_workload_sampled_heads(ssd, rev):
    """The 1,048,576-token bidirectional workload (8 heads x headdim 192,
    d_state 64), one direction per case, y and dy as halves of
    [1, L, 8, 384] buffers: a chunk-state workspace past 2^31 bytes and
    16384-chunk walks.  dx, d d_raw and the initial-state gradient of two
    heads, every column, against the C adjoint oracle (heads are
    independent; dB and dC sum over every head, so they are not compared)."""
    w = WORKLOADS[5]
    d = make_inputs_device(w, DEV)
    b, L, H, P = d["x"].shape
    ycat, _ = ssd.ssd_fwd_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"])
    gen = torch.Generator(device=DEV).manual_seed(29)
    dycat = torch.randn((b, L, H, 2 * P), generator=gen, device=DEV).to(torch.bfloat16)
    dfin = torch.randn((1, H, w.d_state, P), generator=gen, device=DEV)
    half = slice(P, 2 * P) if rev else slice(0, P)
    call = ssd.prepare_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], ycat[..., half],
                           dycat[..., half], reverse=rev, d_final=dfin)
    assert call.workspace.numel() > (1 << 31)
    got = call.run()
    torch.cuda.synchronize()
    heads = [1, 6]
    host = lambda t: t.float().cpu().contiguous()
    ref = cref.ssd_ref_bwd_c(host(d["x"][:, :, heads]), host(d["d_raw"][:, :, heads]),
                             d["d_init"], host(d["B"]), host(d["C"]),
                             host(dycat[..., half][:, :, heads]),
                             d_final=host(dfin[:, heads]), reverse=rev,
                             want=("dx", "dd_raw", "dinit_state"), col_block=8)
    errs = {"dx": F.rel_err(host(got["dx"][:, :, heads]), ref["dx"]),
            "dd_raw": F.rel_err(host(got["dd_raw"][:, :, heads]), ref["dd_raw"]),
            "dinit_state": F.rel_err(host(got["dinit_state"][:, heads]), ref["dinit_state"])}
    print(f"bwd bidir 1M rev={rev} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL[torch.bfloat16], (k, v)


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_projection_views(ssd, reverse):
    """x, B, C and d_raw as views of one [b, L, H*P + 2*G*N + H] projection
    buffer; the gradients go straight into the same places of a gradient
    buffer of that layout (each gradient is written with its input's
    strides); against the adjoint oracle on contiguous copies."""
    # H = 8 keeps a projection row a whole number of 16-byte units
    p = random_problem(361, 2, 300, 8, 64, 64, ngroups=2, dtype="bf16", init_scale=0.5,
                       d_init=-4.6)
    b, L, H, P = p["x"].shape
    G, N = p["B"].shape[2], p["B"].shape[3]
    W = H * P + 2 * G * N + H
    proj = torch.empty((b, L, W), dtype=torch.bfloat16)
    proj[..., :H * P] = p["x"].reshape(b, L, H * P)
    proj[..., H * P:H * P + G * N] = p["B"].reshape(b, L, G * N)
    proj[..., H * P + G * N:H * P + 2 * G * N] = p["C"].reshape(b, L, G * N)
    proj[..., H * P + 2 * G * N:] = p["d_raw"]
    proj = proj.to(DEV)

    def views(t):
        return (t[..., :H * P].view(b, L, H, P), t[..., H * P + 2 * G * N:],
                t[..., H * P:H * P + G * N].view(b, L, G, N),
                t[..., H * P + G * N:H * P + 2 * G * N].view(b, L, G, N))

    x, dr, Bv, Cv = views(proj)
    init = p["init_state"].to(DEV)
    y, _ = ssd.ssd_fwd(x, dr, p["d_init"], Bv, Cv, init_state=init, reverse=reverse)
    g = torch.Generator().manual_seed(13)
    dy = torch.randn((b, L, H, P), generator=g).to(torch.bfloat16)
    dfin = torch.randn((b, H, N, P), generator=g)
    dproj = torch.full((b, L, W), 9.0, dtype=torch.bfloat16, device=DEV)
    gx, gdr, gB, gC = views(dproj)
    got = ssd.ssd_bwd(x, dr, p["d_init"], Bv, Cv, y, _dev(dy), init_state=init, reverse=reverse,
                      d_final=_dev(dfin), grads={"dx": gx, "dd_raw": gdr, "dB": gB, "dC": gC})
    # the same call on contiguous copies: only addresses differ, so every
    # gradient must agree bit for bit
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    yc, _ = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=init,
                        reverse=reverse)
    con = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], yc, _dev(dy),
                      init_state=init, reverse=reverse, d_final=_dev(dfin))
    torch.cuda.synchronize()
    assert torch.equal(y, yc)
    for k, v in (("dx", gx), ("dd_raw", gdr), ("dB", gB), ("dC", gC),
                 ("dinit_state", got["dinit_state"]), ("dd_init", got["dd_init"])):
        assert torch.equal(v, con[k]), k
    assert got["dx"].data_ptr() == gx.data_ptr()
    ref = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                        init_state=p["init_state"], d_final=dfin, reverse=reverse)
    errs = {"dx": F.rel_err(gx.float().cpu(), ref["dx"]),
            "dd_raw": F.rel_err(gdr.float().cpu(), ref["dd_raw"]),
            "dB": F.rel_err(gB.float().cpu(), ref["dB"]),
            "dC": F.rel_err(gC.float().cpu(), ref["dC"]),
            "dinit_state": F.rel_err(got["dinit_state"].cpu(), ref["dinit_state"])}
    print(f"bwd projection rev={reverse} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL[torch.bfloat16], (k, v)


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_dd_raw_strong_decay(ssd, reverse):
    """Step sizes around 0.2 (d_init -2), the problem whose reverse direction
    showed the precision limit of the chunk-local identity for the log-decay
    gradient (1.28e-2 on d d_raw); the kernel's term-by-term form meets the
    bf16 bound.  y is passed as None: the library does not read it."""
    p = random_problem(361, 2, 300, 8, 64, 64, ngroups=2, dtype="bf16", init_scale=0.5,
                       d_init=-2.0)
    d = {k: (_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    b, L, H, P = p["x"].shape
    N = p["B"].shape[3]
    g = torch.Generator().manual_seed(13)
    dy = torch.randn((b, L, H, P), generator=g).to(torch.bfloat16)
    dfin = torch.randn((b, H, N, P), generator=g)
    got = ssd.ssd_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], None, _dev(dy),
                      init_state=d["init_state"], reverse=reverse, d_final=_dev(dfin))
    torch.cuda.synchronize()
    ref = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                        init_state=p["init_state"], d_final=dfin, reverse=reverse)
    errs = {k: F.rel_err(got[k].float().cpu(), ref[k]) for k in KEYS}
    errs["dd_init"] = dd_init_err(float(got["dd_init"].cpu()), ref)
    print(f"bwd strong decay rev={reverse} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL[torch.bfloat16], (k, v)
    # d d_raw at the level of the other gradients (3.0e-3 measured), well
    # inside the bound that the cancelling identity exceeded
    assert errs["dd_raw"] <= 5e-3
