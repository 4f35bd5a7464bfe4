"""GPU parity: libssd (through its C ABI) against the fp64 oracle.

Bound (max|gpu - ref| / max|ref|, separately for y and final_state):
1e-2 for bf16 inputs with fp32 accumulation, 1e-5 for fp32 inputs.
Inputs are the seeded workloads of ssd_inputs; the oracle sees exactly the
values the GPU reads.  Full-size workloads that the oracle cannot finish in
seconds are checked on sampled heads / headdim columns: columns of the
state are independent, so a slice of x gives exactly those outputs.
"""
import os

import numpy as np
import pytest
import torch

from oracle import cref
from oracle import ssd_oracle as O
from ssd_inputs import WORKLOADS, make_inputs, make_inputs_device, random_problem

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_ssd_chunked_02_amd as m
    m.library()
    return m


def to_dev(p):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def run(ssd, p, reverse=False, **kw):
    d = to_dev(p)
    y, f = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                       init_state=d["init_state"], cu_seqlens=d["cu_seqlens"],
                       reverse=reverse, **kw)
    torch.cuda.synchronize()
    return y.float().cpu(), f.cpu()


def oracle(p, reverse=False):
    return cref.ssd_ref_seq_c(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"],
                              p["init_state"], p["cu_seqlens"], reverse=reverse)


def check(ssd, p, reverse=False, label="", tuning=None):
    tol = TOL[p["x"].dtype]
    y, f = run(ssd, p, reverse, tuning=tuning)
    yr, fr = oracle(p, reverse)
    ey, ef = O.rel_err(y, yr), O.rel_err(f, fr)
    print(f"{label} y_err={ey:.3e} final_err={ef:.3e} tol={tol}", flush=True)
    assert np.isfinite(y.numpy()).all() and np.isfinite(f.numpy()).all()
    assert ey <= tol, ey
    assert ef <= tol, ef
    return y, f


# ------------------------------------------------------------ workloads
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_workload_full(ssd, cfg):
    w = WORKLOADS[cfg]
    check(ssd, make_inputs(w), label=w.name)


def test_workload_varlen_full(ssd):
    """16 packed sequences, 65536 tokens, every head and column against the
    C oracle."""
    w = WORKLOADS[4]
    p = make_inputs(w)
    d = to_dev(p)
    plan = ssd.ssd_fwd_plan(ssd.dims_for(d["x"], d["B"], cu_seqlens=d["cu_seqlens"]))
    assert plan.head_wave == 1 and plan.heads_per_wg == 4   # every slot of the 4-head workgroups
    check(ssd, p, label="varlen full")


def test_workload_bidir_sampled_columns(ssd):
    """1,048,576 tokens, forward + reverse written into one [1,L,8,384] y."""
    w = WORKLOADS[5]
    d = make_inputs_device(w, DEV)
    y, fin = ssd.ssd_fwd_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], final_state=True)
    torch.cuda.synchronize()
    heads, cols = [0, 5], [0, 37, 64, 191]
    P = w.headdim
    q = {
        "x": d["x"][:, :, heads][..., cols].float().cpu().contiguous(),
        "d_raw": d["d_raw"][:, :, heads].float().cpu().contiguous(),
        "B": d["B"].float().cpu(), "C": d["C"].float().cpu(),
        "init_state": None, "cu_seqlens": None, "d_init": d["d_init"],
    }
    yf_ref, ff_ref = oracle(q, False)
    yr_ref, fr_ref = oracle(q, True)
    ysel = y[:, :, heads].float().cpu()
    yf = ysel[..., cols]
    yr = ysel[..., [P + c for c in cols]]
    errs = [O.rel_err(yf, yf_ref), O.rel_err(yr, yr_ref),
            O.rel_err(fin[0][:, heads][..., cols].cpu(), ff_ref),
            O.rel_err(fin[1][:, heads][..., cols].cpu(), fr_ref)]
    print("bidir errs", ["%.3e" % e for e in errs], flush=True)
    assert max(errs) <= 1e-2


# ------------------------------------------------------------ shapes
SHAPES = [
    # (batch, seqlen, nheads, headdim, d_state, ngroups)
    (1, 1, 1, 16, 16, 1),
    (1, 63, 2, 16, 32, 1),
    (1, 64, 3, 48, 64, 1),
    (2, 65, 2, 80, 128, 1),
    (1, 200, 4, 64, 128, 2),
    (3, 130, 2, 192, 64, 1),
    (1, 300, 2, 128, 256, 1),
    (1, 257, 1, 512, 16, 1),
]


@pytest.mark.parametrize("family", ["default", "span", "hw"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("reverse", [False, True])
def test_shapes(ssd, shape, dtype, reverse, family):
    """Every shape through the default kernels, through the span kernels
    alone and with the head-wave kernels forced (they take bf16 problems
    with d_state 64 / 128; others keep the span kernels)."""
    b, L, H, P, N, G = shape
    if dtype == "f32" and N > 128:
        pytest.skip("fp32 path is built for d_state <= 128")
    tuning = None
    if family == "span" or (family == "hw" and dtype == "bf16" and N in (64, 128)):
        tuning = {"kernel": family}
    p = random_problem(101, b, L, H, P, N, ngroups=G, dtype=dtype, init_scale=0.5,
                       d_init=-2.0)
    check(ssd, p, reverse, label=f"{shape} {dtype} rev={reverse} {family}", tuning=tuning)


HW_SHAPES = [
    # (batch, seqlen, nheads, headdim, d_state, ngroups)
    (2, 700, 4, 64, 128, 1),
    (1, 333, 8, 128, 64, 2),
    (1, 130, 4, 80, 128, 1),
    (3, 64, 4, 192, 64, 1),
]


@pytest.mark.parametrize("heads", ["1", "2", "4"])
@pytest.mark.parametrize("npb", ["2", "4"])
@pytest.mark.parametrize("k", ["1", "3", "8"])
@pytest.mark.parametrize("shape", HW_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_head_wave_variants(ssd, shape, heads, npb, k):
    """Every head-wave workgroup shape (1 / 2 / 4 heads, waves of 64 or 32
    headdim columns) at several span lengths, forward and reverse, with a
    partial column group (headdim 80) and two B / C groups."""
    b, L, H, P, N, G = shape
    if npb == "4" and N > 64:
        pytest.skip("full-width head waves are built for d_state <= 64")
    hs = min(int(heads), 2)  # the state workgroup takes at most two heads
    tuning = {"kernel": "hw", "heads_scan": int(heads), "heads_state": hs,
              "cols_per_wave": 16 * int(npb), "chunks_per_span": int(k)}
    p = random_problem(211, b, L, H, P, N, ngroups=G, dtype="bf16", init_scale=0.5)
    d = to_dev(p)
    call = ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"])
    plan = ssd.ssd_fwd_plan(call.dims, tuning)
    assert plan.head_wave == 1 and plan.heads_per_wg == int(heads)
    assert plan.cols_per_wave == 16 * int(npb) and plan.chunks_per_span == int(k)
    for rev in (False, True):
        check(ssd, p, rev, label=f"hw {shape} hg={heads} npb={npb} K={k} rev={rev}", tuning=tuning)


@pytest.mark.parametrize("d_init", [-9.0, -3.0, 1.0])
@pytest.mark.parametrize("N", [64, 128])
def test_head_wave_rescaled_state(ssd, d_init, N):
    """The rescaled state across long spans: weak decay (no restart in 16
    chunks), medium decay (the running scale restarts every few chunks) and
    strong decay (every chunk restarts), forward and reverse."""
    tuning = {"kernel": "hw", "chunks_per_span": 16}
    p = random_problem(227, 1, 1500, 4, 64, N, dtype="bf16", init_scale=0.5, d_init=d_init,
                       d_raw_scale=2.0)
    for rev in (False, True):
        check(ssd, p, rev, label=f"hw rescale d_init={d_init} N={N} rev={rev}", tuning=tuning)


@pytest.mark.parametrize("npb", ["2", "4"])
def test_head_wave_varlen(ssd, npb):
    N = 64 if npb == "4" else 128  # full-width waves are built for d_state 64
    tuning = {"kernel": "hw", "cols_per_wave": 16 * int(npb), "chunks_per_span": 2}
    lens = [1, 63, 64, 65, 0, 200, 129, 7, 0, 640]
    p = random_problem(223, 1, 0, 4, 64, N, dtype="bf16", lengths=lens, init_scale=0.3)
    for rev in (False, True):
        check(ssd, p, rev, label=f"hw varlen npb={npb} rev={rev}", tuning=tuning)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("reverse", [False, True])
def test_shapes_fused_launch(ssd, shape, dtype, reverse):
    """The single fused launch, one chunk per span (so every sequence longer
    than 64 tokens hands states between workgroups), on every shape."""
    b, L, H, P, N, G = shape
    if dtype == "f32" and N > 128:
        pytest.skip("fp32 path is built for d_state <= 128")
    if (L + 63) // 64 > 16:
        pytest.skip("more than 16 spans per sequence")
    tuning = {"kernel": "span", "state_pass": "fused", "chunks_per_span": 1}
    p = random_problem(103, b, L, H, P, N, ngroups=G, dtype=dtype, init_scale=0.5,
                       d_init=-2.0)
    check(ssd, p, reverse, label=f"fused {shape} {dtype} rev={reverse}", tuning=tuning)


@pytest.mark.parametrize("fuse", ["1", "2"])
def test_two_heads_per_scan_workgroup(ssd, fuse):
    """Span workgroups carrying two heads (one quad of waves each) in the
    folding and the fused plans."""
    tuning = {"kernel": "span", "state_pass": int(fuse) + 1, "heads_scan": 2,
              "heads_state": 2, "chunks_per_span": 2}
    p = random_problem(107, 2, 700, 4, 64, 64, dtype="bf16", init_scale=0.5)
    check(ssd, p, False, label=f"hg2 fuse={fuse}", tuning=tuning)
    check(ssd, p, True, label=f"hg2 fuse={fuse} rev", tuning=tuning)


@pytest.mark.parametrize("reverse", [False, True])
def test_varlen_ragged(ssd, reverse):
    lens = [1, 63, 64, 65, 0, 200, 129, 7, 0, 640]
    p = random_problem(103, 1, 0, 3, 64, 128, dtype="bf16", lengths=lens, init_scale=0.3)
    check(ssd, p, reverse, label=f"ragged rev={reverse}")


def test_varlen_many_tiny_sequences(ssd):
    rng = np.random.default_rng(5)
    lens = [int(v) for v in rng.integers(0, 12, 1500)]
    p = random_problem(107, 1, 0, 2, 32, 64, dtype="bf16", lengths=lens, init_scale=0.2)
    check(ssd, p, False, label="tiny-seqs")


def test_strong_decay(ssd):
    p = random_problem(109, 1, 512, 4, 64, 128, dtype="bf16", d_init=1.0, d_raw_scale=3.0)
    check(ssd, p, False, label="strong-decay")


def test_weak_decay_long_memory(ssd):
    p = random_problem(113, 1, 1024, 2, 64, 64, dtype="f32", d_init=-9.0, init_scale=1.0)
    check(ssd, p, False, label="weak-decay")


@pytest.mark.parametrize("k", ["1", "2", "3", "8", "64"])
def test_span_length_invariance(ssd, k):
    tuning = {"chunks_per_span": int(k)}
    p = random_problem(127, 2, 777, 3, 64, 128, dtype="bf16", init_scale=0.5)
    check(ssd, p, False, label=f"K={k}", tuning=tuning)
    lens = [100, 700, 1, 333]
    q = random_problem(131, 1, 0, 2, 64, 64, dtype="f32", lengths=lens, init_scale=0.5)
    check(ssd, q, True, label=f"K={k} varlen rev f32", tuning=tuning)


@pytest.mark.parametrize("reverse", [False, True])
def test_one_span_per_sequence(ssd, reverse):
    """A batch of short sequences that each fit one span: the scan folds no
    span state, so no state stage runs and the scan alone writes y and the
    final state (from init_state); ragged last chunks, both directions."""
    tuning = {"kernel": "span", "chunks_per_span": 4}
    p = random_problem(149, 16, 200, 4, 64, 128, dtype="bf16", init_scale=0.5)
    d = to_dev(p)
    call = ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"])
    plan = ssd.ssd_fwd_plan(call.dims, tuning)
    assert plan.fused_pass == 1 and plan.nspan == 16
    check(ssd, p, reverse, label=f"one span rev={reverse}", tuning=tuning)


@pytest.mark.parametrize("fuse", ["0", "1", "2"])
@pytest.mark.parametrize("reverse", [False, True])
def test_state_pass_folded_or_separate(ssd, fuse, reverse):
    """Every way of handing the state from span to span matches the oracle:
    the separate state_pass kernel (0), span_scan folding the earlier span
    states of its sequence itself (1), and the single fused launch whose
    workgroups hand span states to each other (2)."""
    tuning = {"kernel": "span", "state_pass": int(fuse) + 1, "chunks_per_span": 2}
    p = random_problem(151, 2, 1000, 3, 64, 128, dtype="bf16", init_scale=0.5)
    d = to_dev(p)
    call = ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"])
    assert ssd.ssd_fwd_plan(call.dims, tuning).fused_pass == int(fuse)
    check(ssd, p, reverse, label=f"fuse={fuse} bf16", tuning=tuning)
    q = random_problem(157, 3, 500, 2, 32, 64, dtype="f32", init_scale=0.5)
    check(ssd, q, reverse, label=f"fuse={fuse} f32", tuning=tuning)


def test_state_pass_long_walks(ssd):
    """The separate state pass over walks of 1 to 38 spans (one chunk each):
    every position of its two batches of eight in flight, the tail of a walk
    inside either batch, and walks longer than two batches; weak decay, so a
    state carried or dropped wrongly anywhere along a walk shows at its end."""
    tuning = {"kernel": "span", "chunks_per_span": 1}
    lens = [64 * 37 + 5, 64 * 16, 64 * 17 - 3, 64 * 8, 64 * 9, 1, 64 * 24 + 1]
    p = random_problem(173, 1, 0, 2, 16, 16, dtype="f32", lengths=lens, d_init=-6.0,
                       init_scale=1.0)
    check(ssd, p, False, label="long walks", tuning=tuning)
    check(ssd, p, True, label="long walks rev", tuning=tuning)


def _sync_words(ws, chains):
    """Count of timed-out flag waits (header word 2) and each chain's 64-bit
    ticket/epoch word (after the 256-byte header), as (count, epoch) pairs."""
    timeouts = int(ws[8:12].view(torch.int32).item())
    words = ws[256:256 + 8 * chains].view(torch.int32).view(chains, 2).cpu().tolist()
    return timeouts, [tuple(w) for w in words]


FUSED = {"kernel": "span", "state_pass": "fused"}


def test_fused_handoff_repeated_calls(ssd):
    """The fused launch hands span states between workgroups through the
    workspace, with flags it resets before every launch.  Alternate two input
    sets on one workspace: every call must reproduce its input set's first
    result bit for bit (a state left by the other set's call would change
    it), agree with the three-launch plan, and leave every chain's word at
    count 0, epoch 1, with no timed-out waits.  1024 workgroups of 16 spans
    per sequence: more than the GPU holds at once."""
    probs = [random_problem(seed, 8, 4096, 8, 64, 128, dtype="bf16", init_scale=0.5)
             for seed in (161, 163)]
    devs = [to_dev(p) for p in probs]
    calls = [ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"],
                         tuning=FUSED) for d in devs]
    plan = ssd.ssd_fwd_plan(calls[0].dims, FUSED)
    assert plan.fused_pass == 2 and plan.nspan == 8 * 16
    ws = calls[0].workspace
    ws.fill_(0xA5)  # no initialization is needed: start from garbage
    calls = [ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"],
                         workspace=ws, tuning=FUSED) for d in devs]
    first = []
    for i in range(24):
        y, f = calls[i % 2].run()
        y, f = y.clone(), f.clone()
        if i < 2:
            first.append((y, f))
        else:
            y0, f0 = first[i % 2]
            assert torch.equal(y, y0) and torch.equal(f, f0), f"call {i} differs from call {i % 2}"
    torch.cuda.synchronize()
    assert _sync_words(ws, 8 * 8) == (0, [(0, 1)] * 64)
    for k, d in enumerate(devs):
        y3, f3 = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                             init_state=d["init_state"], tuning={"kernel": "span", "state_pass": "pass"})
        torch.cuda.synchronize()
        y0, f0 = first[k]
        assert O.rel_err(y0.float().cpu(), y3.float().cpu()) <= 1e-2
        assert O.rel_err(f0.cpu(), f3.cpu()) <= 1e-2


def test_fused_after_other_plans_and_sizes(ssd):
    """A fused call right after calls of other plans and other sizes on the
    same workspace (their span states sit where the fused words go): each
    fused call matches the oracle and no flag wait runs out."""
    big = random_problem(181, 2, 1000, 4, 64, 128, dtype="bf16", init_scale=0.5)
    small = random_problem(191, 1, 300, 2, 64, 64, dtype="bf16", init_scale=0.5)
    packed = random_problem(193, 1, 0, 4, 64, 128, dtype="bf16", lengths=[500, 1, 700],
                            init_scale=0.5)
    need = max(ssd.ssd_fwd_plan(ssd.dims_for(to_dev(q)["x"], to_dev(q)["B"], cu_seqlens=(
        None if q["cu_seqlens"] is None else to_dev(q)["cu_seqlens"])), t).workspace_bytes
               for q, t in ((big, FUSED), (small, FUSED), (packed, None), (big, None)))
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    order = [(packed, None), (big, FUSED), (big, None), (small, FUSED), (big, FUSED),
             (packed, None), (small, FUSED)]
    for q, t in order:
        d = to_dev(q)
        y, f = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                           init_state=d["init_state"], cu_seqlens=d["cu_seqlens"], workspace=ws,
                           tuning=t)
        torch.cuda.synchronize()
        yr, fr = oracle(q)
        assert O.rel_err(y.float().cpu(), yr) <= 1e-2 and O.rel_err(f.cpu(), fr) <= 1e-2
        if t is FUSED:
            assert int(ws[8:12].view(torch.int32).item()) == 0


def test_empty_sequence_keeps_init(ssd):
    p = random_problem(137, 2, 0, 2, 16, 16, dtype="bf16", init_scale=1.0)
    y, f = run(ssd, p)
    assert y.numel() == 0
    assert torch.equal(f, p["init_state"])


def test_deterministic(ssd):
    p = random_problem(139, 1, 999, 4, 64, 128, dtype="bf16", init_scale=0.5)
    y1, f1 = run(ssd, p)
    y2, f2 = run(ssd, p)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_bidir_matches_two_calls(ssd):
    p = random_problem(149, 1, 300, 2, 32, 64, dtype="bf16")
    d = to_dev(p)
    y, _ = ssd.ssd_fwd_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"])
    yf, _ = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"])
    yr, _ = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(y[..., :32], yf) and torch.equal(y[..., 32:], yr)
    yo, _ = oracle(p, True)
    assert O.rel_err(yr.float().cpu(), yo) <= 1e-2


# (batch, seqlen, nheads, headdim, d_state, dtype, tuning): whole spans, so
# one launch forms both directions' span states
BIDIR_JOINT = [
    (2, 512, 3, 64, 64, "bf16", None),  # the planner's one-chunk spans, folded in the scan
    (1, 1024, 2, 192, 64, "bf16", {"kernel": "hw", "chunks_per_span": 4}),  # head-wave scan, 3 column groups
    (2, 768, 2, 64, 128, "bf16", {"kernel": "span", "chunks_per_span": 3, "state_pass": "pass"}),
    (1, 256, 2, 32, 16, "f32", None),
    (1, 512, 2, 64, 32, "f32", {"kernel": "span", "chunks_per_span": 8, "state_pass": "fold"}),
    (3, 384, 2, 16, 32, "bf16", {"kernel": "span", "chunks_per_span": 2, "state_pass": "pass"}),
    (2, 512, 2, 64, 128, "bf16", {"kernel": "span", "chunks_per_span": 4, "state_f32": 1}),  # fp32 span states
    (2, 256, 2, 64, 128, "bf16", {"kernel": "span", "chunks_per_span": 4}),  # one span each: no state stage
]


@pytest.mark.parametrize("case", BIDIR_JOINT, ids=lambda c: "x".join(map(str, c[:6])) + ("-" + "-".join(
    f"{k}{v}" for k, v in c[6].items()) if c[6] else ""))
def test_bidir_joint_span_states(ssd, case):
    """ssd_fwd_bidir where every span is whole: the forward and the reverse
    span states come from one walk over each span.  Each direction against
    the oracle from its own initial state (y and final state), and against
    the one-direction calls within the same bound."""
    b, L, H, P, N, dt, tun = case
    p = random_problem(173, b, L, H, P, N, dtype=dt, init_scale=0.5, d_init=-3.0)
    g = torch.Generator().manual_seed(5)
    init_rev = 0.5 * torch.randn(p["init_state"].shape, generator=g)
    q = dict(p, init_state=init_rev)
    dims = ssd.dims_for(p["x"], p["B"])
    plan = ssd.ssd_fwd_plan(dims, tun)
    assert L % (64 * plan.chunks_per_span) == 0 and plan.fused_pass != 2
    d = to_dev(p)
    call = ssd.prepare_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                             init_fwd=d["init_state"], init_rev=init_rev.to(DEV),
                             final_state=True, tuning=tun)
    y, (ff, fr) = call.run()
    torch.cuda.synchronize()
    tol = TOL[p["x"].dtype]
    yf_ref, ff_ref = oracle(p, False)
    yr_ref, fr_ref = oracle(q, True)
    errs = {"y_fwd": O.rel_err(y[..., :P].float().cpu(), yf_ref),
            "y_rev": O.rel_err(y[..., P:].float().cpu(), yr_ref),
            "final_fwd": O.rel_err(ff.cpu(), ff_ref), "final_rev": O.rel_err(fr.cpu(), fr_ref)}
    yf1, ff1 = run(ssd, p, False, tuning=tun)
    yr1, fr1 = run(ssd, q, True, tuning=tun)
    errs["vs_calls_rev"] = O.rel_err(y[..., P:].float().cpu(), yr1.double())
    errs["vs_calls_final_rev"] = O.rel_err(fr.cpu(), fr1.double())
    print("bidir joint", case, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert torch.isfinite(y.float()).all()
    for k, v in errs.items():
        assert v <= tol, (k, v)
    errs_f = (O.rel_err(y[..., :P].float().cpu(), yf1.double()), O.rel_err(ff.cpu(), ff1.double()))
    assert max(errs_f) <= tol, errs_f
    if not plan.head_wave:
        # the span kernels' forward state is the one-direction call's arithmetic
        assert torch.equal(y[..., :P].float().cpu(), yf1) and torch.equal(ff.cpu(), ff1)


@pytest.mark.parametrize("dtype,cuts", [("bf16", [0, 256, 640, 1024]), ("bf16", [0, 100, 577, 1024]),
                                         ("f32", [0, 64, 65, 300, 1024])])
@pytest.mark.parametrize("reverse", [False, True])
def test_sequence_shards_chained(ssd, dtype, cuts, reverse):
    """The one-GPU rehearsal of sequence sharding: each shard of a sequence
    is its own call, started from the state the previous shard left (the
    shards walked in processing order), and the shards' outputs and the last
    final state equal one call over the whole sequence and the oracle."""
    p = random_problem(191, 2, cuts[-1], 3, 32, 64, dtype=dtype, init_scale=0.5, d_init=-3.0)
    d = to_dev(p)
    tol = TOL[p["x"].dtype]
    y_all, f_all = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                               init_state=d["init_state"], reverse=reverse)
    shards = list(zip(cuts[:-1], cuts[1:]))
    if reverse:
        shards = shards[::-1]
    y = torch.empty_like(y_all)
    state = d["init_state"]
    for lo, hi in shards:
        sl = lambda t: t[:, lo:hi].contiguous()
        ys, state = ssd.ssd_fwd(sl(d["x"]), sl(d["d_raw"]), d["d_init"], sl(d["B"]), sl(d["C"]),
                                init_state=state, reverse=reverse)
        y[:, lo:hi] = ys
    torch.cuda.synchronize()
    yr, fr = oracle(p, reverse)
    errs = [O.rel_err(y.float().cpu(), yr), O.rel_err(state.cpu(), fr),
            O.rel_err(y.float().cpu(), y_all.float().cpu().double()),
            O.rel_err(state.cpu(), f_all.cpu().double())]
    print("shards", dtype, cuts, reverse, ["%.2e" % e for e in errs], flush=True)
    assert max(errs) <= tol, errs


def test_bidir_joint_in_place_final_states(ssd):
    """ssd_fwd_bidir with each direction's final state written over its
    initial state (whole spans, so the joint state launch runs; the aliased
    directions then pass their states in the separate pass)."""
    p = random_problem(181, 2, 512, 2, 64, 64, dtype="bf16", init_scale=0.5, d_init=-3.0)
    g = torch.Generator().manual_seed(7)
    init_rev = 0.5 * torch.randn(p["init_state"].shape, generator=g)
    d = to_dev(p)
    sf = d["init_state"].clone()
    sr = init_rev.to(DEV)
    call = ssd.prepare_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_fwd=sf,
                             init_rev=sr, final_state=(sf, sr))
    y, _ = call.run()
    torch.cuda.synchronize()
    P = p["x"].shape[3]
    yf_ref, ff_ref = oracle(p, False)
    yr_ref, fr_ref = oracle(dict(p, init_state=init_rev), True)
    errs = [O.rel_err(y[..., :P].float().cpu(), yf_ref), O.rel_err(y[..., P:].float().cpu(), yr_ref),
            O.rel_err(sf.cpu(), ff_ref), O.rel_err(sr.cpu(), fr_ref)]
    print("bidir in place", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) <= TOL[torch.bfloat16], errs


# ------------------------------------------------------------ boundary
def test_ssd_check_rejects_bad_cu_seqlens(ssd, monkeypatch):
    """With SSD_CHECK=1 the library copies cu_seqlens to the host and
    returns SSD_ERR_CU_SEQLENS for a non-monotone one or one that does not
    end at L, launching nothing: sentinel-filled outputs stay as they were."""
    monkeypatch.setenv("SSD_CHECK", "1")
    p = random_problem(197, 1, 0, 2, 64, 64, dtype="bf16", lengths=[100, 50, 50])
    d = to_dev(p)
    L = d["x"].shape[1]
    for bad in ([0, 100, 50, 200], [0, 100, 150, 180], [5, 100, 150, 200]):
        cu = torch.tensor(bad, dtype=torch.int32, device=DEV)
        y = torch.full_like(d["x"], 7.0)
        fin = torch.full((3, 2, 64, 64), -3.0, device=DEV)
        with pytest.raises(ssd.SsdError) as e:
            ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], cu_seqlens=cu, y=y,
                        final_state=fin)
        assert e.value.status == -8
        torch.cuda.synchronize()
        assert bool((y == 7.0).all()) and bool((fin == -3.0).all())
    assert L == 200
    # a valid one passes the check and matches the oracle
    check(ssd, p, label="checked cu_seqlens")


@pytest.mark.parametrize("plan", [None, "fold", "fused"])
def test_final_state_in_place(ssd, plan):
    """final_state written over init_state (one buffer): the library takes
    the separate pass, which reads each entry before writing it; the result
    matches the oracle run from the original initial state.  Eight spans
    per sequence, so the fold would otherwise read init_state in every
    span's workgroup."""
    p = random_problem(199, 2, 2048, 4, 64, 128, dtype="bf16", init_scale=0.5)
    d = to_dev(p)
    tuning = None if plan is None else {"kernel": "span", "state_pass": plan}
    info = ssd.ssd_fwd_plan(ssd.dims_for(d["x"], d["B"]), tuning)
    assert info.fused_pass == {None: 1, "fold": 1, "fused": 2}[plan] and info.nspan == 16
    st = d["init_state"].clone()
    y, f = ssd.ssd_fwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=st,
                       final_state=st, tuning=tuning)
    torch.cuda.synchronize()
    assert f.data_ptr() == st.data_ptr()
    yr, fr = oracle(p)
    assert O.rel_err(y.float().cpu(), yr) <= 1e-2 and O.rel_err(st.cpu(), fr) <= 1e-2


def projection(p, dev=DEV):
    """x, B, C and d_raw as views of one [b, L, H*P + 2*G*N + H] buffer (the
    output of one linear map of the input), filled with the problem's
    values."""
    b, L, H, P = p["x"].shape
    G, N = p["B"].shape[2], p["B"].shape[3]
    W = H * P + 2 * G * N + H
    proj = torch.empty((b, L, W), dtype=p["x"].dtype)
    proj[..., :H * P] = p["x"].reshape(b, L, H * P)
    proj[..., H * P:H * P + G * N] = p["B"].reshape(b, L, G * N)
    proj[..., H * P + G * N:H * P + 2 * G * N] = p["C"].reshape(b, L, G * N)
    proj[..., H * P + 2 * G * N:] = p["d_raw"]
    proj = proj.to(dev)
    views = {"x": proj[..., :H * P].view(b, L, H, P),
             "B": proj[..., H * P:H * P + G * N].view(b, L, G, N),
             "C": proj[..., H * P + G * N:H * P + 2 * G * N].view(b, L, G, N),
             "d_raw": proj[..., H * P + 2 * G * N:]}
    return proj, views


@pytest.mark.parametrize("tuning", [None, {"kernel": "hw"}, {"kernel": "span", "state_pass": "fused"},
                                    {"kernel": "span", "state_pass": "pass"}, {"state_f32": 1}],
                         ids=["default", "hw", "fused", "pass", "f32states"])
@pytest.mark.parametrize("reverse", [False, True])
def test_projection_views(ssd, tuning, reverse):
    """x, B, C and d_raw read through the strides of one projection buffer
    ([b, L, H*P + 2*G*N + H]), y written into the second half of a
    [b, L, H, 2P] buffer; against the oracle on contiguous copies."""
    # H = 8 keeps a projection row (H*P + 2*G*N + H bf16 values) a whole
    # number of 16-byte units, as the strides of x, B and C must be
    p = random_problem(211, 2, 700, 8, 64, 128, dtype="bf16", init_scale=0.5)
    proj, v = projection(p)
    b, L, H, P = p["x"].shape
    ycat = torch.zeros((b, L, H, 2 * P), dtype=torch.bfloat16, device=DEV)
    d_init_state = p["init_state"].to(DEV)
    y, f = ssd.ssd_fwd(v["x"], v["d_raw"], p["d_init"], v["B"], v["C"], init_state=d_init_state,
                       reverse=reverse, y=ycat[..., P:], tuning=tuning)
    torch.cuda.synchronize()
    yr, fr = oracle(p, reverse)
    ey, ef = O.rel_err(y.float().cpu(), yr), O.rel_err(f.cpu(), fr)
    print(f"projection {tuning} rev={reverse} y_err={ey:.3e} final_err={ef:.3e}", flush=True)
    assert ey <= 1e-2 and ef <= 1e-2
    assert bool((ycat[..., :P] == 0).all())


@pytest.mark.parametrize("cfg", [2, 3])
def test_state_f32_option(ssd, cfg):
    """Span states kept in float32 for bf16 inputs (the uncompressed
    reference point of 16-bit state storage): same bound, and the error
    against the oracle of both options is printed."""
    w = WORKLOADS[cfg]
    p = make_inputs(w)
    yr, fr = oracle(p)
    errs = {}
    for opt in (0, 1):
        y, f = run(ssd, p, tuning={"kernel": "span", "state_f32": opt})
        errs[opt] = (O.rel_err(y, yr), O.rel_err(f, fr))
        assert max(errs[opt]) <= 1e-2
    print(f"{w.name} bf16 states y/final err {errs[0][0]:.3e}/{errs[0][1]:.3e}, "
          f"f32 states {errs[1][0]:.3e}/{errs[1][1]:.3e}", flush=True)


# ------------------------------------------------------------ stage level
def _span_states(ssd, call, plan, H, P, N):
    """The span states and decays that the state stage (and, in plan 0, the
    pass) leave in the workspace, as [nspan][H][N][P] float and [nspan][H]:
    states from byte 256 in MFMA result order (entry (n, p) at
    ((pb * N/16 + nb) * 64 + lane) * 4 + i, n = 16 nb + 4 (lane / 16) + i,
    p = 16 pb + lane % 16), the decays at the next 256-byte boundary."""
    ws = call.workspace
    ns, esz = plan.nspan, plan.state_bytes
    n = ns * H * P * N
    raw = ws[256:256 + n * esz].view(torch.bfloat16 if esz == 2 else torch.float32)
    a = raw.float().cpu().reshape(ns, H, P // 16, N // 16, 4, 16, 4)
    st = a.permute(0, 1, 3, 4, 6, 2, 5).reshape(ns, H, N, P)
    off = (256 + n * esz + 255) // 256 * 256
    dec = ws[off:off + ns * H * 4].view(torch.float32).cpu().reshape(ns, H)
    return st.double().numpy(), dec.double().numpy()


def _span_ranges(L, K, j, reverse):
    """Tokens of span j (K chunks of 64) of a length-L sequence, in the
    original order; with reverse the spans run from the sequence's end."""
    a, b = 64 * K * j, min(64 * K * (j + 1), L)
    return (L - b, L - a) if reverse else (a, b)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("dtype,f32_states", [("bf16", 0), ("bf16", 1), ("f32", 0)])
def test_stage_span_states_and_pass(ssd, dtype, f32_states, reverse):
    """Stage-level parity of plan 0: after the state stage alone, every
    span's local state (from a zero state over its own tokens) and its decay
    product against the oracle run on that span's tokens; after the pass
    stage, every span slot holds the state entering the span (the oracle's
    state after the tokens before it, from init_state) and final_state the
    state after the whole sequence.  Two sequences of 13 chunks (spans of
    4, 4, 4 and 1 chunks, the last one ragged) and two column groups."""
    b, L, H, P, N = 2, 64 * 12 + 17, 3, 80, 64
    p = random_problem(211, b, L, H, P, N, dtype=dtype, init_scale=0.5, d_init=-3.0)
    d = to_dev(p)
    tun = {"kernel": "span", "state_pass": "pass", "chunks_per_span": 4, "state_f32": f32_states}
    call = ssd.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], init_state=d["init_state"],
                       reverse=reverse, tuning=tun)
    plan = ssd.ssd_fwd_plan(call.dims, tun)
    assert plan.fused_pass == 0 and plan.head_wave == 0 and plan.chunks_per_span == 4
    sps = plan.nspan // b
    assert sps == 4
    tol = 1e-5 if dtype == "f32" else 1e-2
    dd = O.delta(O.as_f64(p["d_raw"]), p["d_init"])

    call.run(ssd.STAGE_TABLE | ssd.STAGE_STATE)
    torch.cuda.synchronize()
    st, dec = _span_states(ssd, call, plan, H, P, N)
    ref_st, ref_dec = np.zeros_like(st), np.zeros_like(dec)
    for s in range(b):
        for j in range(sps):
            t0, t1 = _span_ranges(L, 4, j, reverse)
            sl = lambda t: t[s:s + 1, t0:t1]
            _, f = O.ssd_ref_seq(sl(p["x"]), sl(p["d_raw"]), p["d_init"], sl(p["B"]), sl(p["C"]),
                                 reverse=reverse)
            ref_st[s * sps + j] = f[0]
            ref_dec[s * sps + j] = -dd[s, t0:t1].sum(axis=0)
    # decays compared as logs: the kernel sums up to 256 fp32 log-steps
    es = O.rel_err(st, ref_st)
    ed = float(np.max(np.abs(np.log(dec) - ref_dec) / np.abs(ref_dec)))
    print(f"stage state {dtype} f32_states={f32_states} rev={reverse}: states {es:.3e} "
          f"decays {ed:.3e}", flush=True)
    assert es <= tol and ed <= 1e-4

    call.run(ssd.STAGE_PASS)
    torch.cuda.synchronize()
    st, _ = _span_states(ssd, call, plan, H, P, N)
    fin = call.final_state.cpu().double().numpy()
    ref_in, ref_fin = np.zeros_like(st), np.zeros_like(fin)
    for s in range(b):
        init = O.as_f64(p["init_state"])[s:s + 1]
        for j in range(sps):
            t0, t1 = _span_ranges(L, 4, j, reverse)
            a, e = (t1, L) if reverse else (0, t0)   # the tokens processed before span j
            if e > a:
                sl = lambda t: t[s:s + 1, a:e]
                _, f = O.ssd_ref_seq(sl(p["x"]), sl(p["d_raw"]), p["d_init"], sl(p["B"]),
                                     sl(p["C"]), init_state=init, reverse=reverse)
                ref_in[s * sps + j] = f[0]
            else:
                ref_in[s * sps + j] = init[0]
        sl = lambda t: t[s:s + 1]
        _, f = O.ssd_ref_seq(sl(p["x"]), sl(p["d_raw"]), p["d_init"], sl(p["B"]), sl(p["C"]),
                             init_state=init, reverse=reverse)
        ref_fin[s] = f[0]
    ei, ef = O.rel_err(st, ref_in), O.rel_err(fin, ref_fin)
    print(f"stage pass {dtype} f32_states={f32_states} rev={reverse}: incoming {ei:.3e} "
          f"final {ef:.3e}", flush=True)
    assert ei <= tol and ef <= tol
