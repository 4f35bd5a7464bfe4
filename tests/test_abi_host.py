"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function include/ssd.h declares, and
rejects bad arguments with the documented status before any HIP call.
Calls that pass made-up device pointers only use argument sets that the
host checks must reject; they are skipped where a GPU is visible so that a
regression in the checks can never launch a kernel on such pointers.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def m():
    import mamba_ssd_chunked_02_amd as m
    m.library()
    return m


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def header_define(name):
    return int(re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read()).group(1))


def test_exports_every_declared_function(m):
    lib = ctypes.CDLL(m._binding.LIB_PATH)
    names = header_functions()
    assert set(names) >= {"ssd_abi_version", "ssd_fwd", "ssd_fwd_workspace_bytes",
                          "ssd_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(m):
    assert m.ssd_abi_version() == header_define("SSD_ABI_VERSION")


def test_status_strings(m):
    codes = [int(v) for v in re.findall(r"SSD_(?:OK|ERR_\w+)\s*=\s*(-?\d+)", open(HEADER).read())]
    assert 0 in codes and -7 in codes and -9 in codes
    for c in codes:
        s = m.ssd_status_string(c)
        assert s and "unknown ssd status" not in s
    assert "unknown ssd status" in m.ssd_status_string(12345)


def test_workspace_bytes(m):
    from ssd_inputs import WORKLOADS
    for w in WORKLOADS.values():
        d = m.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.d_state, w.ngroups,
                        w.chunk_size, w.nseq, m.SSD_BF16 if w.dtype == "bf16" else m.SSD_F32)
        ws = m.ssd_fwd_workspace_bytes(d)
        # the span states dominate: at most one N x P float state per chunk-head
        nch = w.tokens // 64 + w.nseq + w.batch
        assert 0 < ws <= nch * w.nheads * w.headdim * w.d_state * 4 + (1 << 20) * (1 + w.nseq)
        assert ws % 256 == 0
    assert m.ssd_fwd_workspace_bytes(m.make_dims(1, 64, 2, 16, 16, chunk_size=32)) == 0
    assert m.ssd_fwd_workspace_bytes(m.make_dims(1, 64, 2, 24, 16)) == 0
    assert m.ssd_fwd_workspace_bytes(m.make_dims(2, 64, 2, 16, 16, nseq=3)) == 0
    # sequences x heads x state entries: 2^33 and more are out of range (the
    # state pass decodes its threads in 32 bits), just below is accepted
    assert m.ssd_fwd_workspace_bytes(m.make_dims(1 << 12, 64, 64, 256, 128)) == 0
    assert m.ssd_fwd_workspace_bytes(m.make_dims((1 << 12) - 1, 64, 64, 256, 128)) > 0


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: every call below is rejected


def lay(m, dims, **kw):
    """A layout for dims (contiguous unless fields are given)."""
    H, P, G, N = dims.nheads, dims.headdim, dims.ngroups, dims.d_state
    l = m.SsdLayout(H * P, P, H, 1, G * N, N, G * N, N, H * P, P, H * P, P)
    for k, v in kw.items():
        setattr(l, k, v)
    return l


def call(m, dims, layout=None, tuning=None, **kw):
    args = dict(x=FAKE, d_raw=FAKE, d_init=-4.6, B=FAKE, C=FAKE, init=None, cu=None, reverse=0,
                y=FAKE, fin=None, ws=FAKE, wsb=1 << 40, stream=None)
    args.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    a = args
    rest = (vp(a["x"]), vp(a["d_raw"]), a["d_init"], vp(a["B"]), vp(a["C"]), vp(a["init"]),
            vp(a["cu"]), a["reverse"], vp(a["y"]), vp(a["fin"]), vp(a["ws"]), a["wsb"],
            vp(a["stream"]))
    dp = ctypes.byref(dims) if dims else ctypes.POINTER(m.SsdDims)()
    lp = ctypes.byref(layout) if layout is not None else ctypes.POINTER(m.SsdLayout)()
    if tuning is None:
        return m.library().ssd_fwd(dp, lp, *rest)
    t = m.make_tuning(tuning)
    return m.library().ssd_fwd_ex(15, dp, ctypes.byref(t), lp, *rest)


needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="made-up pointers are only passed where no GPU exists")


@needs_no_gpu
def test_rejects_bad_arguments(m):
    ok = m.make_dims(1, 128, 2, 64, 128)
    assert call(m, None) == -1
    assert call(m, ok, x=None) == -1                                   # NULL_ARG
    assert call(m, ok, y=None) == -1
    assert call(m, m.make_dims(1, 128, 2, 64, 128, dtype=7)) == -3     # DTYPE
    assert call(m, m.make_dims(1, 128, 2, 64, 128, chunk_size=32)) == -5  # UNSUPPORTED
    assert call(m, m.make_dims(1, 128, 2, 64, 48)) == -5
    assert call(m, m.make_dims(1, 128, 2, 64, 256, dtype=0)) == -5
    assert call(m, m.make_dims(1, 128, 2, 24, 128)) == -2              # SHAPE headdim
    assert call(m, m.make_dims(1, 128, 3, 64, 128, ngroups=2)) == -2   # H % G
    assert call(m, m.make_dims(2, 128, 2, 64, 128, nseq=2)) == -2      # varlen needs b == 1
    assert call(m, m.make_dims(1, 128, 2, 64, 128, nseq=2)) == -1      # cu_seqlens missing
    assert call(m, ok, cu=FAKE) == -2                                  # cu without nseq
    assert call(m, ok, reverse=2) == -2
    assert call(m, ok, x=FAKE + 8) == -4                               # ALIGN
    assert call(m, ok, y=FAKE + 2) == -4
    assert call(m, ok, d_raw=FAKE + 1) == -4                           # d_raw: bf16 elements
    assert call(m, ok, ws=None) == -6                                  # WORKSPACE
    assert call(m, ok, wsb=16) == -6
    assert call(m, ok, ws=FAKE + 16) == -4


def test_bidir_workspace_bytes(m):
    """Two forward workspaces, each rounded up to 256 bytes; 0 for sizes
    ssd_fwd rejects."""
    from ssd_inputs import WORKLOADS
    for w in WORKLOADS.values():
        d = m.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.d_state, w.ngroups,
                        w.chunk_size, w.nseq, m.SSD_BF16 if w.dtype == "bf16" else m.SSD_F32)
        one = m.ssd_fwd_workspace_bytes(d)
        assert m.library().ssd_fwd_bidir_workspace_bytes(ctypes.byref(d)) == 2 * ((one + 255) // 256 * 256)
    bad = m.make_dims(1, 64, 2, 24, 16)
    assert m.library().ssd_fwd_bidir_workspace_bytes(ctypes.byref(bad)) == 0


def call_bidir(m, dims, **kw):
    args = dict(x=FAKE, d_raw=FAKE, B=FAKE, C=FAKE, init_f=None, init_r=None, y_f=FAKE,
                y_r=FAKE + 4096, fin_f=None, fin_r=None, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    a = args
    return m.library().ssd_fwd_bidir(
        ctypes.byref(dims), None, None, vp(a["x"]), vp(a["d_raw"]), -4.6, vp(a["B"]), vp(a["C"]),
        vp(a["init_f"]), vp(a["init_r"]), vp(a["y_f"]), vp(a["y_r"]), vp(a["fin_f"]),
        vp(a["fin_r"]), vp(a["ws"]), a["wsb"], None)


@needs_no_gpu
def test_bidir_rejects_bad_arguments(m):
    """Either direction's bad argument is reported before anything is queued
    (a launch with these made-up pointers would fail with SSD_ERR_HIP)."""
    ok = m.make_dims(1, 1024, 2, 64, 128)
    half = (m.ssd_fwd_workspace_bytes(ok) + 255) // 256 * 256
    assert call_bidir(m, ok, x=None) == -1
    assert call_bidir(m, ok, y_r=None) == -1
    assert call_bidir(m, ok, y_r=FAKE + 2) == -4
    assert call_bidir(m, ok, ws=None) == -6
    assert call_bidir(m, ok, wsb=half) == -6                        # one direction's worth
    assert call_bidir(m, ok, init_r=FAKE, fin_r=FAKE + 64) == -9    # OVERLAP
    assert call_bidir(m, m.make_dims(1, 1024, 2, 64, 128, nseq=2)) == -2  # batch mode only


@needs_no_gpu
def test_rejects_bad_strides(m):
    """Rows of x, B, C and y are 16-byte units; every stride is >= 0 and
    <= 2^24 elements; d_raw's strides may be any element count."""
    ok = m.make_dims(1, 128, 2, 64, 128)
    for field in ("x_token", "x_head", "B_token", "B_group", "C_token", "C_group",
                  "y_token", "y_head"):
        assert call(m, ok, layout=lay(m, ok, **{field: 4 + 128})) == -4, field   # 8 bytes off
        assert call(m, ok, layout=lay(m, ok, **{field: -8})) == -2, field
        assert call(m, ok, layout=lay(m, ok, **{field: (1 << 24) + 8})) == -2, field
    for field in ("d_raw_token", "d_raw_head"):
        assert call(m, ok, layout=lay(m, ok, **{field: -1})) == -2, field
        assert call(m, ok, layout=lay(m, ok, **{field: (1 << 24) + 1})) == -2, field
    # an odd d_raw stride is fine: the call goes on to the workspace check
    assert call(m, ok, layout=lay(m, ok, d_raw_token=1817, d_raw_head=3), ws=None) == -6


@needs_no_gpu
def test_rejects_partly_overlapping_states(m):
    """final_state may be init_state itself (the separate pass reads each
    entry before writing it), but not overlap it at another offset."""
    ok = m.make_dims(1, 128, 2, 64, 128)
    assert call(m, ok, init=FAKE, fin=FAKE + 4096) == -9
    assert call(m, ok, init=FAKE + 4096, fin=FAKE) == -9
    # the same buffer passes the overlap check (rejected later for the workspace)
    assert call(m, ok, init=FAKE, fin=FAKE, ws=None) == -6
    # disjoint buffers too
    assert call(m, ok, init=FAKE, fin=FAKE + 2 * 128 * 64 * 4, ws=None) == -6


@needs_no_gpu
def test_rejects_bad_tuning(m):
    ok = m.make_dims(1, 128, 2, 64, 128)
    t = m.SsdTuning()
    t.reserved[3] = 1
    assert call(m, ok, tuning=t) == -2
    assert call(m, ok, tuning={"kernel": 3}) == -2
    assert call(m, ok, tuning={"chunks_per_span": 65}) == -2
    assert call(m, ok, tuning={"state_pass": 4}) == -2
    assert call(m, ok, tuning={"cols_per_wave": 48}) == -2
    assert call(m, ok, tuning={"kernel": "hw", "cols_per_wave": 64}) == -2   # 64 needs d_state 64
    assert call(m, ok, tuning={"heads_scan": 3}) == -2
    assert call(m, m.make_dims(1, 128, 2, 64, 128, dtype=0), tuning={"kernel": "hw"}) == -5
    assert call(m, ok, tuning={"state_f32": 1, "state_pass": "fused"}) == -2
    varlen = m.make_dims(1, 128, 2, 64, 128, nseq=2)
    assert call(m, varlen, tuning={"state_pass": "fold"}, cu=FAKE) == -2


def test_binding_rejects_cpu_mismatch(m):
    x = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError):
        m.ssd_fwd(x, torch.zeros(1, 64, 3), -4.6, torch.zeros(1, 64, 1, 16),
                  torch.zeros(1, 64, 1, 16))


def test_layout_of_projection_views(m):
    """x, B, C and d_raw as views of one [b, L, H*P + 2*G*N + H] projection
    buffer: the binding reads their strides into the layout."""
    b, L, H, P, G, N = 2, 16, 3, 32, 1, 64
    W = H * P + 2 * G * N + H
    proj = torch.zeros(b, L, W, dtype=torch.bfloat16)
    x = proj[..., :H * P].view(b, L, H, P)
    B = proj[..., H * P:H * P + G * N].view(b, L, G, N)
    C = proj[..., H * P + G * N:H * P + 2 * G * N].view(b, L, G, N)
    dr = proj[..., H * P + 2 * G * N:]
    l = m.layout_of(x, dr, B, C)
    assert (l.x_token, l.x_head, l.B_token, l.B_group, l.C_token, l.C_group,
            l.d_raw_token, l.d_raw_head) == (W, P, W, N, W, N, W, 1)
    # every other token keeps batch rows L' token strides apart: allowed
    m.layout_of(x[:, ::2], dr[:, ::2], B[:, ::2], C[:, ::2])
    with pytest.raises(ValueError):          # batch rows not L tokens apart
        m.layout_of(x[:, :L - 2], dr[:, :L - 2], B[:, :L - 2], C[:, :L - 2])


def test_plan_folds_state_pass_for_short_sequences(m):
    """Batch mode with 1..8 spans per sequence folds the state pass into
    span_scan; packed sequences, longer ones and empty ones keep the three
    launches; tuning.state_pass forces any of the three plans in batch mode."""
    span = {"kernel": "span"}
    layer_dims = m.make_dims(2, 2048, 24, 64, 128)
    layer = m.ssd_fwd_plan(layer_dims, span)
    assert layer.chunks_per_span == 4 and layer.fused_pass == 1
    long = m.ssd_fwd_plan(m.make_dims(1, 64 * 4 * 9, 2, 64, 128), span)
    assert long.chunks_per_span == 4 and long.fused_pass == 0
    varlen = m.ssd_fwd_plan(m.make_dims(1, 4096, 2, 64, 128, nseq=3), span)
    assert varlen.fused_pass == 0
    assert m.ssd_fwd_plan(m.make_dims(2, 0, 2, 64, 128), span).fused_pass == 0
    for forced in (0, 1, 2):
        assert m.ssd_fwd_plan(layer_dims, {"kernel": "span", "state_pass": forced + 1}).fused_pass == forced


def test_workspace_header_in_every_plan(m):
    """Every plan reserves the 256-byte header at the start of the
    workspace; the fused plan adds one 8-byte ticket/epoch word per chain
    (sequence, head group, column group) and one 4-byte flag per
    workgroup."""
    d = m.make_dims(2, 2048, 24, 64, 128)
    sizes = {f: m.ssd_fwd_plan(d, {"kernel": "span", "state_pass": f + 1}).workspace_bytes
             for f in (0, 1, 2)}
    assert sizes[0] == sizes[1] == m.ssd_fwd_workspace_bytes(d)
    chains = 2 * 24  # sequences x heads x one column group
    nwg = chains * (2048 // 64 // 4)  # x spans per sequence
    assert sizes[2] - sizes[0] == -(-(chains * 8 + nwg * 4) // 256) * 256
    assert m.ssd_fwd_workspace_bytes(m.make_dims(2, 0, 2, 64, 128)) >= 256


def test_state_f32_doubles_span_states(m):
    """tuning.state_f32 stores the span states in float32: the state part of
    the workspace doubles for bf16 inputs; fp32 inputs are unchanged."""
    d = m.make_dims(2, 2048, 24, 64, 128)
    a = m.ssd_fwd_plan(d, {"kernel": "span"})
    b = m.ssd_fwd_plan(d, {"kernel": "span", "state_f32": 1})
    assert (a.state_bytes, b.state_bytes) == (2, 4)
    states = a.nspan * 24 * 64 * 128 * 2
    assert b.workspace_bytes - a.workspace_bytes == states
    f = m.make_dims(2, 2048, 24, 64, 128, dtype=0)
    assert m.ssd_fwd_plan(f, {"state_f32": 1}).workspace_bytes == m.ssd_fwd_workspace_bytes(f)


def test_plan_ignores_the_environment(m, monkeypatch):
    """The library reads no tuning from the environment: setting the names
    of the knobs it once had changes neither the plan nor the workspace."""
    dims = [m.make_dims(2, 2048, 24, 64, 128), m.make_dims(1, 65536, 24, 64, 128, nseq=16),
            m.make_dims(1, 1 << 20, 8, 192, 64)]
    before = [(m.ssd_fwd_workspace_bytes(d), m.ssd_bwd_workspace_bytes(d),
               tuple(getattr(m.ssd_fwd_plan(d), f) for f, _ in m.SsdPlanInfo._fields_[:10]))
              for d in dims]
    for k, v in {"SSD_KERNEL": "hw", "SSD_FUSE_PASS": "2", "SSD_SPAN_CHUNKS": "1",
                 "SSD_HW_NPB": "4", "SSD_HW_HEADS": "1", "SSD_HW_HEADS_STATE": "1",
                 "SSD_HEADS_STATE": "2", "SSD_HEADS_SCAN": "2", "SSD_BWD_HEADS": "1",
                 "SSD_BWD_STATE_CHUNKS": "1"}.items():
        monkeypatch.setenv(k, v)
    after = [(m.ssd_fwd_workspace_bytes(d), m.ssd_bwd_workspace_bytes(d),
              tuple(getattr(m.ssd_fwd_plan(d), f) for f, _ in m.SsdPlanInfo._fields_[:10]))
             for d in dims]
    assert before == after


def test_library_reads_only_ssd_check():
    """The only environment variable the library's sources read is SSD_CHECK."""
    src = os.path.join(ROOT, "mamba_ssd_chunked_02_amd", "csrc")
    names = set()
    for f in os.listdir(src):
        names |= set(re.findall(r'getenv\("(\w+)"\)', open(os.path.join(src, f)).read()))
    assert names == {"SSD_CHECK"}


def test_plan_head_wave_kernels(m):
    """Large bf16 problems with d_state 64 / 128 run the head-wave kernels
    with three launches and long spans; small ones, fp32, other d_state
    values and tuning.kernel = span keep the span kernels; tuning.kernel =
    hw forces the head-wave kernels."""
    varlen = m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, nseq=16))
    assert (varlen.head_wave, varlen.chunks_per_span, varlen.cols_per_wave, varlen.heads_per_wg,
            varlen.heads_per_state_wg, varlen.fused_pass) == (1, 16, 32, 4, 2, 0)
    bidir = m.ssd_fwd_plan(m.make_dims(1, 1 << 20, 8, 192, 64))
    assert (bidir.head_wave, bidir.chunks_per_span, bidir.cols_per_wave, bidir.heads_per_wg) == (1, 64, 32, 2)
    wide = m.ssd_fwd_plan(m.make_dims(1, 8192, 80, 64, 128))   # 10240 items: span kernels
    assert (wide.head_wave, wide.chunks_per_span, wide.fused_pass) == (0, 8, 0)
    assert m.ssd_fwd_plan(m.make_dims(2, 2048, 24, 64, 128)).head_wave == 0   # layer: span kernels
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, dtype=0)).head_wave == 0
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 32)).head_wave == 0
    small = m.ssd_fwd_plan(m.make_dims(2, 2048, 24, 64, 128), {"kernel": "hw"})
    assert small.head_wave == 1 and small.fused_pass == 0
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, nseq=16),
                          {"kernel": "span"}).head_wave == 0
    shaped = m.ssd_fwd_plan(m.make_dims(1, 4096, 8, 64, 64),
                            {"kernel": "hw", "cols_per_wave": 64, "heads_scan": 1,
                             "chunks_per_span": 3})
    assert (shaped.cols_per_wave, shaped.heads_per_wg, shaped.chunks_per_span) == (64, 1, 3)


def call_bwd(m, dims, layout=None, **kw):
    args = dict(x=FAKE, d_raw=FAKE, d_init=-4.6, B=FAKE, C=FAKE, init=None, cu=None, reverse=0,
                y=FAKE, dy=FAKE, dfin=None, dx=FAKE, ddr=FAKE, dB=FAKE, dC=FAKE, dinit=None,
                ddi=None, ws=FAKE, wsb=1 << 40, stream=None)
    args.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    a = args
    lp = ctypes.byref(layout) if layout is not None else ctypes.POINTER(m.SsdLayout)()
    return m.library().ssd_bwd(
        ctypes.byref(dims) if dims else ctypes.POINTER(m.SsdDims)(), lp, vp(a["x"]),
        vp(a["d_raw"]), a["d_init"], vp(a["B"]), vp(a["C"]), vp(a["init"]), vp(a["cu"]),
        a["reverse"], vp(a["y"]), vp(a["dy"]), vp(a["dfin"]), vp(a["dx"]), vp(a["ddr"]),
        vp(a["dB"]), vp(a["dC"]), vp(a["dinit"]), vp(a["ddi"]), vp(a["ws"]), a["wsb"],
        vp(a["stream"]))


def test_bwd_workspace_bytes(m):
    """Two per-chunk state sets dominate: 2 * chunks * H * P * N * e, plus the
    head subsets' fp32 dB / dC partials; unsupported sizes give 0."""
    d = m.make_dims(2, 2048, 24, 64, 128)
    ws = m.ssd_bwd_workspace_bytes(d)
    states = 2 * 64 * 24 * 64 * 128 * 2
    assert states < ws < states + 2 * 24 * 4096 * 128 * 4 + (1 << 20)
    assert ws % 256 == 0
    assert m.ssd_fwd_plan(d).bwd_workspace_bytes == ws
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 192, 64)) > 0      # 3 column groups
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 64, 256)) == 0      # d_state 256
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 16, 64, dtype=0)) == 0
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 16, 32, dtype=0)) > 0
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 0, 2, 16, 16)) > 0         # empty input


def test_bwd_plan_of_layer_workload(m):
    """The layer workload (2 x 2048 tokens, 24 heads): 6 heads per gradient
    workgroup, 4 head subsets of dB / dC partials, four-chunk chunk-state
    walks."""
    info = m.ssd_fwd_plan(m.make_dims(2, 2048, 24, 64, 128))
    assert (info.bwd_heads_per_wg, info.bwd_head_subsets, info.bwd_state_chunks) == (6, 4, 4)


def test_bwd_head_subsets(m):
    """The gradient kernel's head subsets: the largest divisor of the group's
    heads that keeps >= 256 workgroups (one per CU) -- fewer subsets, smaller partials."""
    d = m.make_dims(1, 64 * 1024, 24, 64, 128)   # 1024 chunks
    few = m.ssd_bwd_workspace_bytes(d)
    many = m.ssd_fwd_plan(d, {"bwd_heads": 1}).bwd_workspace_bytes
    part = (24 - 1) * 2 * 64 * 1024 * 128 * 4   # 23 more subsets of dB and dC partials
    assert part <= many - few < part + (1 << 20)
    with pytest.raises(m.SsdError):
        m.ssd_fwd_plan(d, {"bwd_heads": 5})      # does not divide 24


@needs_no_gpu
def test_bwd_rejects_bad_arguments(m):
    ok = m.make_dims(1, 128, 2, 64, 128)
    assert call_bwd(m, None) == -1
    assert call_bwd(m, ok, dy=None) == -1                                  # NULL_ARG
    assert call_bwd(m, ok, dB=None) == -1
    # y is not read: NULL, a misaligned pointer or bad y strides pass the
    # argument checks (the NULL workspace then stops the call)
    assert call_bwd(m, ok, y=None, ws=None) == -6
    assert call_bwd(m, ok, y=FAKE + 4, ws=None) == -6
    assert call_bwd(m, ok, layout=lay(m, ok, y_token=1 << 25), ws=None) == -6
    assert call_bwd(m, m.make_dims(1, 128, 2, 64, 256)) == -5
    assert call_bwd(m, m.make_dims(1, 128, 2, 24, 128)) == -2
    assert call_bwd(m, m.make_dims(1, 128, 2, 64, 128, nseq=2)) == -1      # cu_seqlens missing
    assert call_bwd(m, ok, cu=FAKE) == -2
    assert call_bwd(m, ok, reverse=3) == -2
    assert call_bwd(m, ok, dy=FAKE + 8) == -4                              # ALIGN
    assert call_bwd(m, ok, dx=FAKE + 4) == -4
    assert call_bwd(m, ok, layout=lay(m, ok, dy_token=64 * 2 + 4)) == -4
    assert call_bwd(m, ok, layout=lay(m, ok, dy_token=1 << 25)) == -2
    assert call_bwd(m, ok, ddr=FAKE + 1) == -4
    assert call_bwd(m, ok, dfin=FAKE, dinit=FAKE + 256) == -9             # partial overlap
    assert call_bwd(m, ok, dfin=FAKE, dinit=FAKE, ws=None) == -6          # same buffer: allowed
    assert call_bwd(m, ok, ws=None) == -6                                  # WORKSPACE
    assert call_bwd(m, ok, wsb=16) == -6


def test_noalloc_rejects_sizes_past_its_scratch(m):
    """ssd_fwd_noalloc refuses sizes whose workspace exceeds its fixed
    64 MiB array with SSD_ERR_SCRATCH, before any HIP call (NULL pointers:
    nothing could be launched even if the check were missing)."""
    assert m.ssd_fwd_noalloc_max_bytes() == 64 << 20
    big = m.make_dims(4, 1 << 20, 8, 192, 64)
    assert m.ssd_fwd_workspace_bytes(big) > 64 << 20
    lay = m.SsdLayout(8 * 192, 192, 8, 1, 64, 64, 64, 64, 8 * 192, 192, 8 * 192, 192)
    rc = m.library().ssd_fwd_noalloc(ctypes.byref(big), ctypes.byref(lay), None, None, -4.6,
                                      None, None, None, None, 0, None, None, None)
    assert rc == -10
    assert "scratch" in m.ssd_status_string(-10)
    # the layer, wide and packed workloads fit
    for d in (m.make_dims(2, 2048, 24, 64, 128), m.make_dims(1, 8192, 80, 64, 128),
              m.make_dims(1, 65536, 24, 64, 128, nseq=16)):
        assert m.ssd_fwd_workspace_bytes(d) <= 64 << 20
