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
    assert 0 in codes and -7 in codes
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


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: every call below is rejected


def call(m, dims, **kw):
    args = dict(x=FAKE, d_raw=FAKE, d_init=-4.6, B=FAKE, C=FAKE, init=None, cu=None, reverse=0,
                y=FAKE, yst=(dims.nheads * dims.headdim) if dims else 64,
                ysh=dims.headdim if dims else 16, fin=None, ws=FAKE, wsb=1 << 40, stream=None)
    args.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    return m.library().ssd_fwd(
        ctypes.byref(dims) if dims else ctypes.POINTER(m.SsdDims)(), vp(args["x"]), vp(args["d_raw"]), args["d_init"], vp(args["B"]),
        vp(args["C"]), vp(args["init"]), vp(args["cu"]), args["reverse"], vp(args["y"]),
        args["yst"], args["ysh"], vp(args["fin"]), vp(args["ws"]), args["wsb"], vp(args["stream"]))


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
    assert call(m, ok, yst=64 * 2 + 4) == -4
    assert call(m, ok, ws=None) == -6                                  # WORKSPACE
    assert call(m, ok, wsb=16) == -6
    assert call(m, ok, ws=FAKE + 16) == -4


def test_binding_rejects_cpu_mismatch(m):
    x = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError):
        m.ssd_fwd(x, torch.zeros(1, 64, 3), -4.6, torch.zeros(1, 64, 1, 16),
                  torch.zeros(1, 64, 1, 16))


def test_plan_folds_state_pass_for_short_sequences(m, monkeypatch):
    """Batch mode with 1..8 spans per sequence folds the state pass into
    span_scan; packed sequences, longer ones and empty ones keep the three
    launches; SSD_FUSE_PASS forces any of the three plans in batch mode."""
    monkeypatch.delenv("SSD_FUSE_PASS", raising=False)
    monkeypatch.delenv("SSD_SPAN_CHUNKS", raising=False)
    monkeypatch.setenv("SSD_KERNEL", "span")
    layer_dims = m.make_dims(2, 2048, 24, 64, 128)
    layer = m.ssd_fwd_plan(layer_dims)
    assert layer.chunks_per_span == 4 and layer.fused_pass == 1
    long = m.ssd_fwd_plan(m.make_dims(1, 64 * 4 * 9, 2, 64, 128))
    assert long.chunks_per_span == 4 and long.fused_pass == 0
    varlen = m.ssd_fwd_plan(m.make_dims(1, 4096, 2, 64, 128, nseq=3))
    assert varlen.fused_pass == 0
    assert m.ssd_fwd_plan(m.make_dims(2, 0, 2, 64, 128)).fused_pass == 0
    for forced in (0, 1, 2):
        monkeypatch.setenv("SSD_FUSE_PASS", str(forced))
        assert m.ssd_fwd_plan(layer_dims).fused_pass == forced
        assert m.ssd_fwd_plan(m.make_dims(1, 4096, 2, 64, 128, nseq=3)).fused_pass == 0


def test_workspace_header_in_every_plan(m, monkeypatch):
    """Every plan reserves the 256-byte header at the start of the
    workspace; the fused plan adds one 8-byte ticket/epoch word per chain
    (sequence, head group, column group) and one 4-byte flag per
    workgroup."""
    monkeypatch.delenv("SSD_SPAN_CHUNKS", raising=False)
    monkeypatch.setenv("SSD_KERNEL", "span")
    sizes = {}
    for forced in (0, 1, 2):
        monkeypatch.setenv("SSD_FUSE_PASS", str(forced))
        sizes[forced] = m.ssd_fwd_workspace_bytes(m.make_dims(2, 2048, 24, 64, 128))
    assert sizes[0] == sizes[1]
    chains = 2 * 24  # sequences x heads x one column group
    nwg = chains * (2048 // 64 // 4)  # x spans per sequence
    assert sizes[2] - sizes[0] == -(-(chains * 8 + nwg * 4) // 256) * 256
    assert m.ssd_fwd_workspace_bytes(m.make_dims(2, 0, 2, 64, 128)) >= 256

def test_plan_head_wave_kernels(m, monkeypatch):
    """Large bf16 problems with d_state 64 / 128 run the head-wave kernels
    with three launches and long spans; small ones, fp32, other d_state
    values and SSD_KERNEL=span keep the span kernels; SSD_KERNEL=hw forces
    the head-wave kernels."""
    for v in ("SSD_FUSE_PASS", "SSD_SPAN_CHUNKS", "SSD_KERNEL", "SSD_HW_NPB", "SSD_HW_HEADS"):
        monkeypatch.delenv(v, raising=False)
    varlen = m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, nseq=16))
    assert (varlen.head_wave, varlen.chunks_per_span, varlen.cols_per_wave, varlen.heads_per_wg,
            varlen.fused_pass) == (1, 16, 32, 4, 0)
    bidir = m.ssd_fwd_plan(m.make_dims(1, 1 << 20, 8, 192, 64))
    assert (bidir.head_wave, bidir.chunks_per_span, bidir.cols_per_wave, bidir.heads_per_wg) == (1, 32, 32, 2)
    wide = m.ssd_fwd_plan(m.make_dims(1, 8192, 80, 64, 128))   # 10240 items: span kernels
    assert (wide.head_wave, wide.chunks_per_span, wide.fused_pass) == (0, 8, 0)
    assert m.ssd_fwd_plan(m.make_dims(2, 2048, 24, 64, 128)).head_wave == 0   # layer: span kernels
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, dtype=0)).head_wave == 0
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 32)).head_wave == 0
    monkeypatch.setenv("SSD_KERNEL", "hw")
    small = m.ssd_fwd_plan(m.make_dims(2, 2048, 24, 64, 128))
    assert small.head_wave == 1 and small.fused_pass == 0
    monkeypatch.setenv("SSD_KERNEL", "span")
    assert m.ssd_fwd_plan(m.make_dims(1, 65536, 24, 64, 128, nseq=16)).head_wave == 0


def call_bwd(m, dims, **kw):
    H, P = (dims.nheads, dims.headdim) if dims else (2, 16)
    args = dict(x=FAKE, d_raw=FAKE, d_init=-4.6, B=FAKE, C=FAKE, init=None, cu=None, reverse=0,
                y=FAKE, yst=H * P, ysh=P, dy=FAKE, gst=H * P, gsh=P, dfin=None, dx=FAKE,
                ddr=FAKE, dB=FAKE, dC=FAKE, dinit=None, ddi=None, ws=FAKE, wsb=1 << 40,
                stream=None)
    args.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    a = args
    return m.library().ssd_bwd(
        ctypes.byref(dims) if dims else ctypes.POINTER(m.SsdDims)(), vp(a["x"]), vp(a["d_raw"]),
        a["d_init"], vp(a["B"]), vp(a["C"]), vp(a["init"]), vp(a["cu"]), a["reverse"], vp(a["y"]),
        a["yst"], a["ysh"], vp(a["dy"]), a["gst"], a["gsh"], vp(a["dfin"]), vp(a["dx"]),
        vp(a["ddr"]), vp(a["dB"]), vp(a["dC"]), vp(a["dinit"]), vp(a["ddi"]), vp(a["ws"]),
        a["wsb"], vp(a["stream"]))


def test_bwd_workspace_bytes(m):
    """Two per-chunk state sets dominate: 2 * chunks * H * P * N * e, plus the
    head subsets' fp32 dB / dC partials; unsupported sizes give 0."""
    d = m.make_dims(2, 2048, 24, 64, 128)
    ws = m.ssd_bwd_workspace_bytes(d)
    states = 2 * 64 * 24 * 64 * 128 * 2
    assert states < ws < states + 2 * 24 * 4096 * 128 * 4 + (1 << 20)
    assert ws % 256 == 0
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 192, 64)) > 0      # 3 column groups
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 64, 256)) == 0      # d_state 256
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 16, 64, dtype=0)) == 0
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 64, 2, 16, 32, dtype=0)) > 0
    assert m.ssd_bwd_workspace_bytes(m.make_dims(1, 0, 2, 16, 16)) > 0         # empty input


def test_bwd_head_subsets(m, monkeypatch):
    """The gradient kernel's head subsets: the largest divisor of the group's
    heads that keeps >= 256 workgroups (one per CU) -- fewer subsets, smaller partials."""
    few = m.ssd_bwd_workspace_bytes(m.make_dims(1, 64 * 1024, 24, 64, 128))   # 1024 chunks
    monkeypatch.setenv("SSD_BWD_HEADS", "1")
    many = m.ssd_bwd_workspace_bytes(m.make_dims(1, 64 * 1024, 24, 64, 128))
    part = (24 - 1) * 2 * 64 * 1024 * 128 * 4   # 23 more subsets of dB and dC partials
    assert part <= many - few < part + (1 << 20)


@needs_no_gpu
def test_bwd_rejects_bad_arguments(m):
    ok = m.make_dims(1, 128, 2, 64, 128)
    assert call_bwd(m, None) == -1
    assert call_bwd(m, ok, dy=None) == -1                                  # NULL_ARG
    assert call_bwd(m, ok, dB=None) == -1
    assert call_bwd(m, ok, y=None) == -1
    assert call_bwd(m, m.make_dims(1, 128, 2, 64, 256)) == -5
    assert call_bwd(m, m.make_dims(1, 128, 2, 24, 128)) == -2
    assert call_bwd(m, m.make_dims(1, 128, 2, 64, 128, nseq=2)) == -1      # cu_seqlens missing
    assert call_bwd(m, ok, cu=FAKE) == -2
    assert call_bwd(m, ok, reverse=3) == -2
    assert call_bwd(m, ok, dy=FAKE + 8) == -4                              # ALIGN
    assert call_bwd(m, ok, dx=FAKE + 4) == -4
    assert call_bwd(m, ok, gst=64 * 2 + 4) == -4
    assert call_bwd(m, ok, gst=1 << 25) == -2
    assert call_bwd(m, ok, ddr=FAKE + 1) == -4
    assert call_bwd(m, ok, ws=None) == -6                                  # WORKSPACE
    assert call_bwd(m, ok, wsb=16) == -6
