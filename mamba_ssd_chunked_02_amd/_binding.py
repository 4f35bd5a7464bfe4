"""ctypes binding of libssd (include/ssd.h): argument marshalling only.

Every step of the scan runs in the HIP library; this module maps torch
tensors to pointers and sizes, allocates outputs and workspace with torch,
and passes torch's current HIP stream.  Workspaces it allocates start
zero-filled, as the library requires before a workspace's first use.  If libssd.so is missing the import
of the library raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_F32 = 0
SSD_BF16 = 1
CHUNK = 64

_DTYPES = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}


class SsdDims(ctypes.Structure):
    """Mirror of ``ssd_dims`` in include/ssd.h."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int32),
        ("headdim", ctypes.c_int32),
        ("d_state", ctypes.c_int32),
        ("ngroups", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("nseq", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


STAGE_TABLE, STAGE_STATE, STAGE_PASS, STAGE_SCAN, STAGE_ALL = 1, 2, 4, 8, 15


class SsdLayout(ctypes.Structure):
    """Mirror of ``ssd_layout`` in include/ssd.h (element strides)."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "x_token", "x_head", "d_raw_token", "d_raw_head", "B_token", "B_group",
        "C_token", "C_group", "y_token", "y_head", "dy_token", "dy_head")]


TUNING_FIELDS = ("kernel", "chunks_per_span", "state_pass", "heads_state", "heads_scan",
                 "cols_per_wave", "bwd_heads", "bwd_state_chunks", "state_f32")


class SsdTuning(ctypes.Structure):
    """Mirror of ``ssd_tuning`` in include/ssd.h (0 = the planner's choice)."""
    _fields_ = [(n, ctypes.c_int32) for n in TUNING_FIELDS] + [("reserved", ctypes.c_int32 * 7)]


def make_tuning(tuning):
    """``None`` or a dict of ssd_tuning fields -> SsdTuning or None.  Readable
    values are accepted for two fields: kernel "span" / "hw", state_pass
    "pass" / "fold" / "fused"."""
    if tuning is None:
        return None
    if isinstance(tuning, SsdTuning):
        return tuning
    words = {"kernel": {"span": 1, "hw": 2},
             "state_pass": {"pass": 1, "fold": 2, "fused": 3}}
    t = SsdTuning()
    for k, v in tuning.items():
        if k not in TUNING_FIELDS:
            raise KeyError(f"unknown tuning field {k}")
        setattr(t, k, int(words.get(k, {}).get(v, v)))
    return t


class SsdPlanInfo(ctypes.Structure):
    """Mirror of ``ssd_plan_info`` in include/ssd.h."""
    _fields_ = [
        ("chunks_per_span", ctypes.c_int32),
        ("col_groups", ctypes.c_int32),
        ("nspan", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
        ("fused_pass", ctypes.c_int32),
        ("head_wave", ctypes.c_int32),
        ("heads_per_wg", ctypes.c_int32),
        ("cols_per_wave", ctypes.c_int32),
        ("heads_per_state_wg", ctypes.c_int32),
        ("state_bytes", ctypes.c_int32),
        ("bwd_workspace_bytes", ctypes.c_uint64),
        ("bwd_heads_per_wg", ctypes.c_int32),
        ("bwd_head_subsets", ctypes.c_int32),
        ("bwd_state_chunks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str = "ssd_fwd"):
        self.status = status
        super().__init__(f"{where} returned {status}: {ssd_status_string(status)}")


_lib = None


def library() -> ctypes.CDLL:
    """Load libssd.so (built by ``mamba_ssd_chunked_02_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with `python -m mamba_ssd_chunked_02_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.ssd_abi_version.restype = ctypes.c_int
        lib.ssd_abi_version.argtypes = []
        lib.ssd_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_fwd_workspace_bytes.argtypes = [ctypes.POINTER(SsdDims)]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        P_ = ctypes.c_void_p
        fwd_args = [
            ctypes.POINTER(SsdDims), ctypes.POINTER(SsdLayout),
            P_, P_, ctypes.c_float, P_, P_,
            P_, P_, ctypes.c_int32,
            P_, P_,
            P_, ctypes.c_size_t,
            P_,
        ]
        lib.ssd_fwd.restype = ctypes.c_int
        lib.ssd_fwd.argtypes = fwd_args
        lib.ssd_fwd_ex.restype = ctypes.c_int
        lib.ssd_fwd_ex.argtypes = [ctypes.c_uint32, ctypes.POINTER(SsdDims),
                                   ctypes.POINTER(SsdTuning)] + fwd_args[1:]
        lib.ssd_fwd_bidir_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_fwd_bidir_workspace_bytes.argtypes = [ctypes.POINTER(SsdDims)]
        lib.ssd_fwd_bidir.restype = ctypes.c_int
        lib.ssd_fwd_bidir.argtypes = [
            ctypes.POINTER(SsdDims), ctypes.POINTER(SsdTuning), ctypes.POINTER(SsdLayout),
            P_, P_, ctypes.c_float, P_, P_,
            P_, P_, P_, P_, P_, P_,
            P_, ctypes.c_size_t,
            P_,
        ]
        lib.ssd_fwd_plan.restype = ctypes.c_int
        lib.ssd_fwd_plan.argtypes = [ctypes.POINTER(SsdDims), ctypes.POINTER(SsdTuning),
                                     ctypes.POINTER(SsdPlanInfo)]
        lib.ssd_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_bwd_workspace_bytes.argtypes = [ctypes.POINTER(SsdDims)]
        bwd_args = [
            ctypes.POINTER(SsdDims), ctypes.POINTER(SsdLayout),
            P_, P_, ctypes.c_float, P_, P_,
            P_, P_, ctypes.c_int32,
            P_, P_, P_,
            P_, P_, P_, P_,
            P_, P_,
            P_, ctypes.c_size_t,
            P_,
        ]
        lib.ssd_bwd.restype = ctypes.c_int
        lib.ssd_bwd.argtypes = bwd_args
        lib.ssd_bwd_ex.restype = ctypes.c_int
        lib.ssd_bwd_ex.argtypes = [ctypes.POINTER(SsdDims), ctypes.POINTER(SsdTuning)] + bwd_args[1:]
        lib.ssd_fwd_noalloc.restype = ctypes.c_int
        lib.ssd_fwd_noalloc.argtypes = fwd_args[:11] + [P_]
        lib.ssd_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
        lib.ssd_fwd_noalloc_max_bytes.argtypes = []
        _lib = lib
    return _lib


def ssd_abi_version() -> int:
    return int(library().ssd_abi_version())


def ssd_status_string(status: int) -> str:
    return library().ssd_status_string(int(status)).decode()


def make_dims(batch, seqlen, nheads, headdim, d_state, ngroups=1, chunk_size=CHUNK,
              nseq=0, dtype=SSD_BF16) -> SsdDims:
    return SsdDims(int(batch), int(seqlen), int(nheads), int(headdim), int(d_state),
                   int(ngroups), int(chunk_size), int(nseq), int(dtype))


def ssd_fwd_workspace_bytes(dims: SsdDims) -> int:
    return int(library().ssd_fwd_workspace_bytes(ctypes.byref(dims)))


def ssd_fwd_plan(dims: SsdDims, tuning=None) -> SsdPlanInfo:
    """How the library splits these sizes (tuning: None or a dict of
    ssd_tuning fields)."""
    info = SsdPlanInfo()
    t = make_tuning(tuning)
    rc = library().ssd_fwd_plan(ctypes.byref(dims), None if t is None else ctypes.byref(t),
                                ctypes.byref(info))
    if rc != 0:
        raise SsdError(rc, "ssd_fwd_plan")
    return info


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def dims_for(x, B, chunk_size=CHUNK, cu_seqlens=None) -> SsdDims:
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return make_dims(b, L, H, P, N, G, chunk_size, nseq, _DTYPES[x.dtype])


def _token_strides(t, name, ndim):
    """(token, head/group) element strides of a [b, L, X(, Y)] tensor whose
    innermost dimension is contiguous and whose batch rows are L tokens
    apart (the flattened token index of the C ABI)."""
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if t.numel() == 0:  # nothing is read or written: the contiguous strides
        inner = t.shape[2] * (t.shape[3] if ndim == 4 else 1)
        return inner, (t.shape[3] if ndim == 4 else 1)
    b, L = t.shape[0], t.shape[1]
    if ndim == 4 and t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")
    if b > 1 and L > 0 and t.stride(0) != L * t.stride(1):
        raise ValueError(f"{name} needs batch stride L * token stride")
    return t.stride(1), t.stride(2)


def layout_of(x, d_raw, B, C, y=None, dy=None) -> SsdLayout:
    """The ssd_layout of these tensors (strided views allowed)."""
    lay = SsdLayout()
    lay.x_token, lay.x_head = _token_strides(x, "x", 4)
    lay.d_raw_token, lay.d_raw_head = _token_strides(d_raw, "d_raw", 3)
    lay.B_token, lay.B_group = _token_strides(B, "B", 4)
    lay.C_token, lay.C_group = _token_strides(C, "C", 4)
    yy = x if y is None else y
    lay.y_token, lay.y_head = _token_strides(yy, "y", 4)
    gg = yy if dy is None else dy
    lay.dy_token, lay.dy_head = _token_strides(gg, "dy", 4)
    return lay


class PreparedCall:
    """Marshalled arguments of one ssd_fwd call (tensors kept alive), so a
    loop can launch the same problem repeatedly with no re-marshalling."""

    def __init__(self, dims, tuning, layout, args, keep, y, final_state, workspace):
        self.dims = dims
        self.tuning = tuning
        self.layout = layout
        self.args = args
        self._keep = keep
        self.y = y
        self.final_state = final_state
        self.workspace = workspace

    def run(self, stages: int = STAGE_ALL, stream=None):
        """Launch the given stages on ``stream`` (torch's current stream of
        the tensors' device by default)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.y.device).cuda_stream
        lib = library()
        if stages == STAGE_ALL and self.tuning is None:
            rc = lib.ssd_fwd(ctypes.byref(self.dims), ctypes.byref(self.layout), *self.args,
                             ctypes.c_void_p(stream))
        else:
            t = None if self.tuning is None else ctypes.byref(self.tuning)
            rc = lib.ssd_fwd_ex(stages, ctypes.byref(self.dims), t, ctypes.byref(self.layout),
                                *self.args, ctypes.c_void_p(stream))
        if rc != 0:
            raise SsdError(rc)
        return self.y, self.final_state


def ssd_fwd(x, d_raw, d_init, B, C, chunk_size=CHUNK, init_state=None, cu_seqlens=None,
            reverse=False, y=None, final_state=True, workspace=None, tuning=None):
    """Run the SSD forward scan on the GPU.

    x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N] (bf16 or fp32, one dtype, on
    one GPU; strided views allowed as long as the innermost dimension is
    contiguous and batch rows are L tokens apart); init_state [S,H,N,P]
    fp32 or None; cu_seqlens [nseq+1] int32 (b must be 1) or None.  ``y``
    may be a preallocated [b,L,H,P] tensor or strided view (last dim
    contiguous).  Pass ``final_state=False`` to skip it or a [S,H,N,P] fp32
    tensor to fill (it may be ``init_state`` itself).  ``tuning``: None or
    a dict of ssd_tuning fields.  Returns (y, final_state or None).
    Launches on torch's current stream.
    """
    call = prepare(x, d_raw, d_init, B, C, chunk_size, init_state, cu_seqlens, reverse, y,
                   final_state, workspace, tuning)
    with torch.cuda.device(x.device):
        return call.run()


def prepare(x, d_raw, d_init, B, C, chunk_size=CHUNK, init_state=None, cu_seqlens=None,
            reverse=False, y=None, final_state=True, workspace=None,
            tuning=None) -> PreparedCall:
    """Check and marshal the arguments of ``ssd_fwd``; allocate y,
    final_state and the workspace when not given."""
    if x.dim() != 4 or d_raw.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N] expected")
    b, L, H, P = x.shape
    dev = x.device
    for name, t in (("d_raw", d_raw), ("B", B), ("C", C)):
        if t.device != dev or t.dtype != x.dtype:
            raise ValueError(f"{name} must be on {dev} with dtype {x.dtype}")
    if tuple(d_raw.shape) != (b, L, H) or tuple(B.shape[:2]) != (b, L) or B.shape != C.shape:
        raise ValueError("shape mismatch between x, d_raw, B and C")
    G, N = B.shape[2], B.shape[3]
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on the same device")
        cu_seqlens = cu_seqlens.contiguous()
    S = (cu_seqlens.numel() - 1) if cu_seqlens is not None else b
    if init_state is not None:
        if init_state.dtype != torch.float32 or tuple(init_state.shape) != (S, H, N, P) \
                or init_state.device != dev or not init_state.is_contiguous():
            raise ValueError(f"init_state must be contiguous float32 [{S},{H},{N},{P}] on {dev}")
    if y is None:
        y = torch.empty((b, L, H, P), dtype=x.dtype, device=dev)
    elif tuple(y.shape) != (b, L, H, P) or y.dtype != x.dtype or y.device != dev:
        raise ValueError("y must match x in shape, dtype and device")
    if final_state is True:
        final_state = torch.empty((S, H, N, P), dtype=torch.float32, device=dev)
    elif final_state is False or final_state is None:
        final_state = None
    elif tuple(final_state.shape) != (S, H, N, P) or final_state.dtype != torch.float32 \
            or not final_state.is_contiguous():
        raise ValueError(f"final_state must be contiguous float32 [{S},{H},{N},{P}]")
    dims = dims_for(x, B, chunk_size, cu_seqlens)
    lay = layout_of(x, d_raw, B, C, y)
    tun = make_tuning(tuning)
    if workspace is None:
        if tun is None:
            need = ssd_fwd_workspace_bytes(dims)  # 0 for invalid sizes: ssd_fwd reports why
        else:
            info = SsdPlanInfo()
            rc = library().ssd_fwd_plan(ctypes.byref(dims), ctypes.byref(tun), ctypes.byref(info))
            need = info.workspace_bytes if rc == 0 else 0
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(x), _ptr(d_raw), float(d_init), _ptr(B), _ptr(C),
            _ptr(init_state), _ptr(cu_seqlens), 1 if reverse else 0,
            _ptr(y), _ptr(final_state),
            _ptr(workspace), workspace.numel())
    keep = (x, d_raw, B, C, init_state, cu_seqlens)
    return PreparedCall(dims, tun, lay, args, keep, y, final_state, workspace)


def ssd_fwd_noalloc(x, d_raw, d_init, B, C, y, final_state=None, init_state=None,
                    cu_seqlens=None, reverse=False):
    """ssd_fwd_noalloc: the forward scan with the library's fixed per-GPU
    scratch instead of a workspace.  y (and final_state, if wanted) are the
    caller's preallocated outputs; nothing is allocated.  Returns (y,
    final_state)."""
    b, L, H, P = x.shape
    dims = dims_for(x, B, CHUNK, cu_seqlens)
    lay = layout_of(x, d_raw, B, C, y)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = library().ssd_fwd_noalloc(
            ctypes.byref(dims), ctypes.byref(lay), _ptr(x), _ptr(d_raw), float(d_init), _ptr(B),
            _ptr(C), _ptr(init_state), _ptr(cu_seqlens), 1 if reverse else 0, _ptr(y),
            _ptr(final_state), ctypes.c_void_p(stream))
    if rc != 0:
        raise SsdError(rc, "ssd_fwd_noalloc")
    return y, final_state


def ssd_fwd_noalloc_max_bytes() -> int:
    return int(library().ssd_fwd_noalloc_max_bytes())


class PreparedBidir:
    """Marshalled arguments of one ssd_fwd_bidir call (tensors kept alive)."""

    def __init__(self, dims, tuning, layout, args, keep, y, finals, workspace):
        self.dims = dims
        self.tuning = tuning
        self.layout = layout
        self.args = args
        self._keep = keep
        self.y = y
        self.final_states = finals
        self.workspace = workspace

    def run(self, stream=None):
        """Launch both directions on ``stream`` (torch's current stream of
        the tensors' device by default)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.y.device).cuda_stream
        t = None if self.tuning is None else ctypes.byref(self.tuning)
        rc = library().ssd_fwd_bidir(ctypes.byref(self.dims), t, ctypes.byref(self.layout),
                                     *self.args, ctypes.c_void_p(stream))
        if rc != 0:
            raise SsdError(rc, "ssd_fwd_bidir")
        return self.y, self.final_states


def prepare_bidir(x, d_raw, d_init, B, C, chunk_size=CHUNK, init_fwd=None, init_rev=None,
                  y=None, final_state=False, workspace=None, tuning=None) -> PreparedBidir:
    """Check and marshal the arguments of ``ssd_fwd_bidir`` (batch mode): the
    forward output goes to y[..., :P] and the reverse one to y[..., P:] of a
    [b,L,H,2P] tensor (allocated when not given); ``final_state=True``
    allocates both final states, or pass a (final_fwd, final_rev) pair."""
    if x.dim() != 4 or d_raw.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N] expected")
    b, L, H, P = x.shape
    dev = x.device
    for name, t in (("d_raw", d_raw), ("B", B), ("C", C)):
        if t.device != dev or t.dtype != x.dtype:
            raise ValueError(f"{name} must be on {dev} with dtype {x.dtype}")
    if tuple(d_raw.shape) != (b, L, H) or tuple(B.shape[:2]) != (b, L) or B.shape != C.shape:
        raise ValueError("shape mismatch between x, d_raw, B and C")
    N = B.shape[3]
    for name, st in (("init_fwd", init_fwd), ("init_rev", init_rev)):
        if st is not None and (st.dtype != torch.float32 or tuple(st.shape) != (b, H, N, P)
                               or st.device != dev or not st.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [{b},{H},{N},{P}] on {dev}")
    if y is None:
        y = torch.empty((b, L, H, 2 * P), dtype=x.dtype, device=dev)
    elif tuple(y.shape) != (b, L, H, 2 * P) or y.dtype != x.dtype or y.device != dev:
        raise ValueError("y must be [b,L,H,2P] with x's dtype and device")
    if final_state is True:
        finals = tuple(torch.empty((b, H, N, P), dtype=torch.float32, device=dev) for _ in range(2))
    elif final_state is False or final_state is None:
        finals = (None, None)
    else:
        finals = tuple(final_state)
        for f in finals:
            if f is not None and (tuple(f.shape) != (b, H, N, P) or f.dtype != torch.float32
                                  or not f.is_contiguous()):
                raise ValueError(f"final states must be contiguous float32 [{b},{H},{N},{P}]")
    dims = dims_for(x, B, chunk_size, None)
    yf, yr = y[..., :P], y[..., P:]
    lay = layout_of(x, d_raw, B, C, yf)
    tun = make_tuning(tuning)
    if workspace is None:
        if tun is None:
            need = int(library().ssd_fwd_bidir_workspace_bytes(ctypes.byref(dims)))
        else:
            info = SsdPlanInfo()
            rc = library().ssd_fwd_plan(ctypes.byref(dims), ctypes.byref(tun), ctypes.byref(info))
            need = 2 * ((info.workspace_bytes + 255) // 256 * 256) if rc == 0 else 0
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(x), _ptr(d_raw), float(d_init), _ptr(B), _ptr(C),
            _ptr(init_fwd), _ptr(init_rev), _ptr(yf), _ptr(yr), _ptr(finals[0]), _ptr(finals[1]),
            _ptr(workspace), workspace.numel())
    keep = (x, d_raw, B, C, init_fwd, init_rev, yf, yr)
    return PreparedBidir(dims, tun, lay, args, keep, y, finals, workspace)


def ssd_fwd_bidir(x, d_raw, d_init, B, C, chunk_size=CHUNK, init_state=None,
                  cu_seqlens=None, final_state=False, workspace=None, tuning=None):
    """Bidirectional scan: a forward pass and a reverse pass over the same
    inputs, outputs concatenated on the last dim -> y [b,L,H,2P].  The
    reverse pass runs each sequence from its end to its start and writes at
    each token's own position, so no flipped copies are made.  Both passes
    start from init_state.  Without cu_seqlens this is one ssd_fwd_bidir call
    (which forms both directions' span states in one pass where the spans
    allow); with them, two ssd_fwd calls.
    Returns (y, (final_fwd, final_rev) or None)."""
    b, L, H, P = x.shape
    if cu_seqlens is None:
        call = prepare_bidir(x, d_raw, d_init, B, C, chunk_size, init_state, init_state,
                             final_state=final_state, workspace=workspace, tuning=tuning)
        with torch.cuda.device(x.device):
            y, finals = call.run()
        return y, (finals if final_state else None)
    y = torch.empty((b, L, H, 2 * P), dtype=x.dtype, device=x.device)
    c0 = prepare(x, d_raw, d_init, B, C, chunk_size, init_state, cu_seqlens, False,
                 y=y[..., :P], final_state=final_state, workspace=workspace, tuning=tuning)
    c1 = prepare(x, d_raw, d_init, B, C, chunk_size, init_state, cu_seqlens, True,
                 y=y[..., P:], final_state=final_state, workspace=c0.workspace, tuning=tuning)
    with torch.cuda.device(x.device):
        _, ff = c0.run()
        _, fr = c1.run()
    return y, ((ff, fr) if final_state else None)


def ssd_bwd_workspace_bytes(dims: SsdDims) -> int:
    return int(library().ssd_bwd_workspace_bytes(ctypes.byref(dims)))


class PreparedBwd:
    """Marshalled arguments of one ssd_bwd call (tensors kept alive)."""

    def __init__(self, dims, tuning, layout, args, keep, grads, workspace):
        self.dims = dims
        self.tuning = tuning
        self.layout = layout
        self.args = args
        self._keep = keep
        self.grads = grads
        self.workspace = workspace

    def run(self, stream=None):
        if stream is None:
            stream = torch.cuda.current_stream(self.grads["dx"].device).cuda_stream
        lib = library()
        if self.tuning is None:
            rc = lib.ssd_bwd(ctypes.byref(self.dims), ctypes.byref(self.layout), *self.args,
                             ctypes.c_void_p(stream))
        else:
            rc = lib.ssd_bwd_ex(ctypes.byref(self.dims), ctypes.byref(self.tuning),
                                ctypes.byref(self.layout), *self.args, ctypes.c_void_p(stream))
        if rc != 0:
            raise SsdError(rc, "ssd_bwd")
        return self.grads


def _like(t):
    """An uninitialized tensor with t's shape and strides."""
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)


def prepare_bwd(x, d_raw, d_init, B, C, y, dy, chunk_size=CHUNK, init_state=None,
                cu_seqlens=None, reverse=False, d_final=None, workspace=None, tuning=None,
                grads=None) -> PreparedBwd:
    """Check and marshal the arguments of ``ssd_bwd``; allocate the
    gradients (dict: dx, dd_raw, dB, dC, dinit_state, dd_init) and the
    workspace when not given.  dx, dd_raw, dB and dC are laid out like x,
    d_raw, B and C (the library writes each gradient with its input's
    strides); ``grads`` may supply some or all of them, e.g. as views of one
    projection-gradient buffer laid out like the inputs' projection.  ``y``
    (the forward output) is optional: the library does not read it."""
    if x.dim() != 4 or d_raw.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N] expected")
    b, L, H, P = x.shape
    dev = x.device
    for name, t in (("d_raw", d_raw), ("B", B), ("C", C), ("y", y), ("dy", dy)):
        if t is None and name == "y":
            continue
        if t.device != dev or t.dtype != x.dtype:
            raise ValueError(f"{name} must be on {dev} with dtype {x.dtype}")
    if tuple(d_raw.shape) != (b, L, H) or tuple(B.shape[:2]) != (b, L) or B.shape != C.shape:
        raise ValueError("shape mismatch between x, d_raw, B and C")
    if (y is not None and tuple(y.shape) != (b, L, H, P)) or tuple(dy.shape) != (b, L, H, P):
        raise ValueError("y and dy must have x's shape")
    G, N = B.shape[2], B.shape[3]
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on the same device")
        cu_seqlens = cu_seqlens.contiguous()
    S = (cu_seqlens.numel() - 1) if cu_seqlens is not None else b
    for name, t in (("init_state", init_state), ("d_final", d_final)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (S, H, N, P)
                              or t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [{S},{H},{N},{P}] on {dev}")
    g = dict(grads or {})
    for k, src in (("dx", x), ("dd_raw", d_raw), ("dB", B), ("dC", C)):
        if k not in g:
            g[k] = _like(src)
        elif tuple(g[k].shape) != tuple(src.shape) or g[k].stride() != src.stride() \
                or g[k].dtype != src.dtype or g[k].device != dev:
            raise ValueError(f"{k} must have the shape, strides and dtype of its input")
    g.setdefault("dinit_state", torch.empty((S, H, N, P), dtype=torch.float32, device=dev))
    g.setdefault("dd_init", torch.empty((1,), dtype=torch.float32, device=dev))
    dims = dims_for(x, B, chunk_size, cu_seqlens)
    lay = layout_of(x, d_raw, B, C, y, dy)
    tun = make_tuning(tuning)
    if workspace is None:
        if tun is None:
            need = ssd_bwd_workspace_bytes(dims)  # 0 for unsupported sizes: ssd_bwd reports why
        else:
            info = SsdPlanInfo()
            rc = library().ssd_fwd_plan(ctypes.byref(dims), ctypes.byref(tun), ctypes.byref(info))
            need = info.bwd_workspace_bytes if rc == 0 else 0
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(x), _ptr(d_raw), float(d_init), _ptr(B), _ptr(C),
            _ptr(init_state), _ptr(cu_seqlens), 1 if reverse else 0,
            None, _ptr(dy), _ptr(d_final),
            _ptr(g["dx"]), _ptr(g["dd_raw"]), _ptr(g["dB"]), _ptr(g["dC"]),
            _ptr(g["dinit_state"]), _ptr(g["dd_init"]),
            _ptr(workspace), workspace.numel())
    keep = (x, d_raw, B, C, dy, init_state, cu_seqlens, d_final)
    return PreparedBwd(dims, tun, lay, args, keep, g, workspace)


def ssd_bwd(x, d_raw, d_init, B, C, y, dy, chunk_size=CHUNK, init_state=None,
            cu_seqlens=None, reverse=False, d_final=None, workspace=None, tuning=None,
            grads=None) -> dict:
    """Gradients of the SSD scan on the GPU: given the forward inputs (``y``,
    the forward output, is accepted for the call's shape but not read; None
    is fine), dL/dy (``dy``, same layout rules as y) and
    optionally dL/d final_state (``d_final``), returns a dict with dx,
    dd_raw, dB, dC (input dtype, each laid out like its input), dinit_state
    [S,H,N,P] and dd_init [1] (fp32).  Launches on torch's current stream."""
    call = prepare_bwd(x, d_raw, d_init, B, C, y, dy, chunk_size, init_state, cu_seqlens,
                       reverse, d_final, workspace, tuning, grads)
    with torch.cuda.device(x.device):
        return call.run()
