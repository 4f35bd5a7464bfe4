"""ctypes wrapper and build step for the C fp64 oracles (``ref_seq.c``, the
forward recurrence, and ``ref_bwd.c``, its adjoint).

Test infrastructure only (see ``ssd_oracle.py``).  ``build()`` compiles
``liboracle_ref.so`` next to this file with gcc -O3 -fopenmp, ISO C (no
floating-point contraction) and no fast-math, so the double arithmetic is
the plain IEEE one in the order the sources write it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "ref_seq.c"), os.path.join(HERE, "ref_bwd.c")]
LIB = os.path.join(HERE, "liboracle_ref.so")

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-o", LIB + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(f) for f in SRCS):
            build()
        lib = ctypes.CDLL(LIB)
        lib.ssd_oracle_seq.restype = ctypes.c_int
        lib.ssd_oracle_seq.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.ssd_oracle_threads.restype = ctypes.c_int
        lib.ssd_oracle_bwd.restype = ctypes.c_int
        lib.ssd_oracle_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def threads() -> int:
    return int(_load().ssd_oracle_threads())


def _f32(t):
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu().float().contiguous().numpy()
    return np.ascontiguousarray(t, dtype=np.float32)


def ssd_ref_seq_c(x, d_raw, d_init, B, C, init_state=None, cu_seqlens=None,
                  reverse=False):
    """Same contract as ``ssd_oracle.ssd_ref_seq``; runs the C oracle."""
    xf, df, Bf, Cf = _f32(x), _f32(d_raw), _f32(B), _f32(C)
    h0 = _f32(init_state)
    b, L, H, P = xf.shape
    G, N = Bf.shape[2], Bf.shape[3]
    cu = None
    nseq = 0
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        nseq = len(cu) - 1
    S = nseq if cu is not None else b
    y = np.zeros((b, L, H, P), dtype=np.float64)
    fin = np.zeros((S, H, N, P), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _load().ssd_oracle_seq(
        ptr(xf), ptr(df), float(np.float32(d_init)), ptr(Bf), ptr(Cf), ptr(h0),
        ptr(cu), nseq, b, L, H, P, N, G, 1 if reverse else 0, ptr(y), ptr(fin))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_seq failed: {rc}")
    return y, fin


def ssd_ref_bwd_c(x, d_raw, d_init, B, C, dy, init_state=None, d_final=None,
                  cu_seqlens=None, reverse=False, want=("dx", "dd_raw", "dB", "dC",
                                                         "dinit_state", "dd_init"),
                  col_block=16):
    """Same contract as ``ssd_oracle_bwd.ssd_ref_bwd``; runs the C adjoint
    oracle.  ``want`` names the gradients to compute (others are absent from
    the result); ``col_block`` is the headdim columns per parallel unit (a
    work split only: the result does not depend on it beyond rounding)."""
    xf, df, Bf, Cf, gf = _f32(x), _f32(d_raw), _f32(B), _f32(C), _f32(dy)
    h0, dfin = _f32(init_state), _f32(d_final)
    b, L, H, P = xf.shape
    G, N = Bf.shape[2], Bf.shape[3]
    cu = None
    nseq = 0
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        nseq = len(cu) - 1
    S = nseq if cu is not None else b
    shapes = {"dx": (b, L, H, P), "dd_raw": (b, L, H), "dB": (b, L, G, N), "dC": (b, L, G, N),
              "dinit_state": (S, H, N, P), "dd_init": (1,)}
    out = {k: np.zeros(shapes[k], dtype=np.float64) for k in want}
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _load().ssd_oracle_bwd(
        ptr(xf), ptr(df), float(np.float32(d_init)), ptr(Bf), ptr(Cf), ptr(h0), ptr(gf),
        ptr(dfin), ptr(cu), nseq, b, L, H, P, N, G, 1 if reverse else 0, int(col_block),
        *(ptr(out.get(k)) for k in ("dx", "dd_raw", "dB", "dC", "dinit_state", "dd_init")))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_bwd failed: {rc}")
    if "dd_init" in out:
        out["dd_init"] = float(out["dd_init"][0])
    return out
