"""Seeded synthetic workloads for the SSD chunked scan.

This module only draws random numbers and casts them to the storage dtype.
It holds none of the scan's arithmetic, so both sides of the parity check
(the fp64 oracle under ``oracle/`` and the HIP library) can take their
inputs from it without sharing any of the method.

The five workloads are the shapes the pages use for the Mamba-2 SSD scan:

* ``tiny``    -- 1 x 256 tokens, 2 heads x headdim 16, d_state 16, fp32.
* ``layer``   -- 2 x 2048 tokens, 24 heads x 64, d_state 128, bf16.  The
  width follows the Mamba3 example (d_model 768 expanded x2) on the page
  "长序列 Mamba 多卡训练，算力和显存怎么同时省", section 三.
* ``wide``    -- 1 x 8192 tokens, 80 heads x 64, d_state 128, bf16, with an
  N(0, 0.1) initial state.  d_model 2560 is the mamba-2.8b width from
  section 四 of the same page.
* ``varlen``  -- 16 packed sequences totalling 65536 tokens (cu_seqlens),
  24 heads x 64, d_state 128, d_init -3.0 (the speech row of the
  hyper-parameter table, page "Mamba-2架构与LaCT并行计算技术解析", §3.2).
* ``bidir``   -- 1 x 1,048,576 tokens, 8 heads x 192, d_state 64, run
  forward and reverse (view-synthesis row of the same table, §3.1/§3.2).

Recipe (``make_inputs``, on the host): ``numpy.random.default_rng([seed,
cfg_id])``; draw order X, B, C, d_raw, init_state, lengths; every draw is
standard normal in float32, then rounded to bfloat16 (round to nearest even,
via torch's cast) for the bf16 workloads.  Values handed to the oracle are
exactly the values the GPU reads.

``make_inputs_device`` draws the same distributions with torch's Philox
generator directly on a GPU (seed ``seed * 1000 + cfg_id``).  The 1M-token
workload uses it because drawing 1.6e9 normals on the host takes minutes;
parity checks then copy the sampled slices they need back to the host.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    batch: int
    seqlen: int          # tokens per batch row (total tokens when varlen)
    nheads: int
    headdim: int
    d_state: int
    ngroups: int = 1
    chunk_size: int = 64
    dtype: str = "bf16"  # storage dtype of x, d_raw, B, C and y
    d_init: float = -4.6
    init: str = "zeros"  # "zeros" | "normal0.1"
    nseq: int = 0        # > 0: packed varlen with that many sequences
    bidir: bool = False  # forward + reverse pass, outputs concatenated

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def nstates(self) -> int:
        """Number of independent sequences (rows of init/final state)."""
        return self.nseq if self.nseq else self.batch


WORKLOADS = {
    1: Workload(1, "tiny", 1, 256, 2, 16, 16, dtype="f32"),
    2: Workload(2, "layer", 2, 2048, 24, 64, 128),
    3: Workload(3, "wide", 1, 8192, 80, 64, 128, init="normal0.1"),
    4: Workload(4, "varlen", 1, 65536, 24, 64, 128, d_init=-3.0, nseq=16),
    5: Workload(5, "bidir", 1, 1 << 20, 8, 192, 64, bidir=True),
}


def by_name(name: str) -> Workload:
    for w in WORKLOADS.values():
        if w.name == name:
            return w
    raise KeyError(name)


def varlen_lengths(rng: np.random.Generator, nseq: int, total: int,
                   lo: int = 256, hi: int = 8192) -> np.ndarray:
    """Lengths uniform in [lo, hi], rescaled (floored) to sum to ``total``;
    the rounding remainder goes to the last sequence."""
    raw = rng.integers(lo, hi + 1, nseq).astype(np.int64)
    lens = (raw * total) // raw.sum()
    lens[-1] += total - lens.sum()
    return lens


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """CPU tensors in the storage dtype.

    Keys: x [b,L,H,P], d_raw [b,L,H], B [b,L,G,N], C [b,L,G,N],
    init_state [S,H,N,P] float32 or None, cu_seqlens [nseq+1] int32 or None,
    d_init (python float, representable in float32).
    """
    rng = np.random.default_rng([seed, w.cfg_id])
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.d_state, w.ngroups
    x = rng.standard_normal((b, L, H, P), dtype=np.float32)
    Bm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    Cm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    d_raw = rng.standard_normal((b, L, H), dtype=np.float32)
    init = None
    if w.init == "normal0.1":
        init = torch.from_numpy(
            (0.1 * rng.standard_normal((w.nstates, H, N, P), dtype=np.float32)).astype(np.float32))
    cu = None
    if w.nseq:
        lens = varlen_lengths(rng, w.nseq, w.tokens)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    return {
        "x": _cast(x, w.dtype),
        "d_raw": _cast(d_raw, w.dtype),
        "B": _cast(Bm, w.dtype),
        "C": _cast(Cm, w.dtype),
        "init_state": init,
        "cu_seqlens": cu,
        "d_init": float(np.float32(w.d_init)),
    }


def random_problem(seed: int, batch: int, seqlen: int, nheads: int, headdim: int,
                   d_state: int, ngroups: int = 1, dtype: str = "f32",
                   d_init: float = -4.6, init_scale: float = 0.0,
                   lengths=None, d_raw_scale: float = 1.0) -> dict:
    """A free-form seeded problem for edge-case and property tests.

    ``lengths`` (list of ints) packs that many sequences into one row of
    ``sum(lengths)`` tokens and returns matching cu_seqlens; ``batch`` must
    then be 1 and ``seqlen`` is ignored.
    """
    rng = np.random.default_rng([seed, 1000 + nheads, headdim, d_state])
    if lengths is not None:
        assert batch == 1
        seqlen = int(sum(lengths))
    b, L, H, P, N, G = batch, seqlen, nheads, headdim, d_state, ngroups
    x = rng.standard_normal((b, L, H, P), dtype=np.float32)
    Bm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    Cm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    d_raw = (d_raw_scale * rng.standard_normal((b, L, H), dtype=np.float32)).astype(np.float32)
    S = len(lengths) if lengths is not None else b
    init = None
    if init_scale:
        init = torch.from_numpy(
            (init_scale * rng.standard_normal((S, H, N, P), dtype=np.float32)).astype(np.float32))
    cu = None
    if lengths is not None:
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return {
        "x": _cast(x, dtype),
        "d_raw": _cast(d_raw, dtype),
        "B": _cast(Bm, dtype),
        "C": _cast(Cm, dtype),
        "init_state": init,
        "cu_seqlens": cu,
        "d_init": float(np.float32(d_init)),
    }


def make_inputs_device(w: Workload, device, seed: int = 0) -> dict:
    """Like ``make_inputs`` but drawn on ``device`` with torch's generator
    (different numbers from the host recipe; same shapes and distributions).
    cu_seqlens still come from the host recipe's length generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + w.cfg_id)
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.d_state, w.ngroups
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def draw(shape, scale=1.0):
        t = torch.randn(shape, dtype=torch.float32, device=device, generator=gen)
        if scale != 1.0:
            t.mul_(scale)
        return t

    x = draw((b, L, H, P)).to(dt)
    Bm = draw((b, L, G, N)).to(dt)
    Cm = draw((b, L, G, N)).to(dt)
    d_raw = draw((b, L, H)).to(dt)
    init = draw((w.nstates, H, N, P), 0.1) if w.init == "normal0.1" else None
    cu = None
    if w.nseq:
        rng = np.random.default_rng([seed, w.cfg_id])
        lens = varlen_lengths(rng, w.nseq, w.tokens)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(device)
    return {"x": x, "d_raw": d_raw, "B": Bm, "C": Cm, "init_state": init,
            "cu_seqlens": cu, "d_init": float(np.float32(w.d_init))}
