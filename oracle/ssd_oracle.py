"""fp64 CPU oracle for the Mamba-2 SSD scan (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.

Sources (the pages the method is taken from):

* [M2-LaCT] "Mamba-2架构与LaCT并行计算技术解析" (jsqmd.com).
  §1.1 gives the per-head recurrence: d = softplus(d_raw + d_init),
  H_t = exp(-d_t) H_{t-1} + d_t B_t^T X_t, y_t = C_t H_t, with d_init = -4.6
  mapping to d ~ 0.01 and a zero (or carried-over) initial state.
  §1.2: heads are independent, each with its own state.
  §3.1: the bidirectional mode runs the same scan on the time-flipped input.
* [LongMamba] "长序列 Mamba 多卡训练，算力和显存怎么同时省" (qwbw.cn).
  §一: the sequence transfer matrix is semiseparable -- diagonal blocks
  inside a chunk, low-rank blocks between chunks, only a small state
  crossing chunk borders.  §三: chunk_size and cu_seqlens packing.
* [MindSpeed-CP] "揭秘MindSpeed-LLM多潜在注意力（MLA）与Mamba上下文并行实现原理"
  (gtnt.cn), §三.2: per-shard (local_decay, local_state) pairs combined
  across shards.

What is here:

* ``softplus``            -- numerically stable softplus in fp64.
* ``scan_core``           -- the plain sequential recurrence with a generic
  per-step (log-decay a_t, input weight w_t); the method uses a = -d, w = d.
* ``ssd_ref_seq``         -- THE oracle: the recurrence of [M2-LaCT] §1.1,
  per sequence and head, in token order (reverse order when ``reverse``).
* ``ssd_ref_quadratic``   -- the semiseparable matrix of [LongMamba] §一
  written out element by element (independent pin, tiny sizes only).
* ``ssd_ref_chunked``     -- the chunked decomposition (diagonal blocks +
  (decay, state) pairs passed between chunks), any chunk length, fp64.
* ``combine_pairs``       -- the associative combine of two (decay, state)
  pairs used to pass state between chunks or shards ([MindSpeed-CP] §三.2).
* ``rel_err``             -- max|a-b| / max|b|, the parity metric.

Readings where the pages are silent:
d_init is added before softplus; softplus uses the stable form with no
threshold; decay is exp(-d) (no separate learned A, no D skip, no gate);
y_t reads the state *after* token t's update; B_t^T X_t is the outer product
(N x P) so H is d_state x headdim; head h uses group h*G//H; d_init is one
float32 scalar upcast to fp64; each cu_seqlens sequence starts from its own
initial state; reverse runs the recurrence from the last token to the first
and writes y at the token's own position.

Parity unpinned: none of the functions here -- every one is checked in
tests/test_oracle_pins.py against closed forms, brute force, a library
filter or a page-printed value.
"""
from __future__ import annotations

import numpy as np


def as_f64(t) -> np.ndarray:
    """torch tensor / numpy array -> float64 numpy (exact for bf16/fp32)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if t.dtype.is_floating_point:
            t = t.double()
        return t.numpy()
    return np.asarray(t, dtype=np.float64)


def softplus(z: np.ndarray) -> np.ndarray:
    """softplus(z) = log(1 + e^z), evaluated as max(z,0) + log1p(e^-|z|)."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def delta(d_raw: np.ndarray, d_init: float) -> np.ndarray:
    """[M2-LaCT] §1.1: the step size is softplus of the raw projection plus
    the bias d_init (d_init is one float32 scalar)."""
    return softplus(np.asarray(d_raw, np.float64) + np.float64(np.float32(d_init)))


def scan_core(a: np.ndarray, w: np.ndarray, X: np.ndarray, B: np.ndarray,
              C: np.ndarray, H0: np.ndarray | None):
    """Sequential first-order recurrence over one sequence, all heads at once.

    a, w : [L, H]      per-token log-decay and input weight
    X    : [L, H, P]
    B, C : [L, H, N]   already expanded from groups to heads
    H0   : [H, N, P] or None (zeros)
    Returns y [L, H, P] and the state after the last token [H, N, P].

    Step t:  H <- exp(a_t) * H + w_t * outer(B_t, X_t);   y_t = C_t . H
    """
    L, Hh, P = X.shape
    N = B.shape[2]
    Hs = np.zeros((Hh, N, P)) if H0 is None else np.array(H0, dtype=np.float64)
    y = np.zeros((L, Hh, P))
    for t in range(L):
        Hs = np.exp(a[t])[:, None, None] * Hs \
            + w[t][:, None, None] * (B[t][:, :, None] * X[t][:, None, :])
        y[t] = np.einsum("hn,hnp->hp", C[t], Hs)
    return y, Hs


def _segments(L_row: int, batch: int, cu):
    """List of (batch row, start, length) for every independent sequence."""
    if cu is None:
        return [(i, 0, L_row) for i in range(batch)]
    cu = np.asarray(cu, dtype=np.int64)
    return [(0, int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]


def _expand_groups(Bg: np.ndarray, H: int) -> np.ndarray:
    """[L, G, N] -> [L, H, N]; head h reads group h*G//H."""
    G = Bg.shape[1]
    idx = (np.arange(H) * G) // H
    return Bg[:, idx, :]


def ssd_ref_seq(x, d_raw, d_init, B, C, init_state=None, cu_seqlens=None,
                reverse=False):
    """The oracle: Mamba-2 SSD forward by the plain recurrence, fp64.

    x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N] (any float dtype, upcast
    exactly), d_init float, init_state [S,H,N,P] or None, cu_seqlens [S+1]
    (requires b == 1) or None, reverse: process each sequence from its last
    token to its first ([M2-LaCT] §3.1 runs the scan on the flipped input;
    y is written back at each token's own position).
    Returns y [b,L,H,P] float64 and final_state [S,H,N,P] float64.
    """
    x, d_raw, B, C = as_f64(x), as_f64(d_raw), as_f64(B), as_f64(C)
    H0 = as_f64(init_state)
    b, L, H, P = x.shape
    N = B.shape[3]
    cu = None if cu_seqlens is None else np.asarray(as_f64(cu_seqlens), np.int64)
    segs = _segments(L, b, cu)
    d = delta(d_raw, d_init)
    y = np.zeros_like(x)
    final = np.zeros((len(segs), H, N, P))
    for i, (row, s0, n) in enumerate(segs):
        sl = slice(s0, s0 + n)
        Xs, ds = x[row, sl], d[row, sl]
        Bs, Cs = _expand_groups(B[row, sl], H), _expand_groups(C[row, sl], H)
        h0 = None if H0 is None else H0[i]
        if reverse:
            Xs, ds, Bs, Cs = Xs[::-1], ds[::-1], Bs[::-1], Cs[::-1]
        ys, hN = scan_core(-ds, ds, Xs, Bs, Cs, h0)
        if reverse:
            ys = ys[::-1]
        y[row, sl] = ys
        final[i] = hN
    return y, final


def ssd_ref_quadratic(x, d_raw, d_init, B, C, init_state=None):
    """Independent pin: the sequence map as one semiseparable matrix.

    For one sequence (b rows treated separately, forward order):
      y_t = sum_{s<=t} M_ts X_s + exp(-sum_{r<=t} d_r) C_t H0,
      M_ts = (C_t . B_s) * exp(-sum_{r=s+1..t} d_r) * d_s,
    and the final state is
      H_L = exp(-sum_r d_r) H0 + sum_s exp(-sum_{r=s+1..L-1} d_r) d_s B_s^T X_s.
    Segment sums are taken directly over the slice (O(L^3), tiny L only).
    """
    x, d_raw, B, C = as_f64(x), as_f64(d_raw), as_f64(B), as_f64(C)
    H0 = as_f64(init_state)
    b, L, H, P = x.shape
    N = B.shape[3]
    d = delta(d_raw, d_init)
    y = np.zeros_like(x)
    final = np.zeros((b, H, N, P))
    for row in range(b):
        Bh = _expand_groups(B[row], H)
        Ch = _expand_groups(C[row], H)
        for h in range(H):
            dh = d[row, :, h]
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    seg = dh[s + 1:t + 1].sum()
                    M[t, s] = (Ch[t, h] @ Bh[s, h]) * np.exp(-seg) * dh[s]
            y[row, :, h] = M @ x[row, :, h]
            if H0 is not None:
                for t in range(L):
                    y[row, t, h] += np.exp(-dh[:t + 1].sum()) * (Ch[t, h] @ H0[row, h])
            Hf = np.zeros((N, P))
            if H0 is not None:
                Hf += np.exp(-dh.sum()) * H0[row, h]
            for s in range(L):
                Hf += np.exp(-dh[s + 1:].sum()) * dh[s] * np.outer(Bh[s, h], x[row, s, h])
            final[row, h] = Hf
    return y, final


def combine_pairs(first, second):
    """Associative combine of two (decay, state) pairs, first then second.

    A segment maps an incoming state H to decay * H + state.  Applying
    segment 1 and then segment 2 gives decay2*decay1 * H + (decay2*state1 +
    state2) -- the pair algebra used to pass state across chunks and, in
    [MindSpeed-CP] §三.2, across sequence shards.
    """
    a1, s1 = first
    a2, s2 = second
    a1 = np.asarray(a1)
    a2 = np.asarray(a2)
    return a1 * a2, a2[..., None, None] * s1 + s2


def ssd_ref_chunked(x, d_raw, d_init, B, C, chunk, init_state=None,
                    cu_seqlens=None, reverse=False, return_stages=False):
    """The chunked semiseparable form ([LongMamba] §一), fp64, any chunk.

    Per sequence and chunk k (tokens in processing order, local index q):
      cs_q      = -sum_{j<=q} d_j                       (within the chunk)
      state_k   = sum_s exp(cs_last - cs_s) d_s B_s^T X_s   (chunk-local state)
      decay_k   = exp(cs_last)
      Hprev_k   = state entering chunk k: pairs combined left to right
      y_q       = sum_{s<=q} (C_q.B_s) exp(cs_q - cs_s) d_s X_s
                  + exp(cs_q) C_q Hprev_k
    With ``return_stages`` also returns per-sequence lists of the chunk
    (decay, state) pairs and the Hprev states.
    """
    x, d_raw, B, C = as_f64(x), as_f64(d_raw), as_f64(B), as_f64(C)
    H0 = as_f64(init_state)
    b, L, H, P = x.shape
    N = B.shape[3]
    cu = None if cu_seqlens is None else np.asarray(as_f64(cu_seqlens), np.int64)
    segs = _segments(L, b, cu)
    d = delta(d_raw, d_init)
    y = np.zeros_like(x)
    final = np.zeros((len(segs), H, N, P))
    stages = []
    for i, (row, s0, n) in enumerate(segs):
        sl = slice(s0, s0 + n)
        Xs, ds = x[row, sl], d[row, sl]
        Bs, Cs = _expand_groups(B[row, sl], H), _expand_groups(C[row, sl], H)
        if reverse:
            Xs, ds, Bs, Cs = Xs[::-1], ds[::-1], Bs[::-1], Cs[::-1]
        Hrun = np.zeros((H, N, P)) if H0 is None else H0[i].copy()
        ys = np.zeros((n, H, P))
        pairs, hprevs = [], []
        for k0 in range(0, n, chunk):
            k1 = min(k0 + chunk, n)
            Xc, dc, Bc, Cc = Xs[k0:k1], ds[k0:k1], Bs[k0:k1], Cs[k0:k1]
            cs = -np.cumsum(dc, axis=0)                        # [q, H]
            wst = np.exp(cs[-1][None, :] - cs) * dc            # [q, H]
            state = np.einsum("qh,qhn,qhp->hnp", wst, Bc, Xc)
            dec = np.exp(cs[-1])
            # intra-chunk (diagonal block), causal
            CB = np.einsum("thn,shn->hts", Cc, Bc)
            diff = cs.T[:, :, None] - cs.T[:, None, :]          # [H, t, s]
            q = k1 - k0
            causal = np.tril(np.ones((q, q), dtype=bool))
            Lmat = np.where(causal[None], np.exp(np.where(causal[None], diff, 0.0)), 0.0)
            Lmat = Lmat * dc.T[:, None, :]
            y_in = np.einsum("hts,hts,shp->thp", CB, Lmat, Xc)
            y_off = np.exp(cs)[:, :, None] * np.einsum("thn,hnp->thp", Cc, Hrun)
            ys[k0:k1] = y_in + y_off
            hprevs.append(Hrun.copy())
            pairs.append((dec, state))
            _, Hrun = combine_pairs((np.ones(H), Hrun), (dec, state))
        if reverse:
            ys = ys[::-1]
        y[row, sl] = ys
        final[i] = Hrun
        stages.append({"pairs": pairs, "hprev": hprevs})
    if return_stages:
        return y, final, stages
    return y, final


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (absolute 1e-30 floor when ref is zero)."""
    got = as_f64(got)
    ref = as_f64(ref)
    den = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref))) / den
