"""fp64 CPU oracle for the backward pass of the SSD scan (test infrastructure
only: ``tests/`` may import it, the HIP library never does and shares no code
with it).

The pages name the backward pass without writing it out: [MindSpeed-CP] §三.2
(Mamba context parallelism reduce-scatters the gradients of the shard
pairs) and [M2-LaCT] §2 (training with fast-weight gradients).  Its plain
definition is the gradient of the forward map of [M2-LaCT] §1.1 with respect
to every input, for a loss whose gradients with respect to the outputs are
given:

    L = sum_t <dy_t, y_t> + <d_final, H_T>     (per sequence and head)

``scan_core_bwd`` runs the adjoint of the recurrence token by token, from the
last token back to the first (reverse-mode differentiation written out by
hand).  With G_t = dL/dH_t (everything downstream of H_t):

    G_t      = C_t^T dy_t + exp(-d_{t+1}) G_{t+1},   G_T = C_T^T dy_T + d_final
    dX_t     = d_t * B_t G_t                      (sum over the state rows)
    dB_t     = d_t * G_t X_t^T                    (sum over headdim)
    dC_t     = H_t dy_t
    dd_t     = < G_t, -exp(-d_t) H_{t-1} + B_t^T X_t >
    dH_0     = exp(-d_1) G_1
    d d_raw  = dd * sigmoid(d_raw + d_init)   (softplus' = sigmoid)
    d d_init = sum over every token and head of d d_raw

B and C gradients are summed over the heads of their group.  Pinned in
``tests/test_oracle_pins.py`` by central finite differences of the forward
oracle (``ssd_ref_seq``), which shares nothing with this derivation, and by
planted mistakes that those pins must catch.
"""
from __future__ import annotations

import numpy as np

from . import ssd_oracle as F


def sigmoid(z: np.ndarray) -> np.ndarray:
    """The derivative of softplus, evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def scan_core_bwd(d: np.ndarray, X: np.ndarray, B: np.ndarray, C: np.ndarray,
                  H0: np.ndarray | None, dy: np.ndarray, dfinal: np.ndarray | None):
    """Adjoint of the recurrence over one sequence, all heads at once.

    d [L, H] step sizes, X/dy [L, H, P], B/C [L, H, N] (per head), H0 and
    dfinal [H, N, P] or None (zeros).  Returns dX [L, H, P], dB and dC
    [L, H, N] (per head), dd [L, H] and dH0 [H, N, P].
    """
    L, Hh, P = X.shape
    N = B.shape[2]
    # forward states H_0 .. H_L (H_0 the initial state)
    Hst = np.zeros((L + 1, Hh, N, P))
    if H0 is not None:
        Hst[0] = H0
    for t in range(L):
        Hst[t + 1] = np.exp(-d[t])[:, None, None] * Hst[t] \
            + d[t][:, None, None] * (B[t][:, :, None] * X[t][:, None, :])
    dX = np.zeros_like(X)
    dB = np.zeros((L, Hh, N))
    dC = np.zeros((L, Hh, N))
    dd = np.zeros((L, Hh))
    Gnext = np.zeros((Hh, N, P)) if dfinal is None else np.array(dfinal, dtype=np.float64)
    for t in range(L - 1, -1, -1):
        G = C[t][:, :, None] * dy[t][:, None, :] + Gnext          # dL/dH_t
        Ht, Hprev = Hst[t + 1], Hst[t]
        dC[t] = np.einsum("hnp,hp->hn", Ht, dy[t])
        BG = np.einsum("hn,hnp->hp", B[t], G)                    # B_t G_t
        dX[t] = d[t][:, None] * BG
        dB[t] = d[t][:, None] * np.einsum("hnp,hp->hn", G, X[t])
        outer = B[t][:, :, None] * X[t][:, None, :]
        dd[t] = np.einsum("hnp,hnp->h", G, -np.exp(-d[t])[:, None, None] * Hprev + outer)
        Gnext = np.exp(-d[t])[:, None, None] * G
    return dX, dB, dC, dd, Gnext


def _sum_groups(g_heads: np.ndarray, G: int) -> np.ndarray:
    """[L, H, N] per-head gradients -> [L, G, N]: head h feeds group h*G//H."""
    L, H, N = g_heads.shape
    out = np.zeros((L, G, N))
    for h in range(H):
        out[:, (h * G) // H] += g_heads[:, h]
    return out


def ssd_ref_bwd(x, d_raw, d_init, B, C, dy, init_state=None, d_final=None,
                cu_seqlens=None, reverse=False):
    """Gradients of the forward oracle's outputs, fp64.

    Arguments as ``ssd_oracle.ssd_ref_seq`` plus dy [b, L, H, P] (dL/dy) and
    d_final [S, H, N, P] or None (dL/d final_state).  Returns a dict with
    dx [b,L,H,P], dd_raw [b,L,H], dd_init (float), dB and dC [b,L,G,N] and
    dinit_state [S,H,N,P] (the gradient of the initial state, also when
    none was given: the gradient at a zero initial state).
    """
    x, d_raw, B, C, dy = (F.as_f64(t) for t in (x, d_raw, B, C, dy))
    H0 = F.as_f64(init_state)
    dF = F.as_f64(d_final)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    cu = None if cu_seqlens is None else np.asarray(F.as_f64(cu_seqlens), np.int64)
    segs = F._segments(L, b, cu)
    d = F.delta(d_raw, d_init)
    z = np.asarray(d_raw, np.float64) + np.float64(np.float32(d_init))
    out = {"dx": np.zeros_like(x), "dd_raw": np.zeros((b, L, H)),
           "dB": np.zeros((b, L, G, N)), "dC": np.zeros((b, L, G, N)),
           "dinit_state": np.zeros((len(segs), H, N, P))}
    for i, (row, s0, n) in enumerate(segs):
        sl = slice(s0, s0 + n)
        Xs, ds, dys = x[row, sl], d[row, sl], dy[row, sl]
        Bs, Cs = F._expand_groups(B[row, sl], H), F._expand_groups(C[row, sl], H)
        if reverse:
            Xs, ds, dys, Bs, Cs = Xs[::-1], ds[::-1], dys[::-1], Bs[::-1], Cs[::-1]
        h0 = None if H0 is None else H0[i]
        df = None if dF is None else dF[i]
        dX, dBh, dCh, dd, dH0 = scan_core_bwd(ds, Xs, Bs, Cs, h0, dys, df)
        if reverse:
            dX, dBh, dCh, dd = dX[::-1], dBh[::-1], dCh[::-1], dd[::-1]
        out["dx"][row, sl] = dX
        out["dB"][row, sl] += _sum_groups(dBh, G)
        out["dC"][row, sl] += _sum_groups(dCh, G)
        out["dd_raw"][row, sl] = dd * sigmoid(z[row, sl])
        out["dinit_state"][i] = dH0
    # every token of every row belongs to one segment (cu_seqlens covers [0, L])
    out["dd_init"] = float(out["dd_raw"].sum())
    return out
