"""Pins for the fp64 backward oracle (CPU).

The backward oracle is the hand-written adjoint of the recurrence.  It is
checked here against central finite differences of the *forward* oracle,
which shares no code or derivation with it: for a fixed random dy and
d_final, each input entry is moved by +-eps and the change of
L = <dy, y> + <d_final, final_state> is compared with the oracle's gradient.
Planted mistakes in a copy of the adjoint (a decay taken one token early, a
dropped term, the state read before the update, a missing step weight) must
each fail that comparison.
"""
import numpy as np
import pytest

from oracle import ssd_oracle as F
from oracle import ssd_oracle_bwd as O
from ssd_inputs import random_problem

EPS = 1e-6
FD_TOL = 1e-6


def _loss(p, dy, dfin, cu=None, reverse=False):
    y, f = F.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"],
                         cu_seqlens=cu, reverse=reverse)
    return float((y * dy).sum() + (f * dfin).sum())


def _fd_grad(p, key, dy, dfin, cu=None, reverse=False):
    """Central differences of the forward oracle's loss w.r.t. p[key]."""
    base = F.as_f64(p[key]).copy()
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        q = dict(p)
        up, dn = base.copy(), base.copy()
        up[idx] += EPS
        dn[idx] -= EPS
        q[key] = up
        lp = _loss(q, dy, dfin, cu, reverse)
        q[key] = dn
        lm = _loss(q, dy, dfin, cu, reverse)
        g[idx] = (lp - lm) / (2 * EPS)
    return g


def _fd_dinit(p, dy, dfin, cu=None, reverse=False):
    # d_init is a float32 scalar in the forward map; perturb it in fp64 by
    # moving d_raw instead (d enters only through d_raw + d_init)
    base = F.as_f64(p["d_raw"]).copy()
    q = dict(p)
    q["d_raw"] = base + EPS
    lp = _loss(q, dy, dfin, cu, reverse)
    q["d_raw"] = base - EPS
    lm = _loss(q, dy, dfin, cu, reverse)
    return (lp - lm) / (2 * EPS)


def _problem(seed, b, L, H, P, N, G, cu=None):
    p = random_problem(seed, b, L, H, P, N, ngroups=G, init_scale=0.5, d_init=-1.0)
    p = {k: (F.as_f64(v) if k not in ("d_init", "cu_seqlens") and v is not None else v)
         for k, v in p.items()}
    rng = np.random.default_rng(seed + 1)
    S = b if cu is None else len(cu) - 1
    if cu is not None:
        p["init_state"] = rng.standard_normal((S, H, N, P)) * 0.5
    dy = rng.standard_normal((b, L, H, P))
    dfin = rng.standard_normal((S, H, N, P))
    return p, dy, dfin


CASES = [
    # (seed, b, L, H, P, N, G, cu, reverse)
    (3, 2, 5, 2, 3, 4, 1, None, False),
    (5, 1, 9, 4, 2, 3, 2, [0, 4, 4, 9], True),
    (7, 1, 7, 2, 2, 2, 1, None, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_bwd_matches_finite_differences(case):
    seed, b, L, H, P, N, G, cu, rev = case
    p, dy, dfin = _problem(seed, b, L, H, P, N, G, cu)
    g = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                      init_state=p["init_state"], d_final=dfin, cu_seqlens=cu, reverse=rev)
    for key, gk in [("x", "dx"), ("d_raw", "dd_raw"), ("B", "dB"), ("C", "dC"),
                    ("init_state", "dinit_state")]:
        fd = _fd_grad(p, key, dy, dfin, cu, rev)
        assert F.rel_err(g[gk], fd) < FD_TOL, key
    assert abs(g["dd_init"] - _fd_dinit(p, dy, dfin, cu, rev)) < FD_TOL * max(1.0, abs(g["dd_init"]))


def test_bwd_without_state_gradients():
    """No initial state and no final-state gradient: the gradients of the
    y-part of the loss alone, and dinit_state is the gradient at H0 = 0."""
    p, dy, dfin = _problem(11, 1, 6, 2, 2, 3, 1)
    p["init_state"] = None
    zero = np.zeros_like(dfin)
    g = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy)
    for key, gk in [("x", "dx"), ("d_raw", "dd_raw"), ("B", "dB"), ("C", "dC")]:
        assert F.rel_err(g[gk], _fd_grad(p, key, dy, zero)) < FD_TOL, key
    # gradient of the initial state at zero: move a zero state entry
    q = dict(p)
    q["init_state"] = np.zeros_like(dfin)
    assert F.rel_err(g["dinit_state"], _fd_grad(q, "init_state", dy, zero)) < FD_TOL


def test_bwd_is_linear_in_output_gradients():
    """Every gradient is linear in (dy, d_final) jointly."""
    p, dy, dfin = _problem(13, 1, 8, 2, 3, 2, 1)
    args = (p["x"], p["d_raw"], p["d_init"], p["B"], p["C"])
    g1 = O.ssd_ref_bwd(*args, dy, init_state=p["init_state"], d_final=dfin)
    g2 = O.ssd_ref_bwd(*args, 2.0 * dy, init_state=p["init_state"], d_final=2.0 * dfin)
    for k in ("dx", "dd_raw", "dB", "dC", "dinit_state"):
        assert F.rel_err(g2[k], 2.0 * g1[k]) < 1e-12


# ---------------------------------------------------------- planted mistakes
def _mutant_bwd(kind):
    def core(d, X, B, C, H0, dy, dfinal):
        L, Hh, P = X.shape
        N = B.shape[2]
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
        Gnext = np.zeros((Hh, N, P)) if dfinal is None else np.array(dfinal)
        for t in range(L - 1, -1, -1):
            G = C[t][:, :, None] * dy[t][:, None, :] + Gnext
            if kind == "early_decay":
                G = np.exp(-d[t])[:, None, None] * G
            Ht = Hst[t] if kind == "state_before_update" else Hst[t + 1]
            dC[t] = np.einsum("hnp,hp->hn", Ht, dy[t])
            w = np.ones_like(d[t]) if kind == "no_step_weight" else d[t]
            dX[t] = w[:, None] * np.einsum("hn,hnp->hp", B[t], G)
            dB[t] = d[t][:, None] * np.einsum("hnp,hp->hn", G, X[t])
            outer = B[t][:, :, None] * X[t][:, None, :]
            decay_term = 0.0 if kind == "drop_decay_term" else -np.exp(-d[t])[:, None, None] * Hst[t]
            dd[t] = np.einsum("hnp,hnp->h", G, decay_term + outer)
            Gnext = (G if kind == "early_decay" else np.exp(-d[t])[:, None, None] * G)
        return dX, dB, dC, dd, Gnext
    return core


@pytest.mark.parametrize("kind", ["early_decay", "state_before_update", "no_step_weight",
                                  "drop_decay_term"])
def test_planted_bwd_mistakes_are_caught(kind, monkeypatch):
    p, dy, dfin = _problem(17, 1, 6, 2, 2, 3, 1)
    monkeypatch.setattr(O, "scan_core_bwd", _mutant_bwd(kind))
    g = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                      init_state=p["init_state"], d_final=dfin)
    worst = 0.0
    for key, gk in [("x", "dx"), ("d_raw", "dd_raw"), ("B", "dB"), ("C", "dC"),
                    ("init_state", "dinit_state")]:
        worst = max(worst, F.rel_err(g[gk], _fd_grad(p, key, dy, dfin)))
    assert worst > 1e-3


# ---------------------------------------------------------- the C adjoint oracle
def _f32_problem(p, dy, dfin):
    """Round every input to float32 (what the C oracle reads) so both
    oracles see the same values."""
    r = lambda a: None if a is None else np.asarray(a, np.float32).astype(np.float64)
    q = {k: (r(v) if k not in ("d_init", "cu_seqlens") else v) for k, v in p.items()}
    return q, r(dy), r(dfin)


def _c_vs_numpy(p, dy, dfin, cu, rev, col_block):
    from oracle import cref
    g = O.ssd_ref_bwd(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                      init_state=p["init_state"], d_final=dfin, cu_seqlens=cu, reverse=rev)
    c = cref.ssd_ref_bwd_c(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], dy,
                           init_state=p["init_state"], d_final=dfin, cu_seqlens=cu,
                           reverse=rev, col_block=col_block)
    for k in ("dx", "dd_raw", "dB", "dC", "dinit_state"):
        assert F.rel_err(c[k], g[k]) <= 1e-12, k
    assert abs(c["dd_init"] - g["dd_init"]) <= 1e-12 * max(1.0, float(np.abs(g["dd_raw"]).sum()))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
@pytest.mark.parametrize("col_block", [1, 2, 64])
def test_c_bwd_matches_numpy_on_fd_cases(case, col_block):
    """The C adjoint oracle equals the finite-difference-pinned numpy one
    (to rounding) on the same cases, whatever its column split."""
    seed, b, L, H, P, N, G, cu, rev = case
    p, dy, dfin = _f32_problem(*_problem(seed, b, L, H, P, N, G, cu))
    _c_vs_numpy(p, dy, dfin, cu, rev, col_block)


@pytest.mark.parametrize("rev", [False, True])
def test_c_bwd_long_walks_and_ragged_blocks(rev):
    """Segments of several checkpoints (the walk recomputes states from
    them), a ragged last column block, two B/C groups, and packed sequences
    including an empty one and a one-token one."""
    lens = [300, 0, 1, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    p, dy, dfin = _f32_problem(*_problem(19, 1, int(cu[-1]), 4, 5, 3, 2, cu))
    _c_vs_numpy(p, dy, dfin, cu, rev, col_block=2)
    q, dq, fq = _f32_problem(*_problem(23, 2, 260, 2, 3, 4, 1))
    _c_vs_numpy(q, dq, fq, None, rev, col_block=1)
    q["init_state"] = None
    _c_vs_numpy(q, dq, None, None, rev, col_block=3)
