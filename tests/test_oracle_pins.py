"""Pins for the fp64 oracle, against things other than itself.

Each check below comes from the pages or from mathematics, not from the
oracle's own code: the page-printed softplus value, brute-force evaluation of
the semiseparable matrix, a library IIR filter, closed forms in limits, hand
values, and structural properties (linearity, head independence, packing,
time reversal, resumption).  ``test_planted_mistakes_are_caught`` plants
plausible bugs in a copy of the recurrence and checks that a pin fails.
"""
import math
import os

import numpy as np
import pytest
import scipy.signal

from oracle import ssd_oracle as O
from oracle import cref
from ssd_inputs import WORKLOADS, make_inputs, random_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def _np(p):
    return {k: (O.as_f64(v) if v is not None and k != "d_init" else v) for k, v in p.items()}


# --------------------------------------------------------------- page values
def test_softplus_dinit_printed_value():
    """d_init = -4.6 -> step ~ 0.01 (page-printed, 1 significant digit)."""
    for d_raw, d_init, printed, tol in _golden_rows("softplus_dinit.txt"):
        got = float(O.delta(np.array([d_raw]), d_init)[0])
        assert abs(got - printed) < tol, got


def test_dinit_table_gives_slow_decay():
    for heads, headdim, d_init in _golden_rows("dinit_table.txt"):
        d = float(O.delta(np.array([0.0]), d_init)[0])
        assert 0.0 < d < 0.05
        assert -5.0 <= d_init <= -3.0


def test_softplus_matches_library_logaddexp():
    z = np.linspace(-60, 60, 2001)
    ref = np.logaddexp(0.0, z)
    got = O.softplus(z)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)) < 1e-14


def test_dinit_is_float32_scalar():
    # -4.6 is not representable; the oracle uses the float32 value upcast.
    d = O.delta(np.array([0.0]), -4.6)[0]
    assert d == pytest.approx(math.log1p(math.exp(float(np.float32(-4.6)))), rel=1e-15)


# ------------------------------------------------------- brute-force matrix
@pytest.mark.parametrize("shape", [
    dict(batch=1, seqlen=1, nheads=1, headdim=1, d_state=1),
    dict(batch=2, seqlen=17, nheads=3, headdim=5, d_state=4),
    dict(batch=1, seqlen=40, nheads=4, headdim=3, d_state=6, ngroups=2),
    dict(batch=1, seqlen=64, nheads=2, headdim=16, d_state=16),
])
@pytest.mark.parametrize("init_scale", [0.0, 0.7])
def test_sequential_equals_semiseparable_matrix(shape, init_scale):
    p = random_problem(3, **shape, init_scale=init_scale, d_raw_scale=2.0, d_init=-1.0)
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    yq, fq = O.ssd_ref_quadratic(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    assert O.rel_err(y, yq) < TIGHT
    assert O.rel_err(f, fq) < TIGHT


def test_constant_step_equals_library_iir_filter():
    """With d constant the recurrence per state entry (n, p) is the LTI
    filter H_t = a H_{t-1} + d * B_t[n] X_t[p], a = exp(-d)."""
    rng = np.random.default_rng(7)
    L, P, N = 50, 3, 4
    x = rng.standard_normal((1, L, 1, P))
    B = rng.standard_normal((1, L, 1, N))
    C = rng.standard_normal((1, L, 1, N))
    H0 = rng.standard_normal((1, 1, N, P))
    d_raw = np.full((1, L, 1), 0.3)
    d_init = -1.25
    y, f = O.ssd_ref_seq(x, d_raw, d_init, B, C, H0)
    d = math.log1p(math.exp(0.3 + float(np.float32(d_init))))
    a = math.exp(-d)
    Hs = np.zeros((L, N, P))
    for n in range(N):
        for q in range(P):
            u = B[0, :, 0, n] * x[0, :, 0, q]
            out, _ = scipy.signal.lfilter([d], [1.0, -a], u, zi=[a * H0[0, 0, n, q]])
            Hs[:, n, q] = out
    yref = np.einsum("tn,tnp->tp", C[0, :, 0], Hs)
    assert O.rel_err(y[0, :, 0], yref) < TIGHT
    assert O.rel_err(f[0, 0], Hs[-1]) < TIGHT


# ------------------------------------------------------------ closed forms
def test_hand_value_single_token():
    rng = np.random.default_rng(11)
    P, N = 3, 5
    X = rng.standard_normal((1, 1, 1, P))
    B = rng.standard_normal((1, 1, 1, N))
    C = rng.standard_normal((1, 1, 1, N))
    H0 = rng.standard_normal((1, 1, N, P))
    d_raw = np.array([[[0.4]]])
    y, f = O.ssd_ref_seq(X, d_raw, -4.6, B, C, H0)
    d = math.log1p(math.exp(0.4 + float(np.float32(-4.6))))
    cb = float(C[0, 0, 0] @ B[0, 0, 0])
    yhand = d * cb * X[0, 0, 0] + math.exp(-d) * (C[0, 0, 0] @ H0[0, 0])
    assert O.rel_err(y[0, 0, 0], yhand) < TIGHT
    assert O.rel_err(f[0, 0], math.exp(-d) * H0[0, 0] + d * np.outer(B[0, 0, 0], X[0, 0, 0])) < TIGHT


def test_hand_value_two_tokens_half_decay():
    """z = d_raw + d_init = 0 gives d = ln 2 and decay 1/2, scalar state.
    H1 = H0/2 + ln2*b0*x0;  H2 = H1/2 + ln2*b1*x1;  y_t = c_t * H_t."""
    d_init = -1.5  # exactly representable in float32
    d_raw = np.array([[[1.5], [1.5]]])
    x = np.array([[[[2.0]], [[-3.0]]]])
    B = np.array([[[[0.5]], [[4.0]]]])
    C = np.array([[[[1.0]], [[-2.0]]]])
    H0 = np.array([[[[8.0]]]])
    y, f = O.ssd_ref_seq(x, d_raw, d_init, B, C, H0)
    ln2 = math.log(2.0)
    H1 = 4.0 + ln2 * 1.0
    H2 = H1 / 2 + ln2 * (-12.0)
    assert y[0, 0, 0, 0] == pytest.approx(1.0 * H1, rel=1e-14)
    assert y[0, 1, 0, 0] == pytest.approx(-2.0 * H2, rel=1e-14)
    assert f[0, 0, 0, 0] == pytest.approx(H2, rel=1e-14)


def test_dinit_to_minus_infinity_limit():
    """d -> 0: no input enters the state, so y -> C_t H0 and final -> H0."""
    p = random_problem(5, 1, 96, 3, 8, 6, init_scale=0.0)
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], -60.0, p["B"], p["C"])
    cbx = np.abs(np.einsum("btgn,btgn->bt", O.as_f64(p["C"]), O.as_f64(p["B"]))).max() \
        * np.abs(O.as_f64(p["x"])).max()
    assert np.abs(y).max() <= 1e-20 * cbx
    p = random_problem(5, 1, 96, 3, 8, 6, init_scale=1.0)
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], -60.0, p["B"], p["C"], p["init_state"])
    H0 = O.as_f64(p["init_state"])[0]
    Cm = O.as_f64(p["C"])[0, :, 0]
    yref = np.einsum("tn,hnp->thp", Cm, H0)
    assert O.rel_err(y[0], yref) < 1e-12
    assert O.rel_err(f[0], H0) < 1e-12


def test_all_decay_one_is_cumulative_sum():
    """scan_core with log-decay 0: H_t = H0 + cumsum_s w_s B_s^T X_s."""
    rng = np.random.default_rng(13)
    L, H, P, N = 33, 2, 4, 3
    X = rng.standard_normal((L, H, P))
    B = rng.standard_normal((L, H, N))
    C = rng.standard_normal((L, H, N))
    w = rng.random((L, H))
    H0 = rng.standard_normal((H, N, P))
    y, f = O.scan_core(np.zeros((L, H)), w, X, B, C, H0)
    outer = w[:, :, None, None] * B[:, :, :, None] * X[:, :, None, :]
    Hs = H0[None] + np.cumsum(outer, axis=0)
    yref = np.einsum("thn,thnp->thp", C, Hs)
    assert O.rel_err(y, yref) < TIGHT
    assert O.rel_err(f, Hs[-1]) < TIGHT


# --------------------------------------------------------------- structure
def test_linearity_and_init_superposition():
    p = random_problem(17, 1, 70, 2, 5, 4, init_scale=0.5)
    args = (p["d_raw"], p["d_init"], p["B"], p["C"])
    x1 = O.as_f64(p["x"])
    x2 = np.random.default_rng(1).standard_normal(x1.shape)
    H0 = O.as_f64(p["init_state"])
    y1, f1 = O.ssd_ref_seq(x1, *args)
    y2, f2 = O.ssd_ref_seq(x2, *args)
    y12, f12 = O.ssd_ref_seq(2.5 * x1 - x2, *args)
    assert O.rel_err(y12, 2.5 * y1 - y2) < 1e-12
    assert O.rel_err(f12, 2.5 * f1 - f2) < 1e-12
    yh, fh = O.ssd_ref_seq(np.zeros_like(x1), *args, init_state=H0)
    yb, fb = O.ssd_ref_seq(x1, *args, init_state=H0)
    assert O.rel_err(yb, y1 + yh) < 1e-12
    assert O.rel_err(fb, f1 + fh) < 1e-12


def test_head_permutation_equivariance():
    p = _np(random_problem(19, 2, 30, 5, 4, 3, init_scale=0.3))
    perm = np.array([3, 0, 4, 1, 2])
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    yp, fp = O.ssd_ref_seq(p["x"][:, :, perm], p["d_raw"][:, :, perm], p["d_init"],
                           p["B"], p["C"], p["init_state"][:, perm])
    assert O.rel_err(yp, y[:, :, perm]) < TIGHT
    assert O.rel_err(fp, f[:, perm]) < TIGHT


def test_varlen_packed_equals_separate():
    lens = [1, 63, 64, 65, 130, 7]
    p = _np(random_problem(23, 1, 0, 3, 4, 5, lengths=lens, init_scale=0.4))
    cu = p["cu_seqlens"].astype(np.int64)
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"],
                         p["init_state"], cu_seqlens=cu)
    for i in range(len(lens)):
        sl = slice(cu[i], cu[i + 1])
        yi, fi = O.ssd_ref_seq(p["x"][:, sl], p["d_raw"][:, sl], p["d_init"],
                               p["B"][:, sl], p["C"][:, sl], p["init_state"][i:i + 1])
        assert O.rel_err(y[:, sl], yi) < TIGHT
        assert O.rel_err(f[i], fi[0]) < TIGHT


def test_reverse_equals_flip_forward_flip():
    p = _np(random_problem(29, 2, 45, 2, 3, 4, init_scale=0.2))
    flip = lambda a: a[:, ::-1].copy()
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"],
                         reverse=True)
    yf, ff = O.ssd_ref_seq(flip(p["x"]), flip(p["d_raw"]), p["d_init"], flip(p["B"]),
                           flip(p["C"]), p["init_state"])
    assert O.rel_err(y, flip(yf)) < TIGHT
    assert O.rel_err(f, ff) < TIGHT


def test_chained_halves_equal_one_run():
    p = _np(random_problem(31, 1, 100, 2, 4, 3, init_scale=0.3))
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    a = slice(0, 37)
    b = slice(37, 100)
    ya, fa = O.ssd_ref_seq(p["x"][:, a], p["d_raw"][:, a], p["d_init"], p["B"][:, a],
                           p["C"][:, a], p["init_state"])
    yb, fb = O.ssd_ref_seq(p["x"][:, b], p["d_raw"][:, b], p["d_init"], p["B"][:, b],
                           p["C"][:, b], fa)
    assert O.rel_err(np.concatenate([ya, yb], axis=1), y) < TIGHT
    assert O.rel_err(fb, f) < TIGHT


@pytest.mark.parametrize("chunk", [1, 2, 7, 16, 64, 200])
@pytest.mark.parametrize("reverse", [False, True])
def test_chunked_form_equals_recurrence(chunk, reverse):
    lens = [150, 64, 5, 129]
    p = random_problem(37, 1, 0, 3, 6, 5, ngroups=1, lengths=lens, init_scale=0.3,
                       d_init=-2.0)
    args = (p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"], p["cu_seqlens"])
    y, f = O.ssd_ref_seq(*args, reverse=reverse)
    yc, fc = O.ssd_ref_chunked(*args[:5], chunk, init_state=args[5], cu_seqlens=args[6],
                               reverse=reverse)
    assert O.rel_err(yc, y) < TIGHT
    assert O.rel_err(fc, f) < TIGHT


def test_pair_combine_is_associative_and_shards_compose():
    """Passing state across two shards through combined (decay, state)
    pairs equals one run: the one-device form of context-parallel state
    passing."""
    p = random_problem(41, 1, 256, 2, 4, 3, init_scale=0.0, d_init=-3.0)
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"])
    _, _, st = O.ssd_ref_chunked(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], 64,
                                 return_stages=True)
    pairs = st[0]["pairs"]
    left = O.combine_pairs(pairs[0], pairs[1])
    right = O.combine_pairs(pairs[2], pairs[3])
    tot = O.combine_pairs(left, right)
    seq = pairs[0]
    for q in pairs[1:]:
        seq = O.combine_pairs(seq, q)
    assert O.rel_err(tot[1], seq[1]) < TIGHT
    assert O.rel_err(tot[1], f[0]) < TIGHT


# ------------------------------------------------------------- C oracle
@pytest.mark.parametrize("case", ["tiny", "groups", "varlen_rev", "layer_slice"])
def test_c_oracle_matches_numpy_oracle(case):
    if case == "tiny":
        p = make_inputs(WORKLOADS[1])
        rev = False
    elif case == "groups":
        p = random_problem(43, 2, 80, 4, 6, 5, ngroups=2, init_scale=0.5)
        rev = False
    elif case == "varlen_rev":
        p = random_problem(47, 1, 0, 3, 4, 8, lengths=[5, 70, 1, 33], init_scale=0.5,
                           dtype="bf16")
        rev = True
    else:
        full = make_inputs(WORKLOADS[2])
        p = {k: v for k, v in full.items()}
        p["x"] = full["x"][:, :300, :3]
        p["d_raw"] = full["d_raw"][:, :300, :3]
        p["B"] = full["B"][:, :300]
        p["C"] = full["C"][:, :300]
        rev = False
    args = (p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"], p["cu_seqlens"])
    y, f = O.ssd_ref_seq(*args, reverse=rev)
    yc, fc = cref.ssd_ref_seq_c(*args, reverse=rev)
    assert O.rel_err(yc, y) < TIGHT
    assert O.rel_err(fc, f) < TIGHT


# ---------------------------------------------------------- planted mistakes
def _mutant_scan(kind):
    def core(a, w, X, B, C, H0):
        L, Hh, P = X.shape
        N = B.shape[2]
        Hs = np.zeros((Hh, N, P)) if H0 is None else np.array(H0, dtype=np.float64)
        y = np.zeros((L, Hh, P))
        for t in range(L):
            dec = np.exp(-a[t] if kind == "sign" else a[t])[:, None, None]
            ww = np.ones_like(w[t]) if kind == "no_weight" else w[t]
            Bt, Ct = (C[t], B[t]) if kind == "swap_BC" else (B[t], C[t])
            prev = Hs
            Hs = dec * Hs + ww[:, None, None] * (Bt[:, :, None] * X[t][:, None, :])
            src = prev if kind == "y_before_update" else Hs
            y[t] = np.einsum("hn,hnp->hp", Ct, src)
        return y, Hs
    return core


@pytest.mark.parametrize("kind", ["sign", "no_weight", "swap_BC", "y_before_update"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    p = random_problem(53, 1, 24, 2, 3, 4, init_scale=0.5, d_init=-1.0)
    yq, fq = O.ssd_ref_quadratic(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    monkeypatch.setattr(O, "scan_core", _mutant_scan(kind))
    y, f = O.ssd_ref_seq(p["x"], p["d_raw"], p["d_init"], p["B"], p["C"], p["init_state"])
    assert O.rel_err(y, yq) > 1e-3 or O.rel_err(f, fq) > 1e-3


def test_planted_mistake_dinit_after_softplus(monkeypatch):
    monkeypatch.setattr(O, "delta",
                        lambda d_raw, d_init: O.softplus(np.asarray(d_raw, np.float64)) + d_init)
    for _, d_init, printed, tol in _golden_rows("softplus_dinit.txt"):
        got = float(O.delta(np.array([0.0]), d_init)[0])
        assert not abs(got - printed) < tol
