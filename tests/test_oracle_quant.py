"""Pins for oracle.quant: FitMinMax (Eq. 4), Drift (Eqs. 5-6, Algorithm 1)
and the least-squares Refit (Algorithm 1) of [D-Quant]."""

import itertools
import math

import numpy as np
import pytest

import oracle as O
from oracle.model import budget_fx


def _rates(f):
    return O.rate_table(np.asarray(f))


def test_fit_minmax_closed_form():
    x = np.array([[0.5, -1.25, 3.0, 2.0]], np.float32)
    s, o = O.fit_minmax(x, 8)
    assert o[0] == np.float32(-1.25)
    assert s[0] == np.float32(np.float32(4.25) / np.float32(7))


def _brute_force_frontier(Dim, r_fx):
    """All M^n assignments -> (total rate, total distortion in float64)."""
    n, M = Dim.shape
    out = []
    for a in itertools.product(range(M), repeat=n):
        a = np.array(a)
        out.append((int(r_fx[a].sum()), float(Dim[np.arange(n), a].astype(np.float64).sum())))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_drift_is_everett_optimal(seed):
    """Everett: the Lagrangian minimiser at any lambda has the least distortion
    among all assignments whose rate is not larger than its own."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 9))
    M = int(rng.integers(2, 5)) if n <= 7 else 3
    x = rng.standard_normal((1, n)).astype(np.float32)
    f = O.integer_table(O.sharpen(rng.dirichlet(np.ones(M)), 1.0))
    r = _rates(f)
    s, o = O.fit_minmax(x, M)
    lev = np.arange(M, dtype=np.float32)
    rec = o[0] + s[0] * lev
    Dim = (x[0][:, None] - rec[None, :]) ** 2
    frontier = _brute_force_frontier(Dim, r)
    rmin, rmax = n * int(r.min()), max(R for R, _ in frontier)
    # a budget strictly inside the feasible range so that drift must trade
    B = int(rmin + (rmax - rmin) * rng.uniform(0.1, 0.6))
    m, fb = O.drift(x, s, o, r, B, O.lambda_table())
    assert not fb[0]
    R = int(r[m[0]].sum())
    Dm = float(Dim[np.arange(n), m[0]].astype(np.float64).sum())
    assert R <= B
    tol = n * 2.0 ** -20 * float(Dim.max() + 16 * (Dim.max() - Dim.min()) * 8)
    best = min(D for Rr, D in frontier if Rr <= R)
    assert Dm <= best + tol


def test_drift_trace_has_twelve_bisection_steps():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 1024)).astype(np.float32)
    f, c = O.build_table(6, 1024, 1.4)
    r = _rates(f)
    s, o = O.fit_minmax(x, 6)
    tr = []
    O.drift(x, s, o, r, budget_fx(231), O.lambda_table(), trace=tr)
    mids = np.array(tr[:12])
    assert len(tr) in (12, 13)
    # lambda grid in 1/512 octaves; successive steps halve a 40-octave bracket
    steps = np.abs(np.diff(mids, axis=0))
    for k in range(11):
        assert np.all(steps[k] == 40 * 512 // 2 ** (k + 2))


def test_drift_feasible_and_monotone():
    rng = np.random.default_rng(10)
    E = O.lambda_table()
    for M, C, dist in [(8, 331, "normal"), (6, 231, "normal"), (6, 203, "t"), (8, 292, "t")]:
        f, c = O.build_table(M, 1024, 1.4)
        r = _rates(f)
        if dist == "normal":
            x = rng.standard_normal((64, 1024))
        else:
            x = rng.standard_t(4, (64, 1024))
            x[:, 5] = 40.0
        x = x.astype(np.float32)
        s, o = O.fit_minmax(x, M)
        m, fb = O.drift(x, s, o, r, budget_fx(C), E)
        assert np.all(r[m].sum(axis=1) <= budget_fx(C))
        for i in range(8):
            order = np.argsort(x[i], kind="stable")
            ms = m[i][order]
            viol = np.nonzero(np.diff(ms) < 0)[0]
            # only near-ties of the float32 objective may break monotonicity
            for v in viol:
                a, b = x[i][order[v]], x[i][order[v + 1]]
                assert abs(float(a) - float(b)) <= 4 * np.spacing(np.float32(max(abs(a), abs(b))))


def test_drift_generous_budget_is_nearest_rounding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 1024)).astype(np.float32)
    f, c = O.build_table(8, 1024, 1.4)
    r = _rates(f)
    s, o = O.fit_minmax(x, 8)
    m, fb = O.drift(x, s, o, r, budget_fx(4096), O.lambda_table())
    near = O.nearest_levels(x, s, o, 8)
    assert np.array_equal(m, near)


def test_drift_degenerate_and_ties():
    E = O.lambda_table()
    f, c = O.build_table(6, 128, 1.4)
    r = _rates(f)
    x = np.full((2, 128), 0.75, np.float32)
    s, o = O.fit_minmax(x, 6)
    m, fb = O.drift(x, s, o, r, budget_fx(36), E)
    assert np.all(m == int(np.argmin(r))) and not fb.any()
    # exact tie between levels 0 and 1 with equal rates -> lowest index
    x = np.array([[0.0, 1.0, 0.5, 0.5]], np.float32)
    r2 = np.array([1 << 16, 1 << 16])
    m, fb = O.drift(x, np.array([1.0], np.float32), np.array([0.0], np.float32),
                    r2, budget_fx(100), E)
    assert m[0].tolist() == [0, 1, 0, 0]


def test_drift_fallback_when_hi_is_infeasible():
    """With rates differing by less than 1/8 bit the assignment at 2^hi may
    still exceed the budget; the encoder then uses the cheapest level."""
    E = O.lambda_table()
    r = np.array([65536 + 1000, 65536])             # 1.015 and 1.0 bits
    x = np.array([[0.0] * 60 + [1.0] * 4], np.float32)
    s = np.array([1.0], np.float32)
    o = np.array([0.0], np.float32)
    m, fb = O.drift(x, s, o, r, 64 * 65536, E)      # only all-level-1 fits
    assert fb[0] and np.all(m == 1)


def test_lane_sum_matches_exact_sum():
    rng = np.random.default_rng(12)
    v = rng.standard_normal((20, 1024)) * 1e3
    got = O.lane_sum_f64(v)
    for i in range(20):
        exact = math.fsum(v[i])
        assert abs(got[i] - exact) <= 1024 * 2.0 ** -53 * np.abs(v[i]).sum()
    ints = rng.integers(-1000, 1000, (3, 1000)).astype(np.float64)
    assert np.array_equal(O.lane_sum_f64(ints), ints.sum(axis=1))


def test_refit_matches_lstsq():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((30, 1024)).astype(np.float32)
    f, c = O.build_table(8, 1024, 1.4)
    s, o = O.fit_minmax(x, 8)
    m, _ = O.drift(x, s, o, _rates(f), budget_fx(331), O.lambda_table())
    s1, o1 = O.refit_f64(x, m, s, o)
    for i in range(30):
        A = np.stack([np.ones(1024), m[i].astype(np.float64)], axis=1)
        (oo, ss), *_ = np.linalg.lstsq(A, x[i].astype(np.float64), rcond=None)
        assert abs(s1[i] - ss) <= 1e-12 * abs(ss) + 1e-13
        assert abs(o1[i] - oo) <= 1e-12 * abs(oo) + 1e-13
    s16, o16 = O.refit(x, m, s, o)
    assert np.array_equal(s16, s1.astype(np.float32).astype(np.float16))
    assert np.array_equal(o16, o1.astype(np.float32).astype(np.float16))


def test_refit_exact_recovery_flat_and_guard():
    rng = np.random.default_rng(14)
    m = rng.integers(0, 8, (1, 256))
    x = (np.float32(-1.5) + np.float32(0.25) * m.astype(np.float32)).astype(np.float32)
    s1, o1 = O.refit_f64(x, m, np.array([9.0], np.float32), np.array([9.0], np.float32))
    assert s1[0] == 0.25 and o1[0] == -1.5
    # all symbols equal: slope kept, offset fitted
    m = np.full((1, 64), 3)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    s1, o1 = O.refit_f64(x, m, np.array([0.5], np.float32), np.array([0.0], np.float32))
    assert s1[0] == 0.5
    assert abs(o1[0] - (x.astype(np.float64).mean() - 1.5)) < 1e-12
    # a decreasing fit is rejected
    m = np.arange(8)[None, :]
    x = -np.arange(8, dtype=np.float32)[None, :]
    s1, o1 = O.refit_f64(x, m, np.array([0.125], np.float32), np.array([-7.0], np.float32))
    assert s1[0] == 0.125 and o1[0] == -7.0
