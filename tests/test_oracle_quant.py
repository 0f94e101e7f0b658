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


# ---------------------------------------------------------------------------
# The drift bracket anchor ([D-Quant] Appendix A, Algorithm 1: the bisection on
# log2 lambda runs between hi = log2(8 (max D - min D)) and hi - 40).  The
# reading fixes hi to the exact ceiling of log2(8 Delta), Delta = RN(max D -
# min D) over the float32 distortion matrix.  These pins recompute Delta and
# the ceiling in exact rational arithmetic, without numpy float32 operations
# or frexp, so an anchor one octave off (a floor, or the frexp exponent taken
# as is) fails them.

from fractions import Fraction


def _rn32(q):
    """Round a rational to the nearest binary32 value (ties to even, with
    subnormals), returned as an exact Fraction."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    ulp = Fraction(2) ** (max(e, -126) - 23)
    m, r = divmod(a, ulp)
    m = int(m)
    if r > ulp / 2 or (r == ulp / 2 and m % 2 == 1):
        m += 1
    assert m * ulp < Fraction(2) ** 128, "overflows binary32"
    return sign * m * ulp


def _f32_exact(v):
    return Fraction(float(np.float32(v)))


def _exact_anchor(x_row, s, o, vals):
    """hi0 = min{h : 2^h >= 8 Delta} with Delta = RN32(max D - min D) and
    D_im = RN32(RN32(x_i - RN32(o + RN32(s v_m)))^2), all in exact rationals.
    Returns None when 8 Delta == 0."""
    s, o = _f32_exact(s), _f32_exact(o)
    rec = [_rn32(o + _rn32(s * Fraction(float(v)))) for v in vals]
    D = []
    for xi in x_row:
        xi = _f32_exact(xi)
        for r in rec:
            dl = _rn32(xi - r)
            D.append(_rn32(dl * dl))
    y = 8 * _rn32(max(D) - min(D))
    if y == 0:
        return None
    h = y.numerator.bit_length() - y.denominator.bit_length() - 1
    while Fraction(2) ** h < y:
        h += 1
    while Fraction(2) ** (h - 1) >= y:
        h -= 1
    return h


@pytest.mark.parametrize("scale", [1.0, 3.0e-3, 7.0e5, 2.0 ** -70])
def test_drift_bracket_anchor_is_exact_ceiling(scale):
    """The first bisection midpoint is (lo + hi) / 2 = 512 hi0 - 10240 on the
    1/512-octave grid, for hi0 recomputed exactly.  The scales include one
    whose distortions are binary32 subnormals (2^-70 squared is below 2^-126)."""
    rng = np.random.default_rng(31)
    M = 4
    n = 6
    x = (rng.standard_normal((5, n)) * scale).astype(np.float32)
    s, o = O.fit_minmax(x, M)
    r = _rates(O.integer_table(O.sharpen(np.array([0.1, 0.4, 0.4, 0.1]), 1.0)))
    tr = []
    O.drift(x, s, o, r, budget_fx(2), O.lambda_table(), trace=tr)
    for i in range(x.shape[0]):
        hi0 = _exact_anchor(x[i], s[i], o[i], range(M))
        assert hi0 is not None
        assert int(tr[0][i]) == 512 * hi0 - 10240, (i, hi0, int(tr[0][i]))
    if scale == 2.0 ** -70:
        assert hi0 < -100


def test_drift_bracket_anchor_at_exact_power_of_two():
    """8 Delta = 8 exactly (x = 0 and 1 on the grid {0, 1}): hi0 = 3, not the
    frexp exponent 4 of 8 = 0.5 * 2^4; and 8 Delta = 18 gives hi0 = 5."""
    r = np.array([65536 + 8192, 65536])
    E = O.lambda_table()
    for xs, hi0 in (([0.0, 1.0], 3), ([0.0, 1.5], 5)):
        x = np.array([xs], np.float32)
        assert _exact_anchor(x[0], 1.0, 0.0, range(2)) == hi0
        tr = []
        O.drift(x, np.array([1.0], np.float32), np.array([0.0], np.float32), r, budget_fx(2), E, trace=tr)
        assert int(tr[0][0]) == 512 * hi0 - 10240


def test_drift_top_of_bracket_takes_the_cheapest_level():
    """The page's bracket top: at lambda = 2^hi >= 8 (max D - min D), any level
    whose rate exceeds the cheapest one's by more than 1/8 bit costs more than
    any distortion it saves, so the assignment at 2^hi is all-cheapest and
    fits the smallest budget without the fallback.  Here 8 Delta = 40 (D = 9
    and 4 for x = 3 on the grid {0, 1}), so the ceiling gives lambda = 64; a
    floor would give 32, where level 0 still wins (-5 + 32 (1/8 + 2^-16) < 0)
    and the encoder would fall back."""
    E = O.lambda_table()
    r = np.array([65536 + 8192 + 1, 65536])         # 1/8 bit + 2^-16 more for level 0
    x = np.full((1, 4), 3.0, np.float32)
    s = np.array([1.0], np.float32)
    o = np.array([0.0], np.float32)
    assert _exact_anchor(x[0], s[0], o[0], range(2)) == 6
    tr = []
    m, fb = O.drift(x, s, o, r, 4 * 65536, E, trace=tr)
    assert not fb[0]
    assert np.all(m == 1)
    assert int(tr[0][0]) == 512 * 6 - 10240


def test_drift_bottom_of_bracket_is_nearest_rounding():
    """At lambda = 2^(hi0 - 40) the rate term is at most 2^-37 Delta times the
    largest rate in bits, so the Lagrangian argmin is nearest-level rounding
    except where two levels' distortions are that close (near-ties)."""
    from oracle.quant import _assign, _distortion
    rng = np.random.default_rng(32)
    E = O.lambda_table()
    for M, C in ((8, 331), (6, 231)):
        f, c = O.build_table(M, 1024, 1.4)
        r = _rates(f)
        x = rng.standard_normal((8, 1024)).astype(np.float32)
        s, o = O.fit_minmax(x, M)
        D = _distortion(x, s, o, M)
        rate_f32 = (r.astype(np.float64) / 65536).astype(np.float32)
        # the first midpoint is hi0 - 20 octaves (pinned exactly above); lo is 20 below it
        tr = []
        O.drift(x, s, o, r, budget_fx(C), E, trace=tr)
        lo_u = np.asarray(tr[0], np.int64) - 10240
        m, _ = _assign(D, rate_f32, r, lo_u, E)
        near = O.nearest_levels(x, s, o, M)
        diff = np.nonzero(m != near)
        lam = np.ldexp(2.0, lo_u // 512)           # >= lambda(lo_u)
        for i, j in zip(*diff):
            gap = abs(float(D[i, j, m[i, j]]) - float(D[i, j, near[i, j]]))
            assert gap <= lam[i] * float(rate_f32.max()) + 4 * float(np.spacing(D[i, j].max())), (i, j)
