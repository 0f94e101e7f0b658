"""Pins for non-affine reconstruction levels in the table ([D-Quant] Appendix A:
a table entry carries the reconstruction level v_m; Eqs. (7)-(9) hold for any
v_m).  Levels are given in grid units with v_0 = 0 and v_{M-1} = M - 1, so
FitMinMax is unchanged; nearest rounding, drift, refit and the model use the
level values."""

import itertools

import numpy as np
import pytest

import oracle as O

SYM6 = (0.0, 0.875, 2.125, 2.875, 4.125, 5.0)        # symmetric, exact in fp16
ASYM5 = (0.0, 0.5, 1.75, 3.25, 4.0)


def test_level_validation_and_rounding():
    assert np.array_equal(O.level_values_fp16(4), [0, 1, 2, 3])
    v = O.level_values_fp16(3, (0.0, 0.3, 2.0))
    assert v[1] == np.float32(np.float16(0.3))
    for bad in ((0.5, 1.0, 2.0), (0.0, 1.0, 1.5), (0.0, 1.5, 1.0, 3.0)):
        with pytest.raises(ValueError):
            O.level_values_fp16(len(bad), bad)


def test_affine_values_reproduce_the_default_exactly():
    p0 = O.order_stat_probs(8, 1024)
    p1 = O.order_stat_probs(8, 1024, values=np.arange(8.0))
    assert np.array_equal(p0, p1)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((128, 256)).astype(np.float32)
    v = rng.standard_normal((128, 256)).astype(np.float32)
    a = O.encode_cache(k, v, O.OracleParams(2, 128, 8, 6, 90, 62, 128, 1.4))
    b = O.encode_cache(k, v, O.OracleParams(2, 128, 8, 6, 90, 62, 128, 1.4,
                                            values_k=tuple(range(8)), values_v=tuple(range(6))))
    for key in ("k_cont", "v_cont", "k_sym", "v_sym"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("values", [SYM6, ASYM5])
def test_model_matches_monte_carlo(values):
    """Expected symbol fractions of min-max normalised Gaussian streams rounded
    to the nearest non-affine level, against a seeded Monte-Carlo histogram."""
    M, n, trials = len(values), 256, 6000
    rng = np.random.default_rng(11)
    x = rng.standard_normal((trials, n))
    u = (x - x.min(1, keepdims=True)) / (x.max(1, keepdims=True) - x.min(1, keepdims=True)) * (M - 1)
    v = np.asarray(values)
    sym = np.argmin(np.abs(u[..., None] - v), axis=-1)
    hist = np.bincount(sym.ravel(), minlength=M) / sym.size
    p = O.order_stat_probs(M, n, values=values)
    se = np.sqrt(p * (1 - p) / (trials * 8))      # generous: values within a stream correlate
    assert np.all(np.abs(hist - p) <= 6 * se + 2e-4)
    assert abs(p.sum() - 1.0) < 1e-12
    if values is SYM6:
        assert np.allclose(p, p[::-1], rtol=0, atol=0)


def test_drift_with_values_is_everett_optimal():
    rng = np.random.default_rng(2)
    for trial in range(8):
        n, M = 6, 4
        vals = np.array((0.0, 0.625, 2.25, 3.0), np.float32)
        x = rng.standard_normal((1, n)).astype(np.float32)
        f = O.integer_table(O.sharpen(rng.dirichlet(np.ones(M)), 1.0))
        r = O.rate_table(f)
        s, o = O.fit_minmax(x, M)
        rec = o[0] + s[0] * vals
        Dim = (x[0][:, None] - rec[None, :]) ** 2
        frontier = []
        for a in itertools.product(range(M), repeat=n):
            a = np.array(a)
            frontier.append((int(r[a].sum()), float(Dim[np.arange(n), a].astype(np.float64).sum())))
        rmin, rmax = n * int(r.min()), max(R for R, _ in frontier)
        B = int(rmin + (rmax - rmin) * 0.4)
        m, fb = O.drift(x, s, o, r, B, O.lambda_table(), vals=vals)
        R = int(r[m[0]].sum())
        Dm = float(Dim[np.arange(n), m[0]].astype(np.float64).sum())
        assert not fb[0] and R <= B
        best = min(D for Rr, D in frontier if Rr <= R)
        assert Dm <= best + 1e-5 * max(1.0, best)


def test_refit_with_values_matches_lstsq():
    rng = np.random.default_rng(4)
    vals = O.level_values_fp16(6, SYM6)
    x = rng.standard_normal((20, 256)).astype(np.float32)
    s, o = O.fit_minmax(x, 6)
    m = O.nearest_levels(x, s, o, 6, vals)
    m = np.where(rng.random(m.shape) < 0.1, np.clip(m + rng.integers(-1, 2, m.shape), 0, 5), m)
    s1, o1 = O.refit_f64(x, m, s, o, vals)
    assert np.all(s1 > 0)
    for i in range(20):
        A = np.stack([np.ones(256), vals.astype(np.float64)[m[i]]], 1)
        (oo, ss), *_ = np.linalg.lstsq(A, x[i].astype(np.float64), rcond=None)
        assert abs(s1[i] - ss) <= 1e-12 * max(1, abs(ss)) and abs(o1[i] - oo) <= 1e-12 * max(1, abs(oo))


def test_factored_attention_with_values_equals_plain():
    rng = np.random.default_rng(9)
    T, Hkv, Hq, d = 40, 2, 4, 32
    n = Hkv * d
    kv = O.level_values_fp16(6, SYM6)
    vv = O.level_values_fp16(5, ASYM5)
    k_sym, v_sym = rng.integers(0, 6, (T, n)), rng.integers(0, 5, (T, n))
    k_so = np.stack([rng.uniform(0.1, 1, T), rng.uniform(-3, 0, T)], 1).astype(np.float16)
    v_so = np.stack([rng.uniform(0.1, 1, T), rng.uniform(-3, 0, T)], 1).astype(np.float16)
    mu = rng.standard_normal((T, n)).astype(np.float32)
    q = rng.standard_normal((Hq, d))
    a = O.attention_plain_f64(q, O.dequantize_f64(k_sym, k_so, mu, kv), O.dequantize_f64(v_sym, v_so, None, vv),
                              Hkv, d)
    b = O.attention_factored_f64(q, k_sym, k_so, mu, v_sym, v_so, Hkv, d, k_vals=kv, v_vals=vv)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
