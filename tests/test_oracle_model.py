"""Pins for oracle.model: the order-statistics model, the integer table, the
rate table and the lambda grid ([D-Quant] §3.1, §4.2, §4.4, Algorithm 1)."""

import numpy as np
import pytest

import oracle as O


def _mc_hist(M, n, streams, seed):
    """Monte-Carlo frequencies of nearest-level symbols of min-max normalised
    N(0,1) streams: the quantity the model claims to compute."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((streams, n))
    mn = x.min(axis=1, keepdims=True)
    mx = x.max(axis=1, keepdims=True)
    lev = np.rint((x - mn) / (mx - mn) * (M - 1)).astype(np.int64)
    return np.bincount(lev.ravel(), minlength=M) / float(streams * n)


@pytest.mark.parametrize("M,n,streams", [(8, 1024, 3000), (6, 1024, 3000),
                                         (8, 128, 20000), (6, 128, 20000)])
def test_model_matches_monte_carlo(M, n, streams):
    p = O.order_stat_probs(M, n)
    h = _mc_hist(M, n, streams, seed=M * 1000 + n)
    # symbols of one stream are correlated through (min, max); 6 sigma of the
    # iid binomial error, widened 3x for that correlation
    sig = np.sqrt(p * (1 - p) / (streams * n)) * 3.0
    assert np.all(np.abs(h - p) <= 6 * sig + 1e-5), (h, p)


def test_model_special_cases():
    # n = 2: both values are the min and the max
    p = O.order_stat_probs(5, 2)
    assert np.allclose(p, [0.5, 0, 0, 0, 0.5])
    for M, n in [(8, 1024), (6, 128), (16, 300), (2, 64)]:
        p = O.order_stat_probs(M, n)
        assert abs(p.sum() - 1) < 1e-12
        assert np.array_equal(p, p[::-1])
        assert np.all(p > 0)
    # M = 2: only the min and max endpoints decide; an interior value goes to
    # the upper level iff it is above the midrange, so by symmetry p = 1/2
    assert np.allclose(O.order_stat_probs(2, 100), [0.5, 0.5], atol=1e-12)


def test_quadrature_converged():
    a = O.order_stat_probs(8, 1024, nodes=512)
    b = O.order_stat_probs(8, 1024, nodes=1024)
    assert np.max(np.abs(a - b)) < 1e-12


def test_sharpen_and_integer_table():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    assert np.allclose(O.sharpen(p, 1.0), p)
    q = O.sharpen(p, 1.4)
    assert q[3] > p[3] and q[0] < p[0] and abs(q.sum() - 1) < 1e-15
    # floors [25, 51, 76, 102] = 254, remainders .6,.2,.8,.4 -> +1 to idx 2, 0
    f = O.integer_table(np.array([0.1, 0.2, 0.3, 0.4]))
    assert f.tolist() == [26, 51, 77, 102]
    # clamp to 1 then give units back from the largest count
    f = O.integer_table(np.array([1e-9] * 5 + [1 - 5e-9]))
    assert f.tolist() == [1, 1, 1, 1, 1, 251]
    for M, n in [(8, 1024), (6, 1024), (8, 128), (6, 128), (16, 1024)]:
        f, c = O.build_table(M, n, 1.4)
        assert f.sum() == 256 and f.min() >= 1
        assert c[0] == 0 and np.all(c[1:] == np.cumsum(f)[:-1])


def test_rate_table_powers_of_two():
    r = O.rate_table(np.array([1, 2, 64, 128, 256]))
    assert r.tolist() == [8 << 16, 7 << 16, 2 << 16, 1 << 16, 0]
    r = O.rate_table(np.array([92]))
    assert abs(r[0] / 65536 - (8 - np.log2(92))) <= 2 ** -17


def test_lambda_grid():
    E = O.lambda_table()
    assert E.dtype == np.float32 and E[0] == 1.0
    assert E[256].view(np.uint32) == np.float32(np.sqrt(2.0)).view(np.uint32)
    t = 2.0 ** (np.arange(512) / 512.0)
    # correctly rounded: within half an fp32 ulp of the true value
    assert np.all(np.abs(E.astype(np.float64) - t) <= 2.0 ** -24 * 2)
    assert np.all(np.abs(E.astype(np.float64) - t) <= np.spacing(E).astype(np.float64) / 2)
    assert np.all(np.diff(E) > 0)


def test_decode_table_inverts_cumulative():
    f, c = O.build_table(8, 1024, 1.4)
    sym, fz, bias = O.decode_table(f, c)
    for z in range(256):
        m = sym[z]
        assert c[m] <= z < c[m] + f[m]
        assert fz[z] == f[m] and bias[z] == z - c[m]
