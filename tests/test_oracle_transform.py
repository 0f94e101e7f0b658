"""Pins for oracle.transform: the per-head Hadamard and the INT8 window mean
([D-Quant] Figure 1, §4.2, Appendix A Eq. (7), Appendix B)."""

import numpy as np
import pytest
import scipy.linalg

import oracle as O


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_fwht_columns_are_sylvester_hadamard(d):
    H = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)   # Sylvester order
    cols = O.fwht_f32(np.eye(d, dtype=np.float32))                # row k = H e_k
    assert np.max(np.abs(cols.astype(np.float64) - H.T)) < 1e-7
    assert np.array_equal(O.hadamard_f64(d), H)
    assert np.allclose(H @ H.T, np.eye(d), atol=1e-14)


def test_fwht_isometry_and_involution():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    y = O.fwht_f32(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    assert np.allclose(O.fwht_f32(y), x, atol=1e-5)
    # agrees with the float64 matrix product
    H = O.hadamard_f64(128)
    assert np.allclose(y, x.astype(np.float64) @ H.T, atol=1e-5)


def test_rotate_heads_is_per_head():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 2 * 64)).astype(np.float32)
    y = O.rotate_heads(x, 64)
    assert np.array_equal(y[:, :64], O.fwht_f32(x[:, :64]))
    assert np.array_equal(y[:, 64:], O.fwht_f32(x[:, 64:]))


def test_key_mean_identical_tokens_and_zero():
    # values on a 2^-8 grid in [-4, 4]: every partial sum is exact in fp32
    rng = np.random.default_rng(5)
    tok = (rng.integers(-1024, 1024, 256) / 256.0).astype(np.float32)
    k = np.tile(tok, (128, 1))
    mu_q, sc, mu_hat = O.key_window_mean(k, 128)
    a = np.max(np.abs(tok))
    assert sc[0] == np.float16(np.float32(a) / np.float32(127))
    assert np.all(np.abs(mu_hat[0] - tok) <= np.float32(sc[0]) / 2 * (1 + 1e-6))
    z = np.zeros((256, 64), np.float32)
    mu_q, sc, mu_hat = O.key_window_mean(z, 128)
    assert np.all(mu_q == 0) and np.all(sc == 0) and np.all(mu_hat == 0)


def test_key_mean_error_bound():
    rng = np.random.default_rng(6)
    k = (rng.standard_normal((512, 1024)) + rng.standard_normal(1024)).astype(np.float32)
    mu_q, sc, mu_hat = O.key_window_mean(k, 128)
    mean64 = k.astype(np.float64).reshape(4, 128, 1024).mean(axis=1)
    for w in range(4):
        s = float(np.float32(sc[w]))
        assert np.max(np.abs(mu_hat[w] - mean64[w])) <= s / 2 + 1e-5
        assert np.abs(mu_q[w]).max() in (126, 127)
        assert np.abs(mu_q[w]).max() <= 127


def test_key_mean_token_order_sum():
    # the fp32 running sum in token order, not a pairwise sum: a case where
    # the two orders differ
    k = np.zeros((128, 64), np.float32)
    k[0, 0] = np.float32(2 ** 24)
    k[1:, 0] = np.float32(1.0)
    mu_q, sc, mu_hat = O.key_window_mean(k, 128)
    # running sum: 2^24 + 1 rounds to 2^24 each step -> mean 2^24 / 128 = 2^17
    a = np.float32(2.0 ** 17)
    s = np.float32(np.float16(a / np.float32(127)))
    assert mu_q[0, 0] == np.clip(np.rint(a / s), -127, 127)
