"""Pins for oracle.attention ([D-Quant] Appendix A Eqs. (7)-(9))."""

import numpy as np
import pytest
import torch

import oracle as O


def _random_cache(rng, T, Hkv, d, Mk=8, Mv=6, W=16):
    n = Hkv * d
    k_sym = rng.integers(0, Mk, (T, n))
    v_sym = rng.integers(0, Mv, (T, n))
    k_so = np.stack([rng.uniform(0.1, 1, T), rng.uniform(-3, 0, T)], 1).astype(np.float16)
    v_so = np.stack([rng.uniform(0.1, 1, T), rng.uniform(-3, 0, T)], 1).astype(np.float16)
    mu = np.repeat(rng.standard_normal((T // W, n)).astype(np.float32), W, axis=0)
    return k_sym, k_so, v_sym, v_so, mu


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 2)])
def test_factored_equals_plain(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    T, d = 64, 32
    k_sym, k_so, v_sym, v_so, mu = _random_cache(rng, T, Hkv, d)
    q = rng.standard_normal((Hq, d))
    kh = O.dequantize_f64(k_sym, k_so, mu)
    vh = O.dequantize_f64(v_sym, v_so)
    a = O.attention_plain_f64(q, kh, vh, Hkv, d)
    b = O.attention_factored_f64(q, k_sym, k_so, mu, v_sym, v_so, Hkv, d)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))


def test_plain_matches_torch_sdpa():
    rng = np.random.default_rng(21)
    T, Hkv, Hq, d = 48, 2, 8, 64
    k_sym, k_so, v_sym, v_so, mu = _random_cache(rng, T, Hkv, d)
    q = rng.standard_normal((Hq, d))
    kh = O.dequantize_f64(k_sym, k_so, mu)
    vh = O.dequantize_f64(v_sym, v_so)
    out = O.attention_plain_f64(q, kh, vh, Hkv, d)
    H = O.hadamard_f64(d)
    K = torch.tensor(kh.reshape(T, Hkv, d) @ H).permute(1, 0, 2)      # [Hkv, T, d]
    V = torch.tensor(vh.reshape(T, Hkv, d) @ H).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    Q = torch.tensor(q)[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, 0, :].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_attention_special_cases():
    rng = np.random.default_rng(22)
    d, Hkv = 32, 1
    k_sym, k_so, v_sym, v_so, mu = _random_cache(rng, 16, Hkv, d)
    H = O.hadamard_f64(d)
    vh = O.dequantize_f64(v_sym, v_so)
    q = rng.standard_normal((2, d))
    # one token: the output is that token's value, rotated back
    out = O.attention_plain_f64(q, O.dequantize_f64(k_sym[:1], k_so[:1], mu[:1]), vh[:1], Hkv, d)
    assert np.allclose(out, np.tile(vh[0] @ H, (2, 1)), atol=1e-12)
    # q = 0: uniform weights -> mean of the values
    out = O.attention_plain_f64(np.zeros((1, d)), O.dequantize_f64(k_sym, k_so, mu), vh, Hkv, d)
    assert np.allclose(out[0], (vh @ H).mean(axis=0), atol=1e-12)
    # identical keys: uniform weights as well
    ks = np.tile(k_sym[:1], (16, 1))
    kso = np.tile(k_so[:1], (16, 1))
    out = O.attention_plain_f64(q, O.dequantize_f64(ks, kso, np.tile(mu[:1], (16, 1))), vh, Hkv, d)
    assert np.allclose(out, np.tile((vh @ H).mean(axis=0), (2, 1)), atol=1e-12)
