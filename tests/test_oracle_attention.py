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


# ---- uncompressed residual tail ([D-Quant] §5.1 "Implementation details")

def _residual_setup(seed, T, R, Hkv=2, Hq=8, d=32):
    rng = np.random.default_rng(seed)
    k_sym, k_so, v_sym, v_so, mu = _random_cache(rng, max(T, 16), Hkv, d)
    k_sym, k_so, v_sym, v_so, mu = k_sym[:T], k_so[:T], v_sym[:T], v_so[:T], mu[:T]
    kh = O.dequantize_f64(k_sym, k_so, mu)
    vh = O.dequantize_f64(v_sym, v_so)
    rk = rng.standard_normal((R, Hkv * d))
    rv = rng.standard_normal((R, Hkv * d))
    q = rng.standard_normal((Hq, d))
    return q, kh, vh, rk, rv, Hkv, d


def test_residual_empty_tail_is_plain_attention():
    q, kh, vh, rk, rv, Hkv, d = _residual_setup(1, 32, 0)
    a = O.attention_with_residual_f64(q, kh, vh, rk, rv, Hkv, d)
    b = O.attention_plain_f64(q, kh, vh, Hkv, d)
    assert np.array_equal(a, b)


def test_residual_only_matches_torch_sdpa():
    q, kh, vh, rk, rv, Hkv, d = _residual_setup(2, 0, 37)
    out = O.attention_with_residual_f64(q, kh, vh, rk, rv, Hkv, d)
    Hq, G = q.shape[0], q.shape[0] // Hkv
    K = torch.from_numpy(rk.reshape(-1, Hkv, d)).permute(1, 0, 2).repeat_interleave(G, 0)
    V = torch.from_numpy(rv.reshape(-1, Hkv, d)).permute(1, 0, 2).repeat_interleave(G, 0)
    Q = torch.from_numpy(q)[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, 0, :].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_residual_equals_same_tokens_compressed():
    # tokens given in the tail with their dequantised values (original basis)
    # must act exactly like the same tokens in the compressed part
    q, kh, vh, rk, rv, Hkv, d = _residual_setup(3, 48, 0)
    H = O.hadamard_f64(d)
    orig = lambda x: (x.reshape(-1, Hkv, d) @ H).reshape(x.shape[0], -1)
    a = O.attention_with_residual_f64(q, kh, vh, rk, rv, Hkv, d)
    b = O.attention_with_residual_f64(q, kh[:32], vh[:32], orig(kh[32:]), orig(vh[32:]), Hkv, d)
    c = O.attention_with_residual_f64(q, kh[:0], vh[:0], orig(kh), orig(vh), Hkv, d)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    assert np.max(np.abs(a - c)) <= 1e-12 * np.max(np.abs(a))


def test_residual_single_token_returns_its_value():
    q, kh, vh, rk, rv, Hkv, d = _residual_setup(4, 0, 1)
    out = O.attention_with_residual_f64(q, kh, vh, rk, rv, Hkv, d)
    G = q.shape[0] // Hkv
    for h in range(q.shape[0]):
        assert np.array_equal(out[h], rv[0].reshape(Hkv, d)[h // G])


def test_residual_rejects_empty_attention():
    q, kh, vh, rk, rv, Hkv, d = _residual_setup(5, 0, 0)
    with pytest.raises(ValueError):
        O.attention_with_residual_f64(q, kh, vh, rk, rv, Hkv, d)
