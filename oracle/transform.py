"""Per-head Hadamard rotation and the windowed key channel mean.

Follows [D-Quant] Figure 1 and §4.2 (Hadamard rotation per attention head;
keys then remove a windowed channel-wise mean), Appendix A Eq. (7) (the
decoder adds the mean back) and Appendix B ("windowed INT8 channel-mean
removal for keys").

Readings:
  * Hadamard: Sylvester order (H_1 = [1], H_2k = [[H, H], [H, -H]]),
    orthonormal (divided by sqrt(d)), applied to each head's d-vector.  The
    float32 evaluation is fixed: stages h = 1, 2, 4, ..., d/2; in stage h every
    pair (i, i+h) with bit h of i clear becomes (a + b, a - b); afterwards
    every element is multiplied by c_d = fp32(1/sqrt(d)).  It is applied
    online to keys and values alike (the page folds the value rotation into
    the projection weights offline; here there are no weights).
  * Window: W consecutive tokens [wW, (w+1)W) of one sequence.  The mean is
    taken on rotated keys (Figure 1 order: rotate, then remove the mean).
    mu_j = fp32 running sum over the window's tokens in order, starting from
    +0.0, times 1/W (W a power of two, so the scaling is exact).
  * INT8: a = max_j |mu_j| over the whole stream (all heads); the scale is
    sc = fp16(fp32(a / 127)); mu_q = clamp(rne(fp32(mu / sc)), -127, 127)
    (mu_q = 0 when sc == 0); the value the decoder adds back, and the value
    the encoder subtracts, is mu_hat = fp32(mu_q * sc).
"""

import numpy as np

F32 = np.float32


def fwht_f32(x):
    """Orthonormal Sylvester Hadamard over the last axis, float32 as specified."""
    x = np.array(x, dtype=np.float32, copy=True)
    d = x.shape[-1]
    if d & (d - 1):
        raise ValueError("head_dim must be a power of two")
    lead = x.shape[:-1]
    h = 1
    while h < d:
        y = x.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(lead + (d,))
        h *= 2
    return x * F32(1.0 / np.sqrt(np.float64(d)))


def hadamard_f64(d):
    """The orthonormal Sylvester Hadamard matrix in float64 (Kronecker form)."""
    H = np.ones((1, 1), np.float64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(float(d))


def rotate_heads(x, head_dim):
    """x: [..., n] with n = n_heads * head_dim; rotates every head slice."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    y = fwht_f32(x.reshape(x.shape[:-1] + (n // head_dim, head_dim)))
    return y.reshape(x.shape)


def key_window_mean(k_rot, window):
    """Windowed channel mean of rotated keys of one sequence.

    k_rot: float32 [T, n] with T a multiple of ``window``.
    Returns (mu_q int8 [T/W, n], mu_scale float16 [T/W], mu_hat float32 [T/W, n]).
    """
    k_rot = np.asarray(k_rot, np.float32)
    T, n = k_rot.shape
    if window <= 0 or window & (window - 1) or T % window:
        raise ValueError("window must be a power of two dividing seq_len")
    nw = T // window
    mu_q = np.zeros((nw, n), np.int8)
    mu_sc = np.zeros(nw, np.float16)
    mu_hat = np.zeros((nw, n), np.float32)
    inv_w = F32(1.0 / window)
    for w in range(nw):
        acc = np.zeros(n, np.float32)
        for t in range(w * window, (w + 1) * window):
            acc = acc + k_rot[t]
        mu = acc * inv_w
        a = np.max(np.abs(mu))
        sc16 = np.float16(F32(a) / F32(127.0))
        if not np.isfinite(sc16):
            raise ValueError("key mean scale overflows fp16")
        sc = F32(sc16)
        if sc == 0:
            q = np.zeros(n, np.int8)
        else:
            q = np.clip(np.rint(mu / sc), -127, 127).astype(np.int8)
        mu_q[w] = q
        mu_sc[w] = sc16
        mu_hat[w] = q.astype(np.float32) * sc
    return mu_q, mu_sc, mu_hat
