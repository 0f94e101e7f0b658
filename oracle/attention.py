"""Decode attention over the quantised cache, in float64.

Follows [D-Quant] Appendix A Eq. (7) (reconstruction k_hat = s v_m + o + mu),
Eqs. (8)-(9) (the affine terms fold into the QK and PV contractions) and
§4.2 (the rotation is per head and orthonormal, so attention in the rotated
basis equals attention in the original one after rotating back).

Readings: the softmax scale is tau = 1/sqrt(d) unless given (the page does not
state it; it follows the standard scaled dot-product attention); one decode
query per sequence and no mask; query head h reads KV head floor(h / G),
G = Hq / Hkv.

``attention_plain_f64`` is the plain definition: dequantise, rotate back,
softmax(q K^T tau) V.  ``attention_factored_f64`` evaluates Eqs. (8)-(9) and is
checked against it.  ``attention_with_residual_f64`` adds the most recent
tokens kept uncompressed ([D-Quant] §5.1 "Implementation details": the latest
tokens stay in BF16): they join the same softmax with their raw values.
"""

import numpy as np

from .transform import hadamard_f64

F64 = np.float64


def dequantize_f64(sym, so16, mu_hat_tok=None, vals=None):
    """s v_m + o (+ mu) in float64; sym [T, n], so16 float16 [T, 2], mu [T, n];
    vals are the level values (None: v_m = m)."""
    so = np.asarray(so16, np.float16).astype(F64)
    lev = np.asarray(sym, F64) if vals is None else np.asarray(vals, np.float32).astype(F64)[np.asarray(sym)]
    out = so[:, 0:1] * lev + so[:, 1:2]
    if mu_hat_tok is not None:
        out = out + np.asarray(mu_hat_tok, np.float32).astype(F64)
    return out


def _softmax_rows(z):
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def attention_plain_f64(q, khat_rot, vhat_rot, n_kv_heads, head_dim, scale=None):
    """q [Hq, d]; khat_rot, vhat_rot [T, n] in the rotated basis -> out [Hq, d]."""
    q = np.asarray(q, F64)
    Hq, d = q.shape
    T = khat_rot.shape[0]
    G = Hq // n_kv_heads
    tau = 1.0 / np.sqrt(float(d)) if scale is None else float(scale)
    H = hadamard_f64(d)
    K = np.asarray(khat_rot, F64).reshape(T, n_kv_heads, d) @ H   # H symmetric
    V = np.asarray(vhat_rot, F64).reshape(T, n_kv_heads, d) @ H
    out = np.zeros((Hq, d), F64)
    for h in range(Hq):
        g = h // G
        a = _softmax_rows((K[:, g, :] @ q[h]) * tau)
        out[h] = a @ V[:, g, :]
    return out


def attention_factored_f64(q, k_sym, k_so16, mu_hat_tok, v_sym, v_so16,
                           n_kv_heads, head_dim, scale=None, k_vals=None, v_vals=None):
    """Eqs. (8)-(9): contractions on the decoded levels v_m, affine terms
    applied after (k_vals / v_vals: level values, None for v_m = m)."""
    q = np.asarray(q, F64)
    Hq, d = q.shape
    T = k_sym.shape[0]
    G = Hq // n_kv_heads
    tau = 1.0 / np.sqrt(float(d)) if scale is None else float(scale)
    H = hadamard_f64(d)
    ks = np.asarray(k_so16, np.float16).astype(F64)
    vs = np.asarray(v_so16, np.float16).astype(F64)
    lev = lambda sym, vals: (np.asarray(sym, F64) if vals is None
                             else np.asarray(vals, np.float32).astype(F64)[np.asarray(sym)])
    km = lev(k_sym, k_vals).reshape(T, n_kv_heads, d)
    vm = lev(v_sym, v_vals).reshape(T, n_kv_heads, d)
    mu = np.asarray(mu_hat_tok, np.float32).astype(F64).reshape(T, n_kv_heads, d)
    out = np.zeros((Hq, d), F64)
    for h in range(Hq):
        g = h // G
        qr = H @ q[h]
        logit = (ks[:, 0] * (km[:, g, :] @ qr) + ks[:, 1] * qr.sum()
                 + mu[:, g, :] @ qr) * tau
        a = _softmax_rows(logit)
        o_rot = (a * vs[:, 0]) @ vm[:, g, :] + (a * vs[:, 1]).sum()
        out[h] = H @ o_rot
    return out


def attention_with_residual_f64(q, khat_rot, vhat_rot, res_k, res_v, n_kv_heads, head_dim,
                                scale=None):
    """Plain attention over T compressed tokens (khat_rot, vhat_rot [T, n] in
    the rotated basis, T may be 0) followed by R uncompressed tokens (res_k,
    res_v [R, n] in the original basis, R may be 0)."""
    q = np.asarray(q, F64)
    Hq, d = q.shape
    G = Hq // n_kv_heads
    tau = 1.0 / np.sqrt(float(d)) if scale is None else float(scale)
    H = hadamard_f64(d)
    n = n_kv_heads * head_dim
    kr = np.asarray(khat_rot, F64).reshape(-1, n)
    vr = np.asarray(vhat_rot, F64).reshape(-1, n)
    K = np.concatenate([(kr.reshape(-1, n_kv_heads, d) @ H),
                        np.asarray(res_k, F64).reshape(-1, n_kv_heads, d)])
    V = np.concatenate([(vr.reshape(-1, n_kv_heads, d) @ H),
                        np.asarray(res_v, F64).reshape(-1, n_kv_heads, d)])
    if K.shape[0] == 0:
        raise ValueError("attention over zero tokens")
    out = np.zeros((Hq, d), F64)
    for h in range(Hq):
        g = h // G
        a = _softmax_rows((K[:, g, :] @ q[h]) * tau)
        out[h] = a @ V[:, g, :]
    return out
