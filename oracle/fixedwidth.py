"""Fixed-width comparator of [D-Quant] Appendix B ("Comparison with
Fixed-Width Coding at Matched Storage").

The page keeps the preprocessing of the entropy-coded path (Hadamard
rotation, windowed INT8 key-mean removal, token-wise min-max affine grid,
least-squares refit, FP16 metadata) and replaces rANS + drift by fixed-width
symbols assigned by nearest-level rounding, at 6 key and 3 value levels.

Readings (the page charges the ideal log2 M bits per symbol and prints no
container layout; these fix one):
  * symbols: nearest-level rounding on the fitted grid (lowest index on
    ties, the lambda -> 0 limit of Drift), refit of (s, o) on those symbols
    exactly as in Algorithm 1, FP16 rounding, nearest-level rounding again on
    the FP16 grid;
  * width: b = the smallest of 1, 2, 4, 8 with 2^b >= M (the ideal log2 M bits
    cannot hold every symbol at one fixed width), so a stream takes n b / 8
    bytes;
  * layout: symbol i = 4 c + r (c = i // 4, r = i % 4) sits in byte r of
    little-endian dword c // (8 / b), at bits [b (c mod 8/b), b (c mod 8/b) + b)
    of that byte.  A dword thus holds 8 / b groups of 4 consecutive symbols, and
    group c is (dword >> b (c mod 8/b)) & (2^b - 1) * 0x01010101, one symbol per
    byte.
"""

import numpy as np

from .quant import fit_minmax, nearest_levels, refit
from .transform import rotate_heads, key_window_mean

F32 = np.float32


def fw_bits(levels):
    """Bits per symbol: the smallest of 1, 2, 4, 8 that holds `levels` symbols."""
    for b in (1, 2, 4, 8):
        if (1 << b) >= levels:
            return b
    raise ValueError("more than 256 levels")


def fw_container_bytes(levels, n):
    b = fw_bits(levels)
    if (n * b) % 32:
        raise ValueError("stream does not fill whole dwords")
    return n * b // 8


def fw_pack(m, levels):
    """Symbols m [N, n] -> containers [N, n b / 8] uint8 in the layout above."""
    m = np.asarray(m, np.int64)
    N, n = m.shape
    b = fw_bits(levels)
    per = 8 // b                       # groups of 4 symbols per dword
    out = np.zeros((N, fw_container_bytes(levels, n)), np.uint8)
    for i in range(n):
        c, r = divmod(i, 4)
        byte = 4 * (c // per) + r
        out[:, byte] |= (m[:, i] << (b * (c % per))).astype(np.uint8)
    return out


def fw_unpack(cont, levels, n):
    """Containers [N, n b / 8] -> symbols [N, n]."""
    cont = np.asarray(cont, np.uint8)
    b = fw_bits(levels)
    per = 8 // b
    m = np.zeros((cont.shape[0], n), np.int64)
    for i in range(n):
        c, r = divmod(i, 4)
        m[:, i] = (cont[:, 4 * (c // per) + r].astype(np.int64) >> (b * (c % per))) & ((1 << b) - 1)
    return m


def encode_streams_fw(x, levels):
    """Fixed-width encoding of each row of x (rotated; keys also centred)."""
    x = np.asarray(x, F32)
    s, o = fit_minmax(x, levels)
    m1 = nearest_levels(x, s, o, levels)
    s16, o16 = refit(x, m1, s, o)
    m2 = nearest_levels(x, s16.astype(F32), o16.astype(F32), levels)
    return {"cont": fw_pack(m2, levels), "s16": s16, "o16": o16, "m": m2}


def encode_cache_fw(k, v, n_kv_heads, head_dim, levels_k=6, levels_v=3, mean_window=128):
    """One sequence, k, v [T, n] in the original basis (as oracle.encode_cache)."""
    k = np.asarray(k, F32)
    v = np.asarray(v, F32)
    k_rot = rotate_heads(k, head_dim)
    v_rot = rotate_heads(v, head_dim)
    mu_q, mu_sc, mu_hat = key_window_mean(k_rot, mean_window)
    xk = k_rot - np.repeat(mu_hat, mean_window, axis=0)
    ks = encode_streams_fw(xk, levels_k)
    vs = encode_streams_fw(v_rot, levels_v)
    return {
        "k_cont": ks["cont"], "v_cont": vs["cont"],
        "k_so": np.stack([ks["s16"], ks["o16"]], axis=1), "v_so": np.stack([vs["s16"], vs["o16"]], axis=1),
        "k_mean_q": mu_q, "k_mean_scale": mu_sc, "mu_hat": mu_hat,
        "k_sym": ks["m"], "v_sym": vs["m"],
    }
