"""Whole-cache encode / decode for one sequence, built from the other modules.

Follows [D-Quant] Figure 1 (keys: Hadamard, remove channel mean, affine
quantisation, drift, rANS, container; values: the same without the mean) and
§4.2 (a stream is the n = Hkv * d values of one token's keys, or values, at
one layer; it shares one scale and one offset).

Reading: inside a stream the values are ordered [kv_head][dim], so symbol
i = g d + j; decoding therefore yields one KV head after another.
"""

from dataclasses import dataclass, field

import numpy as np

from .model import build_table, rate_table, lambda_table, budget_fx, level_values_fp16
from .transform import rotate_heads, key_window_mean
from .quant import encode_streams_alg1
from .rans import rans_decode

F32 = np.float32


@dataclass
class OracleParams:
    n_kv_heads: int
    head_dim: int
    levels_k: int = 8
    levels_v: int = 6
    container_bytes_k: int = 331
    container_bytes_v: int = 231
    mean_window: int = 128
    alpha: float = 1.4
    values_k: tuple = None        # non-affine key levels in grid units (None: v_m = m)
    values_v: tuple = None
    _cache: dict = field(default_factory=dict, repr=False, compare=False)

    @property
    def n(self):
        return self.n_kv_heads * self.head_dim

    def vals(self, side):
        """Level values as stored (float16, as float32)."""
        M = self.levels_k if side == "k" else self.levels_v
        return level_values_fp16(M, self.values_k if side == "k" else self.values_v)

    def table(self, side):
        """(f, c, r_fx) for side 'k' or 'v'."""
        if side not in self._cache:
            M = self.levels_k if side == "k" else self.levels_v
            raw = self.values_k if side == "k" else self.values_v
            vals = None if raw is None else self.vals(side).astype(float)
            f, c = build_table(M, self.n, self.alpha, vals)
            self._cache[side] = (f, c, rate_table(f))
        return self._cache[side]

    def lam(self):
        if "E" not in self._cache:
            self._cache["E"] = lambda_table()
        return self._cache["E"]

    def check_feasible(self):
        for side, C in (("k", self.container_bytes_k), ("v", self.container_bytes_v)):
            _, _, r = self.table(side)
            if self.n * int(r.min()) > budget_fx(C):
                raise ValueError(f"container too small for side {side}")


def _encode_side(x, levels, tab, C, E, chunk, vals=None):
    f, c, r = tab
    outs = [encode_streams_alg1(x[i:i + chunk], levels, f, c, r, C, E, vals)
            for i in range(0, x.shape[0], chunk)]
    cat = lambda k: np.concatenate([o[k] for o in outs])
    return {
        "cont": cat("cont"), "so": np.stack([cat("s16"), cat("o16")], axis=1),
        "sym": cat("m"), "payload": cat("payload"),
        "fallback1": int(cat("fallback1").sum()),
        "fallback2": int(cat("fallback2").sum()),
        "changed": sum(o["changed"] for o in outs),
    }


def encode_cache(k, v, p, chunk=256):
    """Encode one sequence: k, v float32-representable [T, n] (original basis)."""
    p.check_feasible()
    k = np.asarray(k, F32)
    v = np.asarray(v, F32)
    T, n = k.shape
    k_rot = rotate_heads(k, p.head_dim)
    v_rot = rotate_heads(v, p.head_dim)
    mu_q, mu_sc, mu_hat = key_window_mean(k_rot, p.mean_window)
    xk = k_rot - np.repeat(mu_hat, p.mean_window, axis=0)
    E = p.lam()
    vk = None if p.values_k is None else p.vals("k")
    vv = None if p.values_v is None else p.vals("v")
    ks = _encode_side(xk, p.levels_k, p.table("k"), p.container_bytes_k, E, chunk, vk)
    vs = _encode_side(v_rot, p.levels_v, p.table("v"), p.container_bytes_v, E, chunk, vv)
    return {
        "k_cont": ks["cont"], "v_cont": vs["cont"],
        "k_so": ks["so"], "v_so": vs["so"],
        "k_mean_q": mu_q, "k_mean_scale": mu_sc, "mu_hat": mu_hat,
        "k_sym": ks["sym"], "v_sym": vs["sym"],
        "k_payload": ks["payload"], "v_payload": vs["payload"],
        "stats": np.array([ks["fallback1"], ks["fallback2"], ks["changed"], 0,
                           vs["fallback1"], vs["fallback2"], vs["changed"], 0],
                          np.uint64),
    }


def decode_cache_symbols(cont, p, side):
    """Symbols of every container row (Algorithm 2)."""
    f, c, _ = p.table(side)
    sym, x_end, ptr = rans_decode(cont, f, c, p.n)
    return sym, x_end, ptr
