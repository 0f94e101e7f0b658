"""Whole-pipeline properties of the oracle on the Tiny shape ([D-Quant]
Figure 1, §4.2 Eq. (3), Appendix A Algorithms 1-2, Appendix C)."""

import json
import os

import numpy as np

import oracle as O
from oracle.model import budget_fx

HERE = os.path.dirname(__file__)


def _tiny():
    from tests.golden.make_oracle_golden import tiny_inputs
    return tiny_inputs()


def test_regression_golden():
    """The oracle still produces the bytes its generator script recorded."""
    g = json.load(open(os.path.join(HERE, "golden", "oracle_tiny_regression.json")))
    k, v = _tiny()
    p = O.OracleParams(1, 128, 8, 6, 36, 36, 128, 1.4)
    r = O.encode_cache(k, v, p)
    assert [bytes(x).hex() for x in r["k_cont"][:8]] == g["k_cont_hex"]
    assert [bytes(x).hex() for x in r["v_cont"][:8]] == g["v_cont_hex"]
    assert r["k_so"][:8].view(np.uint16).tolist() == g["k_so_bits"]
    assert r["stats"].tolist() == g["stats"]


def test_tiny_end_to_end_properties():
    k, v = _tiny()
    p = O.OracleParams(1, 128, 8, 6, 36, 36, 128, 1.4)
    r = O.encode_cache(k, v, p)
    for side, C, M in (("k", 36, 8), ("v", 36, 6)):
        cont = r[f"{side}_cont"]
        assert cont.shape == (128, C)
        sym, x_end, ptr = O.decode_cache_symbols(cont, p, side)
        assert np.array_equal(sym, r[f"{side}_sym"])
        assert np.all(x_end == O.L_RANS)
        assert np.array_equal(ptr, 4 + r[f"{side}_payload"])
        f, c, rfx = p.table(side)
        assert np.all(rfx[sym].sum(axis=1) <= budget_fx(C))
        assert sym.min() >= 0 and sym.max() < M
    # reconstruction error is bounded by the grid: drift moves symbols only as
    # far as the rate needs, so the error stays well under the level spacing
    k_rot = O.rotate_heads(k, 128)
    kh = O.dequantize_f64(r["k_sym"], r["k_so"], np.repeat(r["mu_hat"], 128, axis=0))
    nmse = np.mean((kh - k_rot) ** 2) / np.mean((k_rot - k_rot.mean()) ** 2)
    assert nmse < 0.1


def test_drift_is_sparse_on_gaussian_streams():
    """Appendix C reports sparse, one-level drift on real KV; on Gaussian
    streams at the default 331/231 containers the same holds (plausibility)."""
    rng = np.random.default_rng(1)
    p = O.OracleParams(8, 128)
    k = rng.standard_normal((128, 1024)).astype(np.float32)
    v = rng.standard_normal((128, 1024)).astype(np.float32)
    r = O.encode_cache(k, v, p)
    n_sym = 128 * 1024
    assert r["stats"][2] / n_sym < 0.02          # keys: little drift
    assert r["stats"][6] / n_sym < 0.15          # values: more, still sparse
    v_rot = O.rotate_heads(v, 128)
    s = r["v_so"][:, 0].astype(np.float32)
    o = r["v_so"][:, 1].astype(np.float32)
    near = O.nearest_levels(v_rot, s, o, 6)
    assert np.abs(near - r["v_sym"]).max() <= 1
    assert r["stats"][0] == 0 and r["stats"][4] == 0     # no fallbacks


def test_quantised_attention_improves_with_budget():
    """More container bytes -> a closer attention output (§5.4: increasing the
    storage budget steadily approaches BF16), saturating once no stream needs
    to drift (then only the 8/6-level grid limits it)."""
    k, v = _tiny()
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 128))
    H = O.hadamard_f64(128)
    exact = O.attention_plain_f64(q, k.astype(np.float64) @ H, v.astype(np.float64) @ H, 1, 128)
    errs = []
    drifted = []
    for C in (36, 48, 72):
        p = O.OracleParams(1, 128, 8, 6, C, C, 128, 1.4)
        r = O.encode_cache(k, v, p)
        mu_tok = np.repeat(r["mu_hat"], 128, axis=0)
        out = O.attention_factored_f64(q, r["k_sym"], r["k_so"], mu_tok,
                                       r["v_sym"], r["v_so"], 1, 128)
        errs.append(np.linalg.norm(out - exact) / np.linalg.norm(exact))
        drifted.append(int(r["stats"][2] + r["stats"][6]))
    assert errs[0] > errs[1] >= errs[2]
    assert drifted[0] > drifted[1] > drifted[2] == 0
