"""Pins for oracle.fixedwidth ([D-Quant] Appendix B: the fixed-width comparator)."""

import numpy as np
import pytest

import oracle as O


def test_widths_and_sizes():
    assert [O.fw_bits(M) for M in (2, 3, 4, 5, 6, 8, 9, 16, 17, 256)] == [1, 2, 2, 4, 4, 4, 4, 4, 8, 8]
    # the page's comparator levels: 6 key levels at 4 bits, 3 value levels at 2 bits
    assert O.fw_container_bytes(6, 1024) == 512 and O.fw_container_bytes(3, 1024) == 256


def test_hand_worked_layout():
    # 16 symbols at 4 bits: dword 0 holds groups 0 (low nibbles) and 1 (high
    # nibbles), dword 1 groups 2 and 3; byte r of a dword holds symbol r of each group
    m = np.array([[0, 1, 2, 3, 4, 5, 1, 2, 5, 4, 3, 2, 1, 0, 0, 5]])
    cont = O.fw_pack(m, 6)
    assert cont.tobytes().hex() == "40511223" + "15040352"


def test_two_bit_layout_closed_form():
    rng = np.random.default_rng(1)
    m = rng.integers(0, 3, (5, 64))
    cont = O.fw_pack(m, 3)
    words = cont.view("<u4")
    for c in range(16):
        grp = (words[:, c // 4] >> (2 * (c % 4))) & 0x03030303
        for r in range(4):
            assert np.array_equal((grp >> (8 * r)) & 0xFF, m[:, 4 * c + r])


@pytest.mark.parametrize("M", [2, 3, 6, 16, 200])
def test_round_trip(M):
    rng = np.random.default_rng(M)
    n = 256
    m = rng.integers(0, M, (7, n))
    assert np.array_equal(O.fw_unpack(O.fw_pack(m, M), M, n), m)


def test_symbols_equal_algorithm1_without_budget_pressure():
    # with a container no assignment can overflow, Algorithm 1's drift stops
    # at the small-lambda end, i.e. nearest rounding on each grid, so the
    # fixed-width symbols and scales are those of Algorithm 1
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 256)).astype(np.float32)
    for M in (6, 3):
        f, c = O.build_table(M, 256, 1.4)
        r = O.rate_table(f)
        a = O.encode_streams_alg1(x, M, f, c, r, 4096, O.lambda_table())
        b = O.encode_streams_fw(x, M)
        assert np.array_equal(a["m"], b["m"])
        assert np.array_equal(a["s16"].view(np.uint16), b["s16"].view(np.uint16))
        assert np.array_equal(a["o16"].view(np.uint16), b["o16"].view(np.uint16))


def test_nearest_rounding_error_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((30, 128)).astype(np.float32)
    r = O.encode_streams_fw(x, 6)
    s = r["s16"].astype(np.float64)[:, None]
    o = r["o16"].astype(np.float64)[:, None]
    rec = o + s * r["m"]
    inside = (x >= o) & (x <= o + 5 * s)
    bound = np.broadcast_to(s / 2 * (1 + 1e-3) + 1e-6, x.shape)
    # inside the grid every value is within half a step of its level
    assert np.all(np.abs(x - rec)[inside] <= bound[inside])


def test_cache_fw_equals_entropy_pipeline_without_budget_pressure():
    # The whole-cache comparator (rotation, key means, streams) against the
    # entropy-coded pipeline with containers too large for drift to act: the
    # two share every step but the coding, so their symbols, metadata and key
    # means must agree exactly.
    rng = np.random.default_rng(8)
    T, Hkv, d = 256, 1, 128
    mu = rng.normal(0, 0.5, Hkv * d).astype(np.float32)
    k = (rng.standard_normal((T, Hkv * d)) + mu).astype(np.float32)
    v = rng.standard_normal((T, Hkv * d)).astype(np.float32)
    fw = O.encode_cache_fw(k, v, Hkv, d, 6, 3, 128)
    ent = O.encode_cache(k, v, O.OracleParams(Hkv, d, 6, 3, 200, 200, 128, 1.4))
    for key in ("k_sym", "v_sym", "k_mean_q"):
        assert np.array_equal(fw[key], ent[key]), key
    for key in ("k_so", "v_so", "k_mean_scale"):
        assert np.array_equal(np.asarray(fw[key]).view(np.uint16), np.asarray(ent[key]).view(np.uint16)), key
    assert fw["k_cont"].shape == (T, O.fw_container_bytes(6, Hkv * d))
    assert np.array_equal(O.fw_unpack(fw["k_cont"], 6, Hkv * d), fw["k_sym"])
    assert np.array_equal(O.fw_unpack(fw["v_cont"], 3, Hkv * d), fw["v_sym"])
