"""The Figure 6 (left) analogue of the studies against the oracle (CPU).

kv_cache_entropy_amd.studies.max_alphabet asks the library which alphabets
are feasible for a payload (plan creation fails with KVQ_EINFEASIBLE when the
cheapest symbol of every value does not fit); the oracle's tables decide the
same question independently: n min_m r_fx[m] <= B_fx(C), with its own
frequency tables and rates.  The fixed-width columns are pinned to the
page's statement that equal-rate fixed-width coding at the default 2.68 /
1.84 bits per value permits 6 key and 3 value levels ([D-Quant] Appendix B),
and the default 8/6 alphabet must lie inside the entropy-coded feasible
region at the default 331/231-byte containers (Appendix C, Figure 6 left).
"""

import functools
import math

import pytest

from oracle.model import build_table, rate_table, budget_fx

PAYLOADS = [0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.25, 2.5, 3.0, 4.0]


def _studies():
    try:
        from kv_cache_entropy_amd import studies
        return studies
    except OSError as e:                 # library not built
        pytest.skip(f"libkvq not loadable: {e}")


@functools.lru_cache(maxsize=None)
def oracle_min_rate(M, n, alpha=1.4):
    f, _ = build_table(M, n, alpha)
    return int(rate_table(f).min())


def oracle_feasible(M, n, C):
    return n * oracle_min_rate(M, n) <= budget_fx(C)


def test_feasible_alphabets_match_the_oracle():
    studies = _studies()
    rows = studies.max_alphabet(8, 128, PAYLOADS)
    n = 1024
    for r in rows:
        want = [M for M in range(2, 17) if oracle_feasible(M, n, r["container_bytes"])]
        assert r["feasible_levels"] == want, (r["payload_bits"], r["feasible_levels"], want)
        assert r["max_levels_entropy"] == (max(want) if want else None)
        assert r["container_bytes"] == math.ceil((r["payload_bits"] * n + 32) / 8)


def test_entropy_coding_holds_more_levels_than_fixed_width():
    studies = _studies()
    for r in studies.max_alphabet(8, 128, PAYLOADS):
        if r["max_levels_entropy"] is not None:
            assert r["max_levels_entropy"] >= r["max_levels_fixed_width_ideal"]
            assert r["max_levels_fixed_width_ideal"] >= r["max_levels_fixed_width_whole_bits"]


def test_fixed_width_at_the_default_rates_matches_appendix_b():
    studies = _studies()
    k, v = studies.max_alphabet(8, 128, [2.68, 1.84])
    assert (k["max_levels_fixed_width_ideal"], v["max_levels_fixed_width_ideal"]) == (6, 3)


def test_default_alphabet_is_feasible_at_the_default_containers():
    studies = _studies()
    # 331 and 231 bytes carry (8 C - 32) / 1024 bits per value of payload
    k, v = studies.max_alphabet(8, 128, [(8 * 331 - 32) / 1024, (8 * 231 - 32) / 1024])
    assert (k["container_bytes"], v["container_bytes"]) == (331, 231)
    assert 8 in k["feasible_levels"] and 6 in v["feasible_levels"]
