"""The committed parity goldens agree with the oracle as it stands.

tests/golden/parity/ is written by tests/golden/make_parity_goldens.py from
oracle/ alone; the GPU parity tests compare the HIP path with these files.
This CPU test recomputes the cheapest cases with the oracle and requires the
same digests, counters and float64 attention, so that a change to the oracle
cannot leave stale goldens behind unnoticed; every case must have its files."""

import json
import os

import numpy as np
import pytest

from tests.golden import cases as C
from tests.golden.make_parity_goldens import compute


def test_every_case_has_a_golden():
    for case in C.ALL:
        jpath, apath = C.golden_paths(case)
        assert os.path.exists(jpath), case["name"]
        assert os.path.exists(apath) == case["attention"], case["name"]


@pytest.mark.parametrize("name", ["tiny", "gqa_s2_scale025", "layout8x1", "dim32"])
def test_golden_matches_the_oracle(name):
    case = C.BY_NAME[name]
    rec, attn = compute(case, procs=1)
    jpath, apath = C.golden_paths(case)
    stored = json.load(open(jpath))
    assert json.loads(json.dumps(rec)) == stored
    if case["attention"]:
        assert np.array_equal(np.load(apath), attn)
