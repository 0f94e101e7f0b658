"""The drift study (Figure 6 right analogue) on the GPU against the oracle.

tests/golden/study/drift_gqa_2x512.json is written by
tests/golden/make_study_goldens.py, which calls only oracle/ on the gqa
workload's sequences 0 and 1, tokens 0..511, from the seeded CPU generators.
The test generates the same inputs on the CPU, runs
kv_cache_entropy_amd.studies.drift_study through the C ABI (the launch holds
exactly these two sequences) and requires, per side and container size:
the symbol counts, the number of symbols drift changed (the encoder's
counters against nearest rounding on the final grid) and every stream's
remaining budget B - sum_i r_fx[m_i] to equal the oracle's exactly, the
remaining budget to be non-negative (drift's constraint) and the histogram
to count every stream once.
"""

import json
import os

import pytest
import torch

from kv_cache_entropy_amd import synth
from tests.golden import cases as C

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "study", "drift_gqa_2x512.json")


def test_drift_study_matches_the_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_entropy_amd import kvq, studies
    g = json.load(open(GOLDEN))
    w = synth.WORKLOADS[g["workload"]]
    k, v = synth.cache_inputs(w, "cpu", g["seqs"], tuple(g["tokens"]))
    assert {"k": C.input_digest(k), "v": C.input_digest(v)} == g["inputs"], \
        "this host's CPU generator gives other inputs than the golden's"
    k, v = k.cuda(), v.cuda()
    for case in g["cases"]:
        ck, cv = case["containers"]
        print(f"drift study {g['workload']} seqs {g['seqs']} tokens {g['tokens']} C=({ck},{cv})", flush=True)
        plan = kvq.Plan(w.n_kv_heads, w.head_dim, 8, 6, ck, cv, 128, 1.4)
        ds = studies.drift_study(plan, k, v)
        for side in ("k", "v"):
            got, want = ds[side], case[side]
            assert got["symbol_counts"] == want["symbol_counts"], side
            assert got["changed_symbols"] == want["changed_symbols"], side
            assert got["remaining_fx"] == want["remaining_fx"], side
            assert min(got["remaining_fx"]) >= 0
            assert sum(got["remaining_hist"]["counts"]) == len(want["remaining_fx"])
            assert got["overruns"] == 0
            print(f"  {side}: changed {got['changed_frac']:.3%}, remaining bits min "
                  f"{got['remaining_bits']['min']:.2f} median {got['remaining_bits']['median']:.1f}", flush=True)
