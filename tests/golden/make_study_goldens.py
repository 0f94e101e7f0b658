"""Writes tests/golden/study/drift_gqa_2x512.json by calling only oracle/.

The expected values of the drift study (the Figure 6 right analogue of
kv_cache_entropy_amd.studies.drift_study): for the gqa workload's sequences 0
and 1, tokens 0..511 (seeded CPU generators), at 8/6 levels with 331/231- and
292/203-byte containers, per side:
  * the symbol counts of the encoded streams,
  * the number of symbols drift changed against nearest rounding on the
    final FP16 grid (the encoder's counters),
  * every stream's remaining budget B - sum_i r_fx[m_i] in the rates' fixed
    point (B = 8 C - 32 bits, [D-Quant] §4.2 Eq. (3)),
  * for information, the largest distance in levels between a drifted symbol
    and nearest rounding (Appendix C reports at most one level).
Run from the repository root (a few minutes on one core):

    python tests/golden/make_study_goldens.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from oracle.model import budget_fx  # noqa: E402
from oracle.quant import nearest_levels  # noqa: E402
from oracle.transform import rotate_heads, key_window_mean  # noqa: E402
from kv_cache_entropy_amd import synth  # noqa: E402
from tests.golden import cases as C  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "study", "drift_gqa_2x512.json")
SEQS = [0, 1]
TOKENS = (0, 512)
CONTAINERS = [(331, 231), (292, 203)]


def main():
    w = synth.WORKLOADS["gqa"]
    k, v = synth.cache_inputs(w, "cpu", SEQS, TOKENS)
    rec = {"workload": w.name, "seqs": SEQS, "tokens": list(TOKENS), "levels": [8, 6],
           "inputs": {"k": C.input_digest(k), "v": C.input_digest(v)}, "cases": []}
    for ck, cv in CONTAINERS:
        p = O.OracleParams(w.n_kv_heads, w.head_dim, 8, 6, ck, cv, 128, 1.4)
        case = {"containers": [ck, cv]}
        per = {"k": [], "v": []}
        counts = {"k": np.zeros(8, np.int64), "v": np.zeros(6, np.int64)}
        changed = {"k": 0, "v": 0}
        moves = {"k": 0, "v": 0}
        for s in range(len(SEQS)):
            ks, vs = k[s].float().numpy(), v[s].float().numpy()
            r = O.encode_cache(ks, vs, p)
            st = [int(x) for x in r["stats"]]
            changed["k"] += st[2]
            changed["v"] += st[6]
            # the streams the encoder quantised, for the distance of each drifted symbol
            k_rot = rotate_heads(np.asarray(ks, np.float32), w.head_dim)
            _, _, mu_hat = key_window_mean(k_rot, 128)
            xs = {"k": k_rot - np.repeat(mu_hat, 128, axis=0),
                  "v": rotate_heads(np.asarray(vs, np.float32), w.head_dim)}
            for side, M, Cb in (("k", 8, ck), ("v", 6, cv)):
                sym = r[f"{side}_sym"]
                _, _, rate = p.table(side)
                per[side] += [int(budget_fx(Cb) - int(rate[row].sum())) for row in sym]
                counts[side] += np.bincount(sym.ravel(), minlength=M)
                so = r[f"{side}_so"].astype(np.float32)
                near = nearest_levels(xs[side], so[:, 0], so[:, 1], M)
                moves[side] = max(moves[side], int(np.abs(near - sym).max()))
        for side in ("k", "v"):
            case[side] = {"symbol_counts": [int(x) for x in counts[side]], "changed_symbols": changed[side],
                          "remaining_fx": per[side], "max_level_move": moves[side]}
            print(f"{ck}/{cv} {side}: changed {changed[side]}, max move {moves[side]}, "
                  f"min remaining {min(per[side]) / 65536:.2f} bits", flush=True)
        rec["cases"].append(case)
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    with open(OUT, "w") as fh:
        json.dump(rec, fh)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
