"""Writes tests/golden/oracle_tiny_regression.json by calling only oracle/.

Seeded input (numpy PCG64, seed 0): the first 128-token window of a 1-head,
d = 128 cache with per-channel key offsets N(0, 0.5^2), K = N(0,1) + offset,
V = N(0,1), fp32; 36-byte containers, 8/6 levels, alpha 1.4.  The file pins
the oracle against unintended changes of its own arithmetic; a deliberate
change regenerates it (python tests/golden/make_oracle_golden.py) in a commit
that names the passage or reading that justifies it.
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402


def tiny_inputs():
    rng = np.random.default_rng(0)
    mu = rng.normal(0.0, 0.5, 128).astype(np.float32)
    k = (rng.standard_normal((128, 128)) + mu).astype(np.float32)
    v = rng.standard_normal((128, 128)).astype(np.float32)
    return k, v


def main():
    k, v = tiny_inputs()
    p = O.OracleParams(1, 128, 8, 6, 36, 36, 128, 1.4)
    r = O.encode_cache(k, v, p)
    fk, ck, rk = p.table("k")
    fv, cv, rv = p.table("v")
    out = {
        "table_k": {"f": fk.tolist(), "c": ck.tolist(), "r_fx": rk.tolist()},
        "table_v": {"f": fv.tolist(), "c": cv.tolist(), "r_fx": rv.tolist()},
        "k_cont_hex": [bytes(row).hex() for row in r["k_cont"][:8]],
        "v_cont_hex": [bytes(row).hex() for row in r["v_cont"][:8]],
        "k_so_bits": r["k_so"][:8].view(np.uint16).tolist(),
        "v_so_bits": r["v_so"][:8].view(np.uint16).tolist(),
        "k_mean_q": r["k_mean_q"][0, :16].tolist(),
        "k_mean_scale_bits": int(r["k_mean_scale"].view(np.uint16)[0]),
        "stats": r["stats"].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_regression.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
