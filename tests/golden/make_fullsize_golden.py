"""Writes tests/golden/gqa_fullsize_expected.json by calling only oracle/.

Expected values for the full-size GQA decode check: the oracle's encoding of
one whole sequence of the 512 x 8192-token cache (the last one, s = 511) and
of the first key-mean window of sequence 0, and the oracle's float64
attention output for sequence 511.  Inputs are the seeded generators of
kv_cache_entropy_amd.synth run on the CPU (the GPU test generates these two
sequences on the CPU as well and the other 510 on the GPU).  Run with
    python tests/golden/make_fullsize_golden.py
(about four minutes on eight cores).  Container bytes are stored as SHA-256
digests of the C-contiguous arrays, so the file stays small.
"""

import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from kv_cache_entropy_amd import synth  # noqa: E402
from tests.oracle_pool import encode_cache_parallel  # noqa: E402

SEQ_FULL = 511
SEQ_WINDOW = 0


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def encoded_digests(r, t0, t1, w0, w1):
    return {
        "k_cont": digest(r["k_cont"][t0:t1]), "v_cont": digest(r["v_cont"][t0:t1]),
        "k_so": digest(r["k_so"][t0:t1].view(np.uint16)), "v_so": digest(r["v_so"][t0:t1].view(np.uint16)),
        "k_mean_q": digest(r["k_mean_q"][w0:w1]),
        "k_mean_scale": digest(r["k_mean_scale"][w0:w1].view(np.uint16)),
    }


def main():
    w = synth.WORKLOADS["gqa"]
    ck, cv = w.containers[0]
    p = O.OracleParams(w.n_kv_heads, w.head_dim, 8, 6, ck, cv, 128, 1.4)
    out = {"workload": "gqa", "containers": [ck, cv], "levels": [8, 6],
           "seq_full": SEQ_FULL, "seq_window": SEQ_WINDOW}
    t = time.time()
    k, v = synth.sequence_kv(w, SEQ_FULL, "cpu")
    r = encode_cache_parallel(k.float().numpy(), v.float().numpy(), p)
    print(f"encoded sequence {SEQ_FULL} in {time.time() - t:.0f} s", flush=True)
    out["full"] = encoded_digests(r, 0, w.seq_len, 0, w.seq_len // 128)
    out["full"]["stats"] = r["stats"].tolist()
    q = synth.queries(w, "cpu", [SEQ_FULL])[0].float().numpy().astype(np.float64)
    mu_tok = np.repeat(r["mu_hat"], p.mean_window, axis=0)
    ref = O.attention_factored_f64(q, r["k_sym"], r["k_so"], mu_tok, r["v_sym"], r["v_so"],
                                   p.n_kv_heads, p.head_dim)
    out["attention_f64"] = [[float(x) for x in row] for row in ref]
    k0, v0 = synth.sequence_kv(w, SEQ_WINDOW, "cpu", (0, 128))
    r0 = O.encode_cache(k0.float().numpy(), v0.float().numpy(), p)
    out["window0"] = encoded_digests(r0, 0, 128, 0, 1)
    out["window0"]["stats"] = r0["stats"].tolist()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gqa_fullsize_expected.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
