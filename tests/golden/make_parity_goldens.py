"""Writes tests/golden/parity/<case>.json (+ <case>_attention.npy) by calling
only oracle/.

For every case in tests/golden/cases.py, the oracle encodes each covered
sequence (inputs from the seeded CPU generators), and the file records
SHA-256 digests of every bit-exact surface per sequence: containers, fp16
(scale, offset) bits, INT8 key means and their fp16 scales, and the encoder's
symbols (which decoding a container must return), plus container digests per
chunk of 1024 tokens, the drift counters and the float64 attention output of
each sequence's decode query.  Run from the repository root:

    python tests/golden/make_parity_goldens.py [case names ...]

(all cases: about ten minutes on eight cores), and

    python tests/golden/make_parity_goldens.py --inputs

for the digests of every case's inputs (tests/golden/parity/inputs.json).
"""

import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from tests.golden import cases as C  # noqa: E402
from tests.oracle_pool import encode_cache_parallel  # noqa: E402


def oracle_params(case):
    w = case["w"]
    ck, cv = C.containers(case)
    mk, mv = case["levels"]
    vk, vv = case["values"]
    return O.OracleParams(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, case["window"], 1.4,
                          values_k=vk, values_v=vv)


def surfaces(r):
    return {
        "k_cont": r["k_cont"], "v_cont": r["v_cont"],
        "k_so": r["k_so"].view(np.uint16), "v_so": r["v_so"].view(np.uint16),
        "k_mean_q": r["k_mean_q"], "k_mean_scale": r["k_mean_scale"].view(np.uint16),
        "k_sym": r["k_sym"].astype(np.uint8), "v_sym": r["v_sym"].astype(np.uint8),
    }


def compute(case, procs=None):
    """(record, attention array or None) of one case, from the oracle."""
    p = oracle_params(case)
    w = case["w"]
    k, v, q = C.cpu_inputs(case)
    seqs = []
    stats = np.zeros(8, np.uint64)
    attn = []
    for i, s in enumerate(case["seqs"]):
        r = encode_cache_parallel(k[i].float().numpy(), v[i].float().numpy(), p, procs=procs)
        stats += r["stats"].astype(np.uint64)
        surf = surfaces(r)
        T = r["k_cont"].shape[0]
        seqs.append({
            "seq": int(s),
            "digests": {key: C.digest(a) for key, a in surf.items()},
            "chunks": {key: [C.digest(surf[key][t:t + C.CHUNK_TOKENS]) for t in range(0, T, C.CHUNK_TOKENS)]
                       for key in ("k_cont", "v_cont")},
        })
        if case["attention"]:
            mu_tok = np.repeat(r["mu_hat"], p.mean_window, axis=0)
            kv = None if p.values_k is None else p.vals("k")
            vv = None if p.values_v is None else p.vals("v")
            attn.append(O.attention_factored_f64(
                q[i].float().numpy().astype(np.float64), r["k_sym"], r["k_so"], mu_tok, r["v_sym"],
                r["v_so"], p.n_kv_heads, p.head_dim, scale=case["scale"] or None, k_vals=kv, v_vals=vv))
    ck, cv = C.containers(case)
    rec = {"case": case["name"], "workload": w.name, "containers": [ck, cv], "levels": list(case["levels"]),
           "window": case["window"], "tokens": case["tokens"], "seqs": case["seqs"],
           "softmax_scale": case["scale"], "launch": case["launch"],
           "stats": [int(x) for x in stats], "sequences": seqs}
    return rec, (np.stack(attn) if attn else None)


def make(case):
    rec, attn = compute(case)
    jpath, apath = C.golden_paths(case)
    os.makedirs(C.PARITY_DIR, exist_ok=True)
    with open(jpath, "w") as fh:
        json.dump(rec, fh, indent=0)
    if attn is not None:
        np.save(apath, attn)
    elif os.path.exists(apath):
        os.remove(apath)


def input_digests():
    """SHA-256 of every case's CPU-generated inputs (K, V, q as bf16/fp32 bits):
    the GPU tests check them first, so that a host whose CPU generator gives
    other bits is reported as such rather than as a kernel mismatch."""
    out = {}
    for case in C.ALL:
        k, v, q = C.cpu_inputs(case)
        out[case["name"]] = {key: C.input_digest(t) for key, t in (("k", k), ("v", v), ("q", q))}
    with open(C.INPUTS_PATH, "w") as fh:
        json.dump(out, fh, indent=0)


def main():
    if sys.argv[1:] == ["--inputs"]:
        input_digests()
        return
    names = sys.argv[1:] or [c["name"] for c in C.ALL]
    for name in names:
        t = time.time()
        make(C.BY_NAME[name])
        print(f"{name}: {time.time() - t:.1f} s", flush=True)


if __name__ == "__main__":
    main()
