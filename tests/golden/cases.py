"""Parity cases shared by the golden writer and the GPU tests.

Each case names a seeded synthetic workload (kv_cache_entropy_amd.synth), a
budget, the sequences and token range it covers, the alphabet and key-mean
window, an optional deterministic edit of the inputs and the softmax scale.
Inputs of the sequences a golden covers are always generated on the CPU, so
that make_parity_goldens.py (which calls only oracle/) and the GPU tests see
the same values.  This module holds no arithmetic of the method: input
generation, edits and SHA-256 digests only.

Full-size cases ("launch" set) run in the shape the benchmark times: the GPU
test builds the whole cache (sequences outside the golden are generated on
the GPU) and checks the golden's sequences inside it.
"""

import hashlib
import os

import numpy as np
import torch

from kv_cache_entropy_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
PARITY_DIR = os.path.join(HERE, "parity")
INPUTS_PATH = os.path.join(PARITY_DIR, "inputs.json")
CHUNK_TOKENS = 1024          # container digests are also kept per chunk of this many tokens


def _layout(hq, hkv, cont):
    return synth.Workload(f"layout{hq}x{hkv}", hq, hkv, 128, 2, 1, 640, 11 + hq + hkv, "keymeans",
                          (cont,), (0.0,))


def _window(window, tokens):
    return synth.Workload(f"window{window}", 32, 8, 128, 2, 1, tokens, 53 + window // 64, "keymeans",
                          ((331, 231),), (0.0,))


def _dims(hkv, d, cont):
    return synth.Workload(f"dim{d}", hkv, hkv, d, 2, 1, 256, 61 + d, "keymeans", (cont,), (0.0,))


def _levels(cont):
    return synth.Workload("levels", 32, 8, 128, 2, 1, 640, 41, "keymeans", (cont,), (0.0,))


def _case(name, workload, bi=0, seqs=(0,), tokens=None, levels=(8, 6), values=(None, None), window=128,
          mutate=None, scale=0.0, attention=True, launch=False):
    w = synth.WORKLOADS[workload] if isinstance(workload, str) else workload
    return dict(name=name, w=w, bi=bi, seqs=list(seqs), tokens=tokens, levels=levels, values=values,
                window=window, mutate=mutate, scale=scale, attention=attention, launch=launch)


NONAFFINE = [
    ((8, 6), ((0.0, 0.75, 1.875, 3.0, 4.0, 5.125, 6.25, 7.0), (0.0, 0.875, 2.125, 2.875, 4.125, 5.0)),
     (331, 231)),
    ((12, 4), ((0.0, 0.5, 1.25, 2.5, 3.75, 5.0, 6.0, 7.25, 8.5, 9.75, 10.5, 11.0), (0.0, 0.625, 2.0, 3.0)),
     (380, 190)),
]

REDUCED = [
    _case("tiny", "tiny"),
    _case("gqa_s0_s511_t0", "gqa", 0, (0, 511), (0, 512)),
    _case("long_b200_s0_s127_t0", "long", 0, (0, 127), (0, 512)),
    _case("long_b226_s0_t1024", "long", 1, (0,), (1024, 1536)),
    _case("long_b300_s5_t0", "long", 2, (5,), (0, 512)),
    _case("verylong_t0_1024", "verylong", 0, (0,), (0, 1024)),
    # 130 one-tile splits: the two-pass combine (groups of 64, 64 and 2), 65 key-mean windows
    _case("verylong_t0_8320", "verylong", 0, (0,), (0, 8320)),
    _case("heavy_b200_s0_s7_t0", "heavy", 0, (0, 7), (0, 512)),
    _case("heavy_b300_s3_t0", "heavy", 1, (3,), (0, 512)),
    _case("heavy_b400_s6_t512", "heavy", 2, (6,), (512, 1024)),
    # a softmax scale other than 1/sqrt(d)
    _case("heavy_b200_s1_scale005", "heavy", 0, (1,), (0, 512), scale=0.05),
    _case("gqa_s2_scale025", "gqa", 0, (2,), (0, 256), scale=0.25),
    # other head layouts and alphabets
    _case("layout8x4", _layout(8, 4, (180, 130)), 0, (0, 1)),          # 2 query heads per KV head
    _case("layout2x2", _layout(2, 2, (100, 70)), 0, (0, 1)),           # 1 query head per KV head
    _case("layout8x1", _layout(8, 1, (48, 36)), 0, (0, 1)),            # 8 query heads on one KV head
    _case("layout8x2_v9", _layout(8, 2, (96, 90)), 0, (0, 1), levels=(8, 9)),   # 9 V levels
    _case("layout4x4_m6_4", _layout(4, 4, (150, 100)), 0, (0, 1), levels=(6, 4)),
    # alphabet extremes: 16 key levels (drift without the register cache), 2 value
    # levels with the budget met exactly
    _case("layout4x4_m16_2", _layout(4, 4, (220, 68)), 0, (0, 1), levels=(16, 2)),
    # key-mean windows of 64 tokens (one per tile) and 256 (four tiles per window)
    _case("window64", _window(64, 640), 0, (0, 1), window=64),
    _case("window256", _window(256, 768), 0, (0, 1), window=256),
    # write side at head dimensions 32, 64 and 256 (the attention reports KVQ_EUNSUPPORTED)
    _case("dim32", _dims(2, 32, (24, 18)), 0, (0, 1), attention=False),
    _case("dim64", _dims(4, 64, (80, 56)), 0, (0, 1), attention=False),
    _case("dim256", _dims(2, 256, (160, 112)), 0, (0, 1), attention=False),
    # non-affine reconstruction levels
    _case("levels_8_6", _levels(NONAFFINE[0][2]), 0, (0, 1), levels=NONAFFINE[0][0], values=NONAFFINE[0][1]),
    _case("levels_12_4", _levels(NONAFFINE[1][2]), 0, (0, 1), levels=NONAFFINE[1][0], values=NONAFFINE[1][1]),
    # streams the method treats specially (see _mutate_degenerate)
    _case("degenerate", "gqa", 0, (0, 1), (0, 512), mutate="degenerate"),
]

LAUNCH = [
    # whole sequences in the benchmark's launch shapes
    _case("verylong_full", "verylong", 0, (0,), launch=True),
    _case("heavy_full_b200", "heavy", 0, range(8), launch=True),
    _case("heavy_full_b300", "heavy", 1, range(8), launch=True),
    _case("heavy_full_b400", "heavy", 2, range(8), launch=True),
    _case("long_full_b200_s0", "long", 0, (0,), launch=True),
    _case("long_full_b226_s0", "long", 1, (0,), launch=True),
    _case("long_full_b300_s0", "long", 2, (0,), launch=True),
]

ALL = REDUCED + LAUNCH
BY_NAME = {c["name"]: c for c in ALL}


def _mutate_degenerate(k, v):
    """* an all-zero key and value window (sequence 0, tokens 128..255): the key
       mean is 0, every stream is constant, s = 0 and drift keeps the cheapest
       symbol;
    * isolated zero value tokens;
    * a token 1000 times its neighbours (its own grid; it dominates its
      key-mean window and, through its logits, the softmax);
    * a key token equal to one number everywhere (one non-zero coefficient per
      head after the rotation)."""
    k[0, 128:256] = 0
    v[0, 128:256] = 0
    v[1, 5] = 0
    v[1, 300:310] = 0
    k[1, 17] *= 1000
    v[1, 17] *= 1000
    k[0, 400] = 3.0


MUTATIONS = {"degenerate": _mutate_degenerate}


def containers(case):
    return case["w"].containers[case["bi"]]


def cpu_inputs(case):
    """K, V [S', T', n] and q [S', Hq, d] of the case's sequences, on the CPU."""
    w = case["w"]
    k, v = synth.cache_inputs(w, "cpu", case["seqs"], case["tokens"])
    if case["mutate"]:
        MUTATIONS[case["mutate"]](k, v)
    q = synth.queries(w, "cpu", case["seqs"])
    return k, v, q


def input_digest(t):
    t = t.contiguous()
    return digest(t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy())


def digest(a):
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.tobytes()).hexdigest()


def golden_paths(case):
    return (os.path.join(PARITY_DIR, case["name"] + ".json"),
            os.path.join(PARITY_DIR, case["name"] + "_attention.npy"))
