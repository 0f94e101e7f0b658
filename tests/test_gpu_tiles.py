"""The tile layout of the container arrays (KVQ_LAYOUT_TILES) on the GPU.

A stream's container is the same C bytes in either layout; only its place in
the cache array differs (dword k of a 64-token tile's containers side by
side).  For golden cases of tests/golden/cases.py (written by the oracle
alone, see test_gpu_parity.py) the test encodes with the tile layout and
requires:
  * the containers, read back as rows, the fp16 (scale, offset) bits and the
    INT8 key means to match the oracle's digests, and kvq_decode_symbols on
    the tile-layout array to return the oracle's symbols with every stream
    ending at the start state;
  * decode attention over the tile-layout cache to be bit-identical to decode
    attention over the row-layout cache of the same inputs (the same symbols
    in the same order), fp32 and bf16, which test_gpu_parity.py checks
    against the oracle;
  * streaming append window by window to write exactly the bytes of one
    whole-sequence encode, and attention over a compressed prefix plus a bf16
    tail to match the row layout bit for bit.
"""

import json

import numpy as np
import pytest
import torch

from kv_cache_entropy_amd import synth
from tests.golden import cases as C

pytestmark = pytest.mark.gpu

CASES = ["tiny", "gqa_s0_s511_t0", "heavy_b200_s0_s7_t0", "layout8x1", "layout2x2", "layout4x4_m16_2",
         "window64", "window256", "levels_8_6", "degenerate", "verylong_t0_1024", "verylong_t0_8320"]
FULL = ["heavy_full_b200", "verylong_full"]


def _kvq():
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return kvq


def say(*a):
    print(*a, flush=True)


def plan_of(kvq, case, layout):
    w = case["w"]
    ck, cv = C.containers(case)
    mk, mv = case["levels"]
    vk, vv = case["values"]
    return kvq.Plan(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, case["window"], 1.4, values_k=vk, values_v=vv,
                    layout=layout)


def encode(kvq, plan, k, v):
    S, T = int(k.shape[0]), int(k.shape[1])
    c = kvq.alloc_cache(plan, S, T)
    stats = torch.zeros(8, dtype=torch.int64, device="cuda")
    kvq.kvq_encode_streams(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"], c["k_mean_q"],
                           c["k_mean_scale"], stats=stats)
    torch.cuda.synchronize()
    return c, stats.cpu().tolist()


def attention(kvq, plan, q, c, Hq, scale, T):
    S = int(q.shape[0])
    ws = torch.empty(plan.workspace_bytes(1, S, T, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, Hq, plan.params.head_dim, dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty(S, Hq, plan.params.head_dim, dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention(plan, q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"], c["k_mean_q"],
                             c["k_mean_scale"], out, ws, out_f32=o32, softmax_scale=scale)
    torch.cuda.synchronize()
    return out, o32


def check_against_golden(kvq, plan, case, c, T, stats):
    g = json.load(open(C.golden_paths(case)[0]))
    for i, gs in enumerate(g["sequences"]):
        for key, side in (("k_cont", 0), ("v_cont", 1)):
            rows = kvq.container_rows(plan, side, c[key][i:i + 1], T)[0].cpu().numpy()
            assert C.digest(rows) == gs["digests"][key], f"{key} of sequence {gs['seq']} (tile layout)"
            # decode the tile-layout array directly
            cont = c[key][i:i + 1]
            n = int(cont.shape[1])
            sym = torch.empty(1, n, plan.n, dtype=torch.uint8, device="cuda")
            ok = torch.zeros(1, n, dtype=torch.int32, device="cuda")
            kvq.kvq_decode_symbols(plan, side, cont, sym, ok)
            torch.cuda.synchronize()
            assert int(ok[0, :T].sum()) == T, f"{key}: a stream does not end at the start state"
            assert C.digest(sym[0, :T].cpu().numpy()) == gs["digests"]["k_sym" if side == 0 else "v_sym"]
        for key in ("k_so", "v_so", "k_mean_scale"):
            assert C.digest(c[key][i].view(torch.int16).cpu().numpy()) == gs["digests"][key], key
        assert C.digest(c["k_mean_q"][i].cpu().numpy()) == gs["digests"]["k_mean_q"]
    assert stats == g["stats"], f"drift counters {stats} != oracle {g['stats']}"


def run(case_name):
    kvq = _kvq()
    case = C.BY_NAME[case_name]
    w = case["w"]
    say(f"tile layout: case {case_name} seqs={case['seqs']} tokens={case['tokens']}")
    k, v, q = C.cpu_inputs(case)
    T = int(k.shape[1])
    k, v, q = k.cuda(), v.cuda(), q.cuda()
    pt, pr = plan_of(kvq, case, kvq.KVQ_LAYOUT_TILES), plan_of(kvq, case, kvq.KVQ_LAYOUT_ROWS)
    ct, st = encode(kvq, pt, k, v)
    check_against_golden(kvq, pt, case, ct, T, st)
    say("  containers, metadata and symbols match the oracle")
    if not case["attention"]:
        return
    cr, _ = encode(kvq, pr, k, v)
    ot, ot32 = attention(kvq, pt, q, ct, w.n_q_heads, case["scale"], T)
    orow, orow32 = attention(kvq, pr, q, cr, w.n_q_heads, case["scale"], T)
    assert torch.equal(ot32.view(torch.int32), orow32.view(torch.int32)), "fp32 attention differs between layouts"
    assert torch.equal(ot.view(torch.int16), orow.view(torch.int16)), "bf16 attention differs between layouts"
    say("  attention bit-identical to the row layout")


@pytest.mark.parametrize("name", CASES)
def test_tile_layout(name):
    run(name)


@pytest.mark.parametrize("name", FULL)
def test_tile_layout_whole_sequences(name):
    run(name)


def test_tile_layout_append_and_tail():
    kvq = _kvq()
    w = synth.WORKLOADS["gqa"]
    S, T, W, cap = 2, 512, 128, 1024
    k, v = synth.cache_inputs(w, "cuda", [3, 4], (0, T))
    q = synth.queries(w, "cuda", [3, 4])
    say(f"tile layout: append {T // W} windows into capacity {cap}, then a bf16 tail")
    pt = kvq.Plan(8, 128, 8, 6, 331, 231, W, 1.4, layout=kvq.KVQ_LAYOUT_TILES)
    pr = kvq.Plan(8, 128, 8, 6, 331, 231, W, 1.4)
    whole, _ = encode(kvq, pt, k, v)
    app = kvq.alloc_cache(pt, S, cap)
    for key in app:
        app[key].zero_()
    for t0 in range(0, T, W):
        kvq.kvq_encode_append(pt, k[:, t0:t0 + W].contiguous(), v[:, t0:t0 + W].contiguous(), app, t0)
    torch.cuda.synchronize()
    for key, side in (("k_cont", 0), ("v_cont", 1)):
        assert torch.equal(kvq.container_rows(pt, side, app[key], T), kvq.container_rows(pt, side, whole[key], T))
    for key in ("k_so", "v_so"):
        assert torch.equal(app[key][:, :T], whole[key])
    # a prefix of 384 compressed tokens plus a 100-token bf16 tail, both layouts
    rows_app = kvq.alloc_cache(pr, S, cap)
    for t0 in range(0, T, W):
        kvq.kvq_encode_append(pr, k[:, t0:t0 + W].contiguous(), v[:, t0:t0 + W].contiguous(), rows_app, t0)
    tail_k = k[:, 384:484].contiguous()
    tail_v = v[:, 384:484].contiguous()
    outs = []
    for plan, cache in ((pt, app), (pr, rows_app)):
        ws = torch.empty(plan.workspace_bytes(1, S, 384, w.n_q_heads), dtype=torch.uint8, device="cuda")
        out = torch.empty(S, w.n_q_heads, 128, dtype=torch.bfloat16, device="cuda")
        kvq.kvq_decode_attention_ex(plan, q, cache, 384, tail_k, tail_v, 100, out, ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    say("  append bit-identical to a whole encode; prefix + tail attention equal to the row layout")


def test_tile_layout_rejects_what_reads_rows_only():
    kvq = _kvq()
    pt = kvq.Plan(8, 128, 8, 9, 331, 231, 128, 1.4, layout=kvq.KVQ_LAYOUT_TILES)   # 9 V levels
    w = synth.WORKLOADS["gqa"]
    k, v = synth.cache_inputs(w, "cuda", [0], (0, 128))
    q = synth.queries(w, "cuda", [0])
    c, _ = encode(kvq, pt, k, v)
    with pytest.raises(kvq.KvqError) as e:
        attention(kvq, pt, q, c, 32, 0.0, 128)
    assert e.value.status == -3
