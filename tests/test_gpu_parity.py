"""GPU parity of the HIP path against the oracle on the same seeded inputs.

Containers, (scale, offset) metadata, INT8 key means, decoded symbols and the
drift counters must be bit-identical; decode attention must be within 2e-3 of
the float64 reference row-normwise on the fp32 output, and the bf16 output
must be the round-to-nearest-even of the fp32 one.  The oracle encodes the
inputs itself: nothing the GPU produced is ever fed to it."""

import os

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_entropy_amd import synth
from tests.oracle_pool import encode_cache_parallel

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _kvq():
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return kvq


def say(*a):
    print(*a, flush=True)


def gpu_encode(kvq, plan, k, v):
    S, T = int(k.shape[0]), int(k.shape[1])
    c = kvq.alloc_cache(plan, S, T)
    stats = torch.zeros(8, dtype=torch.int64, device="cuda")
    kvq.kvq_encode_streams(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                           c["k_mean_q"], c["k_mean_scale"], stats=stats)
    torch.cuda.synchronize()
    return c, stats


def gpu_attention(kvq, plan, q, c, Hq):
    S, T = int(c["k_cont"].shape[0]), int(c["k_cont"].shape[1])
    ws = torch.empty(plan.workspace_bytes(1, S, T, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, Hq, plan.params.head_dim, dtype=torch.bfloat16, device="cuda")
    out32 = torch.empty(S, Hq, plan.params.head_dim, dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention(plan, q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                             c["k_mean_q"], c["k_mean_scale"], out, ws, out_f32=out32)
    torch.cuda.synchronize()
    return out, out32


def oracle_attention(q, r, p):
    mu_tok = np.repeat(r["mu_hat"], p.mean_window, axis=0)
    kv = None if p.values_k is None else p.vals("k")
    vv = None if p.values_v is None else p.vals("v")
    return O.attention_factored_f64(q.astype(np.float64), r["k_sym"], r["k_so"], mu_tok,
                                    r["v_sym"], r["v_so"], p.n_kv_heads, p.head_dim,
                                    k_vals=kv, v_vals=vv)


def check_attention(out, out32, ref):
    o32 = out32.cpu().numpy().astype(np.float64)
    err = (np.abs(o32 - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max()
    assert err <= TOL, f"attention row-normwise error {err:.3e} > {TOL}"
    rne = out32.cpu().to(torch.bfloat16).view(torch.int16)
    assert torch.equal(rne, out.cpu().view(torch.int16))
    return err


def compare_cache(c, stats, refs, p, S):
    """refs: per-sequence oracle results; c: GPU cache tensors."""
    for s in range(S):
        r = refs[s]
        for key in ("k_cont", "v_cont", "k_mean_q"):
            got = c[key][s].cpu().numpy().view(np.uint8 if key != "k_mean_q" else np.int8)
            assert np.array_equal(got, r[key]), f"{key} differs in sequence {s}"
        for key in ("k_so", "v_so"):
            got = c[key][s].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, r[key].view(np.uint16)), f"{key} differs in sequence {s}"
        got = c["k_mean_scale"][s].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, r["k_mean_scale"].view(np.uint16))
    tot = np.sum([refs[s]["stats"] for s in range(S)], axis=0)
    assert stats.cpu().numpy().astype(np.uint64).tolist() == tot.tolist()


def run_case(name, budget_idx, seqs, tokens, w=None, levels=(8, 6), values=(None, None), mutate=None,
             window=128):
    kvq = _kvq()
    w = w or synth.WORKLOADS[name]
    ck, cv = w.containers[budget_idx]
    mk, mv = levels
    say(f"case {w.name} budget={w.budgets[budget_idx]} C=({ck},{cv}) M=({mk},{mv}) "
        f"heads={w.n_q_heads}/{w.n_kv_heads} seqs={seqs} tokens={tokens} W={window}")
    plan = kvq.Plan(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, window, 1.4, values_k=values[0], values_v=values[1])
    p = O.OracleParams(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, window, 1.4, values_k=values[0],
                       values_v=values[1])
    k, v = synth.cache_inputs(w, "cuda", seqs, tokens)
    if mutate is not None:
        mutate(k, v)
    q = synth.queries(w, "cuda", seqs)
    c, stats = gpu_encode(kvq, plan, k, v)
    say("  gpu encode done")
    refs = [encode_cache_parallel(k[s].float().cpu().numpy(), v[s].float().cpu().numpy(), p)
            for s in range(len(seqs))]
    say("  oracle encode done")
    compare_cache(c, stats, refs, p, len(seqs))
    # decoded symbols
    for side, key, sk in ((0, "k_cont", "k_sym"), (1, "v_cont", "v_sym")):
        sym = torch.empty(*c[key].shape[:2], p.n, dtype=torch.uint8, device="cuda")
        ok = torch.zeros(*c[key].shape[:2], dtype=torch.int32, device="cuda")
        kvq.kvq_decode_symbols(plan, side, c[key], sym, ok)
        torch.cuda.synchronize()
        assert int(ok.sum()) == ok.numel()
        for s in range(len(seqs)):
            assert np.array_equal(sym[s].cpu().numpy(), refs[s][sk])
    out, out32 = gpu_attention(kvq, plan, q, c, w.n_q_heads)
    ref = np.stack([oracle_attention(q[s].float().cpu().numpy(), refs[s], p) for s in range(len(seqs))])
    err = check_attention(out, out32, ref)
    say(f"  attention max row-normwise error {err:.3e}")


def test_tiny_full():
    run_case("tiny", 0, [0], None)


@pytest.mark.parametrize("name,bi,seqs,tokens", [
    ("gqa", 0, [0, 511], (0, 512)),
    ("long", 0, [0, 127], (0, 512)),
    ("long", 1, [0], (1024, 1536)),
    ("long", 2, [5], (0, 512)),
    ("verylong", 0, [0], (0, 1024)),
    ("verylong", 0, [0], (0, 8320)),    # 130 one-tile splits: two-pass combine (groups of 64, 64, 2), 65 windows
    ("heavy", 0, [0, 7], (0, 512)),
    ("heavy", 1, [3], (0, 512)),
    ("heavy", 2, [6], (512, 1024)),
])
def test_reduced_configs(name, bi, seqs, tokens):
    run_case(name, bi, seqs, tokens)


@pytest.mark.parametrize("hq,hkv,levels,cont", [
    (8, 4, (8, 6), (180, 130)),      # 2 query heads per KV head
    (2, 2, (8, 6), (100, 70)),       # one query head per KV head, two KV heads
    (8, 1, (8, 6), (48, 36)),        # 8 query heads on one KV head (two MFMA groups)
    (8, 2, (8, 9), (96, 90)),        # 9 V levels: the non-interleaved kernel
    (4, 4, (6, 4), (150, 100)),      # other alphabets
    (4, 4, (16, 2), (220, 68)),      # alphabet extremes: 16 key levels (drift without the
                                     # register cache), 2 value levels with the budget met exactly
])
def test_other_head_layouts_and_alphabets(hq, hkv, levels, cont):
    w = synth.Workload(f"layout{hq}x{hkv}", hq, hkv, 128, 2, 1, 640, 11 + hq + hkv, "keymeans",
                       (cont,), (0.0,))
    run_case(None, 0, [0, 1], None, w=w, levels=levels)


@pytest.mark.parametrize("window,tokens", [(64, 640), (256, 768)])
def test_other_key_mean_windows(window, tokens):
    # one key mean per window of W tokens ([D-Quant] §4.5): W = 64, the smallest the
    # attention takes (one window per tile), and W = 256 (four tiles per window)
    w = synth.Workload(f"window{window}", 32, 8, 128, 2, 1, tokens, 53 + window // 64, "keymeans",
                       ((331, 231),), (0.0,))
    run_case(None, 0, [0, 1], None, w=w, window=window)


@pytest.mark.parametrize("hkv,d,cont", [(2, 32, (24, 18)), (4, 64, (80, 56)), (2, 256, (160, 112))])
def test_encode_other_head_dims(hkv, d, cont):
    """The write side at head dimensions other than 128 (the plan takes powers of
    two from 32 to 256): containers, metadata, key means, drift counters and
    decoded symbols bit-exact.  The decode attention is built for d = 128 and
    reports KVQ_EUNSUPPORTED for these plans without launching anything."""
    kvq = _kvq()
    say(f"case head_dim={d} kv_heads={hkv} C={cont}")
    w = synth.Workload(f"dim{d}", hkv, hkv, d, 2, 1, 256, 61 + d, "keymeans", (cont,), (0.0,))
    plan = kvq.Plan(hkv, d, 8, 6, cont[0], cont[1], 128, 1.4)
    p = O.OracleParams(hkv, d, 8, 6, cont[0], cont[1], 128, 1.4)
    k, v = synth.cache_inputs(w, "cuda", [0, 1], None)
    c, stats = gpu_encode(kvq, plan, k, v)
    refs = [encode_cache_parallel(k[s].float().cpu().numpy(), v[s].float().cpu().numpy(), p) for s in range(2)]
    compare_cache(c, stats, refs, p, 2)
    for side, key, sk in ((0, "k_cont", "k_sym"), (1, "v_cont", "v_sym")):
        sym = torch.empty(*c[key].shape[:2], p.n, dtype=torch.uint8, device="cuda")
        ok = torch.zeros(*c[key].shape[:2], dtype=torch.int32, device="cuda")
        kvq.kvq_decode_symbols(plan, side, c[key], sym, ok)
        torch.cuda.synchronize()
        assert int(ok.sum()) == ok.numel()
        for s in range(2):
            assert np.array_equal(sym[s].cpu().numpy(), refs[s][sk])
    q = synth.queries(w, "cuda", [0, 1])
    with pytest.raises(kvq.KvqError) as e:
        gpu_attention(kvq, plan, q, c, hkv)
    assert e.value.status == -3


def test_encode_is_deterministic():
    kvq = _kvq()
    w = synth.WORKLOADS["heavy"]
    plan = kvq.Plan(8, 128, 8, 6, 292, 203, 128, 1.4)
    k, v = synth.cache_inputs(w, "cuda", [1], (0, 1024))
    a, sa = gpu_encode(kvq, plan, k, v)
    b, sb = gpu_encode(kvq, plan, k, v)
    for key in a:
        assert torch.equal(a[key], b[key])
    assert torch.equal(sa, sb)


@pytest.mark.parametrize("levels,values,cont", [
    ((8, 6), ((0.0, 0.75, 1.875, 3.0, 4.0, 5.125, 6.25, 7.0), (0.0, 0.875, 2.125, 2.875, 4.125, 5.0)),
     (331, 231)),
    ((12, 4), ((0.0, 0.5, 1.25, 2.5, 3.75, 5.0, 6.0, 7.25, 8.5, 9.75, 10.5, 11.0), (0.0, 0.625, 2.0, 3.0)),
     (380, 190)),
])
def test_non_affine_levels(levels, values, cont):
    # [D-Quant] Appendix A: table entries carry arbitrary reconstruction levels
    w = synth.Workload("levels", 32, 8, 128, 2, 1, 640, 41, "keymeans", (cont,), (0.0,))
    run_case(None, 0, [0, 1], None, w=w, levels=levels, values=values)


def test_degenerate_streams():
    """Streams the method treats specially, on the gqa layout:
    * an all-zero key and value window: the key mean is 0, so every stream in it
      is constant, its grid has s = 0 and drift keeps the cheapest symbol;
    * isolated zero value tokens;
    * a token 1000 times larger than its neighbours (its own grid; it dominates
      its key-mean window and, through its logits, the softmax);
    * a key token equal to one number everywhere (a single non-zero coefficient
      per head after the rotation)."""
    def mutate(k, v):
        k[0, 128:256] = 0
        v[0, 128:256] = 0
        v[1, 5] = 0
        v[1, 300:310] = 0
        k[1, 17] *= 1000
        v[1, 17] *= 1000
        k[0, 400] = 3.0
    run_case("gqa", 0, [0, 1], (0, 512), mutate=mutate)
