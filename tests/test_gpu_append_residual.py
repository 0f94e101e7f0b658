"""Streaming append and the uncompressed residual tail on the GPU, against the oracle.

[D-Quant] §5.1 "Implementation details": the most recent tokens stay in BF16.
A cache with spare capacity is filled window by window with kvq_encode_append;
the appended rows must be bit-identical to the oracle's encoding of those
tokens, and rows beyond them untouched.  kvq_decode_attention_ex then attends
over the compressed prefix plus a bf16 tail of 0..200 tokens and must be within
2e-3 (row-normwise, fp32 output) of the oracle's float64 attention over the
dequantised prefix followed by the raw tail.
"""

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_entropy_amd import synth
from tests.oracle_pool import encode_cache_parallel

pytestmark = pytest.mark.gpu
TOL = 2e-3
CAP = 1024
ENC = 640          # tokens appended (5 windows)
SENTINEL = 0xA5


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def appended():
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = synth.WORKLOADS["gqa"]
    seqs = [0, 511]
    k, v = synth.cache_inputs(w, "cuda", seqs, (0, ENC + 256))
    plan = kvq.Plan(w.n_kv_heads, w.head_dim, 8, 6, 331, 231, 128, 1.4)
    c = kvq.alloc_cache(plan, len(seqs), CAP)
    for key in c:
        c[key].view(torch.uint8).fill_(SENTINEL)
    stats = torch.zeros(8, dtype=torch.int64, device="cuda")
    say(f"case append: seqs={seqs} windows [0,128) [128,384) [384,640) into capacity {CAP}")
    for t0, t1 in ((0, 128), (128, 384), (384, ENC)):
        kvq.kvq_encode_append(plan, k[:, t0:t1].contiguous(), v[:, t0:t1].contiguous(), c, t0, stats=stats)
    torch.cuda.synchronize()
    p = O.OracleParams(w.n_kv_heads, w.head_dim, 8, 6, 331, 231, 128, 1.4)
    refs = [encode_cache_parallel(k[i, :ENC].float().cpu().numpy(), v[i, :ENC].float().cpu().numpy(), p)
            for i in range(len(seqs))]
    say("  oracle encode done")
    q = synth.queries(w, "cuda", seqs)
    return dict(kvq=kvq, w=w, plan=plan, p=p, c=c, k=k, v=v, q=q, refs=refs, stats=stats)


def test_append_matches_oracle_and_leaves_other_rows(appended):
    A = appended
    c, refs = A["c"], A["refs"]
    for i, r in enumerate(refs):
        assert np.array_equal(c["k_cont"][i, :ENC].cpu().numpy(), r["k_cont"])
        assert np.array_equal(c["v_cont"][i, :ENC].cpu().numpy(), r["v_cont"])
        assert np.array_equal(c["k_so"][i, :ENC].cpu().numpy().view(np.uint16), r["k_so"].view(np.uint16))
        assert np.array_equal(c["v_so"][i, :ENC].cpu().numpy().view(np.uint16), r["v_so"].view(np.uint16))
        nw = ENC // 128
        assert np.array_equal(c["k_mean_q"][i, :nw].cpu().numpy(), r["k_mean_q"])
        assert np.array_equal(c["k_mean_scale"][i, :nw].cpu().numpy().view(np.uint16),
                              r["k_mean_scale"].view(np.uint16))
        for key, rows in (("k_cont", ENC), ("v_cont", ENC), ("k_so", ENC), ("v_so", ENC),
                          ("k_mean_q", nw), ("k_mean_scale", nw)):
            rest = c[key][i, rows:].contiguous().view(torch.uint8)
            assert bool((rest == SENTINEL).all()), f"{key} rows past the appended tokens changed"
    tot = np.sum([r["stats"] for r in refs], axis=0)
    assert A["stats"].cpu().numpy().astype(np.uint64).tolist() == tot.tolist()


def test_append_equals_whole_sequence_encode(appended):
    A = appended
    kvq = A["kvq"]
    w = A["w"]
    c2 = kvq.alloc_cache(A["plan"], 2, ENC)
    kvq.kvq_encode_streams(A["plan"], A["k"][:, :ENC].contiguous(), A["v"][:, :ENC].contiguous(),
                           c2["k_cont"], c2["v_cont"], c2["k_so"], c2["v_so"], c2["k_mean_q"],
                           c2["k_mean_scale"])
    torch.cuda.synchronize()
    for key in c2:
        rows = c2[key].shape[1]
        assert torch.equal(A["c"][key][:, :rows], c2[key]), key


@pytest.mark.parametrize("n_tok,res_len", [(512, 0), (512, 1), (512, 37), (512, 127), (384, 200),
                                           (128, 64), (0, 100), (0, 1)])
def test_attention_with_residual(appended, n_tok, res_len):
    A = appended
    kvq, w, p = A["kvq"], A["w"], A["p"]
    S, d, Hq = 2, w.head_dim, w.n_q_heads
    say(f"case residual: compressed {n_tok} tokens (capacity {CAP}), bf16 tail {res_len}")
    RCAP = 256
    rk = torch.zeros(S, RCAP, w.n, dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    rk[:, :res_len] = A["k"][:, n_tok:n_tok + res_len]
    rv[:, :res_len] = A["v"][:, n_tok:n_tok + res_len]
    ws = torch.empty(A["plan"].workspace_bytes(1, S, n_tok, Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, Hq, d, dtype=torch.bfloat16, device="cuda")
    out32 = torch.empty(S, Hq, d, dtype=torch.float32, device="cuda")
    cache = A["c"] if n_tok > 0 else None
    kvq.kvq_decode_attention_ex(A["plan"], A["q"], cache, n_tok, rk if res_len else None,
                                rv if res_len else None, res_len, out, ws, out_f32=out32)
    torch.cuda.synchronize()
    errs = []
    for i, r in enumerate(A["refs"]):
        mu_tok = np.repeat(r["mu_hat"], p.mean_window, axis=0)[:n_tok]
        kh = O.dequantize_f64(r["k_sym"][:n_tok], r["k_so"][:n_tok], mu_tok)
        vh = O.dequantize_f64(r["v_sym"][:n_tok], r["v_so"][:n_tok])
        tk = A["k"][i, n_tok:n_tok + res_len].float().cpu().numpy()
        tv = A["v"][i, n_tok:n_tok + res_len].float().cpu().numpy()
        ref = O.attention_with_residual_f64(A["q"][i].float().cpu().numpy(), kh, vh, tk, tv,
                                            w.n_kv_heads, d)
        o32 = out32[i].cpu().numpy().astype(np.float64)
        errs.append((np.abs(o32 - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())
    err = max(errs)
    say(f"  max row-normwise error {err:.3e}")
    assert err <= TOL
    assert torch.equal(out32.cpu().to(torch.bfloat16).view(torch.int16), out.cpu().view(torch.int16))


@pytest.mark.parametrize("hkv,hq,res_len", [(8, 8, 70), (4, 8, 129), (8, 64, 100), (2, 16, 1), (1, 4, 64)])
def test_residual_only_head_layouts(hkv, hq, res_len):
    """A bf16 tail with no compressed prefix, for 1, 2, 4 and 8 query heads per
    KV head: the tail kernel's logits, softmax and value sums against the
    oracle's float64 attention over the raw tail."""
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d, S, RCAP = 128, 3, 160
    n = hkv * d
    say(f"case residual only: Hkv={hkv} Hq={hq} tail {res_len}")
    g = torch.Generator().manual_seed(1000 * hkv + hq + res_len)
    q = (torch.randn(S, hq, d, generator=g) * 0.5).to(torch.bfloat16)
    rk = torch.zeros(S, RCAP, n, dtype=torch.bfloat16)
    rv = torch.zeros(S, RCAP, n, dtype=torch.bfloat16)
    rk[:, :res_len] = (torch.randn(S, res_len, n, generator=g) * 0.7).to(torch.bfloat16)
    rv[:, :res_len] = torch.randn(S, res_len, n, generator=g).to(torch.bfloat16)
    ck = max(36, (n * 9) // 32)
    cv = max(36, (n * 7) // 32)
    plan = kvq.Plan(hkv, d, 8, 6, ck, cv, 128, 1.4)
    ws = torch.empty(plan.workspace_bytes(1, S, 0, hq), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, hq, d, dtype=torch.bfloat16, device="cuda")
    out32 = torch.empty(S, hq, d, dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention_ex(plan, q.cuda(), None, 0, rk.cuda(), rv.cuda(), res_len, out, ws, out_f32=out32)
    torch.cuda.synchronize()
    empty = np.zeros((0, n))
    err = 0.0
    for i in range(S):
        ref = O.attention_with_residual_f64(q[i].float().numpy(), empty, empty, rk[i, :res_len].float().numpy(),
                                            rv[i, :res_len].float().numpy(), hkv, d)
        o32 = out32[i].cpu().numpy().astype(np.float64)
        err = max(err, (np.abs(o32 - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())
    say(f"  max row-normwise error {err:.3e}")
    assert err <= TOL
    assert torch.equal(out32.cpu().to(torch.bfloat16).view(torch.int16), out.cpu().view(torch.int16))
