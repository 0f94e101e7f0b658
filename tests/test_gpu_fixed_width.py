"""GPU parity of the fixed-width comparator ([D-Quant] Appendix B) with the oracle.

Same preprocessing as the entropy-coded path, nearest rounding at 6 key and 3
value levels, power-of-two symbol widths: containers, metadata and key means
must be bit-identical to oracle.encode_cache_fw; the fused fixed-width
decode attention must be within 2e-3 (row-normwise, fp32 output) of the
oracle's float64 attention over the same symbols, with bf16 = RNE(fp32).
"""

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_entropy_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("hq,hkv,levels,seqs,tokens", [
    (32, 8, (6, 3), [0, 511], (0, 512)),        # the page's comparator levels, gqa layout
    (32, 8, (4, 3), [3], (256, 768)),           # 2-bit keys and values
    (8, 8, (8, 8), [1], (0, 256)),              # 4-bit keys and values, one query head per KV head
    (64, 8, (6, 3), [2], (0, 384)),             # 8 query heads per KV head: two MFMA groups
])
def test_fixed_width_parity(hq, hkv, levels, seqs, tokens):
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = synth.WORKLOADS["gqa"]
    w = synth.Workload(f"fw{hq}x{hkv}", hq, hkv, 128, base.batch, base.layers, base.seq_len, base.seed,
                       base.dist)
    mk, mv = levels
    ck = kvq.kvq_fixed_width_container_bytes(mk, w.n)
    cv = kvq.kvq_fixed_width_container_bytes(mv, w.n)
    say(f"case fixed width {hq}/{hkv} heads, levels {mk}/{mv}, containers {ck}/{cv}, seqs {seqs}, tokens {tokens}")
    plan = kvq.Plan(hkv, 128, mk, mv, ck, cv, 128, 1.4)
    k, v = synth.cache_inputs(w, "cuda", seqs, tokens)
    q = synth.queries(w, "cuda", seqs)
    S, T = k.shape[0], k.shape[1]
    c = kvq.alloc_cache(plan, S, T)
    kvq.kvq_encode_fixed_width(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                               c["k_mean_q"], c["k_mean_scale"])
    ws = torch.empty(plan.workspace_bytes(1, S, T, hq), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, hq, 128, dtype=torch.bfloat16, device="cuda")
    out32 = torch.empty(S, hq, 128, dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention_fixed_width(plan, q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                                         c["k_mean_q"], c["k_mean_scale"], out, ws, out_f32=out32)
    torch.cuda.synchronize()
    errs = []
    for i in range(S):
        r = O.encode_cache_fw(k[i].float().cpu().numpy(), v[i].float().cpu().numpy(), hkv, 128, mk, mv, 128)
        assert np.array_equal(c["k_cont"][i].cpu().numpy(), r["k_cont"])
        assert np.array_equal(c["v_cont"][i].cpu().numpy(), r["v_cont"])
        assert np.array_equal(c["k_so"][i].cpu().numpy().view(np.uint16), r["k_so"].view(np.uint16))
        assert np.array_equal(c["v_so"][i].cpu().numpy().view(np.uint16), r["v_so"].view(np.uint16))
        assert np.array_equal(c["k_mean_q"][i].cpu().numpy(), r["k_mean_q"])
        assert np.array_equal(c["k_mean_scale"][i].cpu().numpy().view(np.uint16), r["k_mean_scale"].view(np.uint16))
        assert np.array_equal(O.fw_unpack(r["k_cont"], mk, w.n), r["k_sym"])
        mu_tok = np.repeat(r["mu_hat"], 128, axis=0)
        ref = O.attention_factored_f64(q[i].float().cpu().numpy(), r["k_sym"], r["k_so"], mu_tok,
                                       r["v_sym"], r["v_so"], hkv, 128)
        o32 = out32[i].cpu().numpy().astype(np.float64)
        errs.append((np.abs(o32 - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())
    err = max(errs)
    say(f"  containers bit-exact; attention max row-normwise error {err:.3e}")
    assert err <= TOL
    assert torch.equal(out32.cpu().to(torch.bfloat16).view(torch.int16), out.cpu().view(torch.int16))


def test_fixed_width_splits_of_several_tiles():
    """32 sequences x 8192 tokens: 4096 tiles, so each split holds two and the
    kernel carries its prefetch from one tile's last head to the next tile's
    first.  Sequence 0 is checked against the oracle (containers bit-exact,
    attention within 2e-3); the rest only have to be finite."""
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = synth.WORKLOADS["gqa"]
    mk, mv = 6, 3
    seqs, tokens = list(range(32)), (0, 8192)
    ck, cv = kvq.kvq_fixed_width_container_bytes(mk, w.n), kvq.kvq_fixed_width_container_bytes(mv, w.n)
    say(f"case fixed width, {len(seqs)} sequences x {tokens[1]} tokens, levels {mk}/{mv}")
    plan = kvq.Plan(w.n_kv_heads, 128, mk, mv, ck, cv, 128, 1.4)
    k, v = synth.cache_inputs(w, "cuda", seqs, tokens)
    q = synth.queries(w, "cuda", seqs)
    S, T = k.shape[0], k.shape[1]
    c = kvq.alloc_cache(plan, S, T)
    kvq.kvq_encode_fixed_width(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                               c["k_mean_q"], c["k_mean_scale"])
    ws = torch.empty(plan.workspace_bytes(1, S, T, w.n_q_heads), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, w.n_q_heads, 128, dtype=torch.bfloat16, device="cuda")
    out32 = torch.empty(S, w.n_q_heads, 128, dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention_fixed_width(plan, q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                                         c["k_mean_q"], c["k_mean_scale"], out, ws, out_f32=out32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out32).all())
    r = O.encode_cache_fw(k[0].float().cpu().numpy(), v[0].float().cpu().numpy(), w.n_kv_heads, 128, mk, mv, 128)
    say("  oracle encode of sequence 0 done")
    assert np.array_equal(c["k_cont"][0].cpu().numpy(), r["k_cont"])
    assert np.array_equal(c["v_cont"][0].cpu().numpy(), r["v_cont"])
    mu_tok = np.repeat(r["mu_hat"], 128, axis=0)
    ref = O.attention_factored_f64(q[0].float().cpu().numpy(), r["k_sym"], r["k_so"], mu_tok,
                                   r["v_sym"], r["v_so"], w.n_kv_heads, 128)
    o32 = out32[0].cpu().numpy().astype(np.float64)
    err = (np.abs(o32 - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max()
    say(f"  sequence 0: attention max row-normwise error {err:.3e}")
    assert err <= TOL
    assert torch.equal(out32.cpu().to(torch.bfloat16).view(torch.int16), out.cpu().view(torch.int16))
