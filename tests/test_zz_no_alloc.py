"""kvq_decode_attention_noalloc (no workspace, the library's fixed scratch array)
against kvq_decode_attention (caller workspace), through the C ABI: the same
kernels, so the outputs must be bit-identical.  Two calls in a row, the second
smaller than the first, so the second runs on scratch still holding the
first call's partials."""

import pytest
import torch

from kv_cache_entropy_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def test_noalloc_matches_the_workspace_entry_point():
    from kv_cache_entropy_amd import kvq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = synth.WORKLOADS["heavy"]
    plan = kvq.Plan(w.n_kv_heads, w.head_dim, 8, 6, 292, 203, 128, 1.4)
    for S, T in ((6, 2048), (2, 512)):
        say(f"case no-alloc decode attention: heavy layout 32/8 heads, {S} sequences x {T} tokens")
        k, v = synth.cache_inputs(w, "cuda", range(S), (0, T))
        q = synth.queries(w, "cuda", range(S))
        c = kvq.alloc_cache(plan, S, T)
        kvq.kvq_encode_streams(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                               c["k_mean_q"], c["k_mean_scale"])
        need = plan.workspace_bytes(1, S, T, w.n_q_heads)
        assert need <= kvq.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        shape = (S, w.n_q_heads, w.head_dim)
        ref, ref32 = torch.empty(shape, dtype=torch.bfloat16, device="cuda"), torch.empty(shape, device="cuda")
        got, got32 = torch.empty_like(ref), torch.empty_like(ref32)
        args = (plan, q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"], c["k_mean_q"], c["k_mean_scale"])
        kvq.kvq_decode_attention(*args, ref, ws, out_f32=ref32)
        kvq.kvq_decode_attention_noalloc(*args, got, out_f32=got32)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(got32.view(torch.int32), ref32.view(torch.int32))
        assert torch.isfinite(got32).all()
        say("  bit-identical to kvq_decode_attention")
