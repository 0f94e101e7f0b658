"""CPU tests of libkvq: it loads, exports every entry point of include/kvq.h,
its host planner reproduces the oracle's tables independently, and argument
errors are reported before any device work (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
kvq = pytest.importorskip("kv_cache_entropy_amd.kvq")


def _lib():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq.lib()


def test_exports_every_declared_symbol():
    L = _lib()
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    names = set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", hdr))
    assert len(names) >= 11
    for name in sorted(names):
        assert hasattr(L, name), name


@pytest.mark.parametrize("hkv,d,mk,mv,ck,cv,alpha", [
    (1, 128, 8, 6, 36, 36, 1.4), (8, 128, 8, 6, 331, 231, 1.4), (8, 128, 8, 6, 292, 203, 1.4),
    (8, 128, 8, 6, 593, 414, 1.4), (4, 64, 16, 4, 200, 100, 1.0), (2, 256, 5, 7, 300, 300, 2.0),
])
def test_planner_tables_match_oracle(hkv, d, mk, mv, ck, cv, alpha):
    _lib()
    plan = kvq.Plan(hkv, d, mk, mv, ck, cv, 128, alpha)
    n = hkv * d
    for side, M in ((0, mk), (1, mv)):
        f, c = O.build_table(M, n, alpha)
        r = O.rate_table(f)
        pf, pc, pr = plan.tables(side)
        assert pf == f.tolist() and pc == c.tolist() and pr == r.tolist()
    E = O.lambda_table()
    assert np.array_equal(np.array(plan.lambda_grid(), np.float32).view(np.uint32), E.view(np.uint32))
    assert abs(plan.bits_per_elem(True) - O.bits_per_elem(ck, cv, n, 128)) < 1e-12
    assert abs(plan.bits_per_elem(False) - O.bits_per_elem(ck, cv, n, 128, metadata=False)) < 1e-12


def test_budget_helper_matches_oracle():
    _lib()
    for b in (1.96, 2.0, 2.26, 2.5, 3.0, 4.0):
        assert kvq.kvq_containers_for_budget(b, 8, 128, 128) == O.containers_for_budget(b, 1024, 128)


def test_plan_errors():
    _lib()
    with pytest.raises(kvq.KvqError) as e:
        kvq.Plan(8, 100)                       # head_dim not a power of two
    assert e.value.status == -1
    with pytest.raises(kvq.KvqError) as e:
        kvq.Plan(8, 128, 8, 6, 100, 231)       # 1024 cheapest K symbols need > 96 bytes
    assert e.value.status == -2
    with pytest.raises(kvq.KvqError):
        kvq.Plan(8, 128, 1, 6)                 # one level
    with pytest.raises(kvq.KvqError):
        kvq.Plan(8, 128, mean_window=100)


def test_device_entry_points_reject_bad_arguments_before_launch():
    L = _lib()
    plan = kvq.Plan(8, 128)
    p = ctypes.c_void_p
    a16 = p(1 << 20)                          # never dereferenced: checks fail first
    bad = p((1 << 20) + 8)
    st = p(0)
    # null pointer
    assert L.kvq_encode_streams(plan.handle, None, a16, 1, 1, 128, a16, a16, a16, a16, a16, a16,
                                None, st) == -1
    # misaligned pointer
    assert L.kvq_encode_streams(plan.handle, a16, bad, 1, 1, 128, a16, a16, a16, a16, a16, a16,
                                None, st) == -1
    # seq_len not a multiple of the window
    assert L.kvq_encode_streams(plan.handle, a16, a16, 1, 1, 200, a16, a16, a16, a16, a16, a16,
                                None, st) == -1
    # Hq not a multiple of Hkv
    assert L.kvq_decode_attention(plan.handle, a16, 12, a16, a16, a16, a16, a16, a16, 1, 1024, 0.0,
                                  a16, None, a16, 1 << 30, st) == -1
    # too small a workspace
    need = plan.workspace_bytes(1, 2, 1024, 32)
    assert need > 0
    assert L.kvq_decode_attention(plan.handle, a16, 32, a16, a16, a16, a16, a16, a16, 2, 1024, 0.0,
                                  a16, None, a16, need - 1, st) == -6
    # unsupported head layout (3 query heads per KV head)
    assert L.kvq_decode_attention(plan.handle, a16, 24, a16, a16, a16, a16, a16, a16, 1, 1024, 0.0,
                                  a16, None, a16, 1 << 30, st) == -3
    assert L.kvq_decode_symbols(plan.handle, 2, a16, 4, a16, None, st) == -1
    assert plan.workspace_bytes(0, 4, 1024, 32) == 0


def test_append_and_residual_entry_points_reject_bad_arguments():
    L = _lib()
    plan = kvq.Plan(8, 128)
    p = ctypes.c_void_p
    a16 = p(1 << 20)                          # never dereferenced: checks fail first
    st = p(0)
    ok_args = lambda **kw: dict(dict(n=128, cap=1024, off=0), **kw)

    def append(n, cap, off):
        return L.kvq_encode_append(plan.handle, a16, a16, 1, 2, n, cap, off, a16, a16, a16, a16, a16,
                                   a16, None, st)
    assert append(**ok_args(off=64)) == -1            # offset not a multiple of W
    assert append(**ok_args(n=100)) == -1             # tokens not a multiple of W
    assert append(**ok_args(off=1024)) == -1          # past the capacity
    assert append(**ok_args(cap=1000)) == -1          # capacity not a multiple of W

    def attend(n_tok, res_len, res_cap=256, res=a16, cap=1024):
        return L.kvq_decode_attention_ex(plan.handle, a16, 32, a16, a16, a16, a16, a16, a16, 2, cap, n_tok,
                                         res, res, res_cap, res_len, 0.0, a16, None, a16, 1 << 30, st)
    assert attend(0, 0) == -1                         # nothing to attend
    assert attend(128, 300) == -1                     # tail longer than its buffer
    assert attend(0, 10, res=None) == -1              # tail without buffers
    assert attend(100, 0) == -1                       # not a multiple of W
    assert attend(2048, 0) == -1                      # more tokens than the capacity
    assert plan.workspace_bytes(1, 2, 0, 32) > 0      # a tail-only call still needs partials


def test_encode_rejects_stream_lengths_without_a_kernel():
    """The encoder has one instantiation per stream length n = 64 * 2^k; other
    lengths (here 3 KV heads of 64 channels) return KVQ_EUNSUPPORTED before any
    launch, so no output array is touched."""
    L = _lib()
    p = ctypes.c_void_p
    a16, st = p(1 << 20), p(0)
    for hkv, d, want in ((3, 64, -3), (1, 32, -3), (5, 128, -3)):
        plan = kvq.Plan(hkv, d, 8, 6, 200, 150)
        assert L.kvq_encode_streams(plan.handle, a16, a16, 1, 1, 128, a16, a16, a16, a16, a16, a16, None,
                                    st) == want


def test_size_limits_are_rejected_before_launch():
    """The decode attention addresses a sequence's containers with 32-bit
    offsets and puts sequences on the grid's y axis: past those limits it
    returns KVQ_EUNSUPPORTED (the header's stated limits) and launches nothing."""
    L = _lib()
    plan = kvq.Plan(8, 128)                                # 331/231-byte containers
    p = ctypes.c_void_p
    a16, st = p(1 << 20), p(0)

    def attend(n_seqs, n_tok):
        return L.kvq_decode_attention(plan.handle, a16, 32, a16, a16, a16, a16, a16, a16, n_seqs, n_tok, 0.0,
                                      a16, None, a16, 1 << 62, st)
    t_big = (2 ** 31 // 331 // 128 + 1) * 128            # first W-multiple with T * C_K >= 2^31
    assert t_big * 331 + 16 > 2 ** 31 - 1 and (t_big - 128) * 331 + 16 <= 2 ** 31 - 1
    assert attend(1, t_big) == -3
    assert attend(65536, 128) == -3                       # more sequences than grid rows
    assert attend(65536 - 1, 128 + 1) == -1               # (shape errors still come first)


@pytest.mark.parametrize("M,n,alpha", [(8, 1024, 1.0), (6, 1024, 1.4), (8, 128, 1.0), (3, 1024, 2.0)])
def test_model_probs_match_oracle(M, n, alpha):
    _lib()
    got = np.array(kvq.kvq_model_probs(M, n, alpha))
    p = O.order_stat_probs(M, n)
    want = O.sharpen(p, alpha) if alpha != 1.0 else p
    assert np.max(np.abs(got - want)) <= 1e-9


def test_fixed_width_sizes_and_errors():
    L = _lib()
    assert kvq.kvq_fixed_width_container_bytes(6, 1024) == 512 == O.fw_container_bytes(6, 1024)
    assert kvq.kvq_fixed_width_container_bytes(3, 1024) == 256 == O.fw_container_bytes(3, 1024)
    assert kvq.kvq_fixed_width_container_bytes(2, 1024) == 128
    with pytest.raises(kvq.KvqError):
        kvq.kvq_fixed_width_container_bytes(6, 4)          # 16 bits: not whole dwords
    p = ctypes.c_void_p
    a16 = p(1 << 20)
    st = p(0)
    plan = kvq.Plan(8, 128, 6, 3, 331, 231)                # entropy-coded sizes, not fixed-width ones
    assert L.kvq_encode_fixed_width(plan.handle, a16, a16, 1, 1, 128, a16, a16, a16, a16, a16, a16, st) == -1
    assert L.kvq_decode_attention_fixed_width(plan.handle, a16, 32, a16, a16, a16, a16, a16, a16, 1, 128, 0.0,
                                              a16, None, a16, 1 << 30, st) == -1
    fw = kvq.Plan(8, 128, 16, 3, 512, 256)                 # 16 key levels: no 4-entry level lookup
    assert L.kvq_decode_attention_fixed_width(fw.handle, a16, 32, a16, a16, a16, a16, a16, a16, 1, 128, 0.0,
                                              a16, None, a16, 1 << 30, st) == -3


@pytest.mark.parametrize("values_k,values_v", [
    ((0.0, 0.75, 1.875, 3.0, 4.0, 5.125, 6.25, 7.0), (0.0, 0.875, 2.125, 2.875, 4.125, 5.0)),
    ((0.0, 0.3, 1.1, 3.0), None),
    (None, (0.0, 0.5, 1.75, 3.25, 4.0)),
])
def test_planner_tables_with_levels_match_oracle(values_k, values_v):
    _lib()
    mk = len(values_k) if values_k else 8
    mv = len(values_v) if values_v else 6
    plan = kvq.Plan(8, 128, mk, mv, 331, 231, 128, 1.4, values_k=values_k, values_v=values_v)
    p = O.OracleParams(8, 128, mk, mv, 331, 231, 128, 1.4, values_k=values_k, values_v=values_v)
    for side, key in ((0, "k"), (1, "v")):
        f, c, r = p.table(key)
        pf, pc, pr = plan.tables(side)
        assert pf == f.tolist() and pc == c.tolist() and pr == r.tolist()
        assert np.array_equal(np.array(plan.levels(side), np.float32), p.vals(key))


def test_planner_rejects_bad_levels():
    _lib()
    for vk in ((0.5, 1.0, 2.0, 3.0), (0.0, 1.0, 1.0, 3.0), (0.0, 1.0, 2.0, 2.5)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.Plan(8, 128, 4, 6, 331, 231, values_k=vk)
        assert e.value.status == -1


def test_binding_rejects_host_tensors_and_short_buffers():
    """The C ABI takes bare device pointers; the binding refuses host tensors
    (a kernel would fault on them) before anything reaches the library."""
    import torch
    from kv_cache_entropy_amd import kvq
    plan = kvq.Plan(2, 128, 8, 6, 90, 62, 128, 1.4)
    k = torch.zeros(1, 128, 256, dtype=torch.bfloat16)
    c = {key: torch.zeros(4, dtype=torch.uint8) for key in
         ("k_cont", "v_cont", "k_so", "v_so", "k_mean_q", "k_mean_scale")}
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.kvq_encode_streams(plan, k, k, *c.values())
    with pytest.raises(ValueError, match="k/v must hold"):
        kvq.kvq_encode_streams(plan, k[:, :, :128], k[:, :, :128], *c.values())
    with pytest.raises(ValueError, match="container size"):
        kvq.kvq_decode_symbols(plan, 0, torch.zeros(3, 91, dtype=torch.uint8), torch.zeros(3, 256, dtype=torch.uint8))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library the binding raises; nothing falls back to
    another implementation."""
    from kv_cache_entropy_amd import kvq
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "libkvq.so"))
    with pytest.raises(RuntimeError, match="missing"):
        kvq.Plan(2, 128)
    with pytest.raises(RuntimeError, match="missing"):
        kvq.kvq_model_probs(8, 1024)


def test_noalloc_rejects_calls_beyond_its_scratch_without_launching():
    """kvq_decode_attention_noalloc checks the call's workspace size against its
    fixed scratch array on the host and returns KVQ_EWORKSPACE before touching
    any pointer or the device (so this runs without a GPU)."""
    from kv_cache_entropy_amd import kvq
    L = kvq.lib()
    plan = kvq.Plan(8, 128, 8, 6, 331, 231, 128, 1.4)
    a16 = ctypes.c_void_p(1 << 20)
    S, T, Hq = 4096, 65536, 64
    assert plan.workspace_bytes(1, S, T, Hq) > kvq.NOALLOC_SCRATCH_BYTES
    st = L.kvq_decode_attention_noalloc(plan.handle, a16, Hq, a16, a16, a16, a16, a16, a16, S, T, 0.0,
                                        a16, None, None)
    assert st == -6
    assert L.kvq_decode_attention_noalloc(None, a16, Hq, a16, a16, a16, a16, a16, a16, 1, 1024, 0.0,
                                          a16, None, None) == -1
