"""Thin Python binding of libkvq (include/kvq.h): argument marshalling only.

Every function below has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU; their data pointers and the current HIP stream are
passed straight through.  Every step of the computation runs in the HIP
library; if it is not built this module raises instead of doing anything else.
"""

import ctypes
import os

import torch  # loads the HIP runtime libkvq links against (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_F32, KVQ_BF16 = 0, 1
_STATUS = {0: "KVQ_OK", -1: "KVQ_EINVAL", -2: "KVQ_EINFEASIBLE", -3: "KVQ_EUNSUPPORTED",
           -4: "KVQ_EDEVICE", -5: "KVQ_ENOMEM", -6: "KVQ_EWORKSPACE"}


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().kvq_status_str(status).decode()
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({msg})")


class kvq_params(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("levels_k", ctypes.c_int32), ("levels_v", ctypes.c_int32),
                ("container_bytes_k", ctypes.c_int32), ("container_bytes_v", ctypes.c_int32),
                ("mean_window", ctypes.c_int32), ("sharpen_alpha", ctypes.c_double),
                ("container_layout", ctypes.c_int32)]


KVQ_LAYOUT_ROWS, KVQ_LAYOUT_TILES = 0, 1


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_SIGS = {
    "kvq_plan_create": (_I32, [ctypes.POINTER(kvq_params), ctypes.POINTER(_P)]),
    "kvq_plan_create_levels": (_I32, [ctypes.POINTER(kvq_params), _P, _P, ctypes.POINTER(_P)]),
    "kvq_plan_levels": (_I32, [_P, ctypes.c_int, _P]),
    "kvq_plan_destroy": (None, [_P]),
    "kvq_plan_tables": (_I32, [_P, ctypes.c_int, _P, _P, _P]),
    "kvq_plan_lambda_grid": (_I32, [_P, _P]),
    "kvq_model_probs": (_I32, [_I32, _I32, ctypes.c_double, _P]),
    "kvq_bits_per_elem": (ctypes.c_double, [ctypes.POINTER(kvq_params), ctypes.c_int]),
    "kvq_containers_for_budget": (_I32, [ctypes.c_double, _I32, _I32, _I32,
                                         ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "kvq_workspace_bytes": (_I32, [_P, ctypes.c_int, _I64, _I64, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "kvq_encode_streams": (_I32, [_P, _P, _P, ctypes.c_int, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kvq_decode_attention": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float,
                                    _P, _P, _P, ctypes.c_size_t, _P]),
    "kvq_encode_append": (_I32, [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                                 _P, _P, _P]),
    "kvq_decode_attention_noalloc": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _I64, _I64,
                                            ctypes.c_float, _P, _P, _P]),
    "kvq_decode_attention_ex": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P,
                                       _I64, _I64, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "kvq_fixed_width_container_bytes": (_I32, [_I32, _I32, ctypes.POINTER(_I32)]),
    "kvq_encode_fixed_width": (_I32, [_P, _P, _P, ctypes.c_int, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "kvq_decode_attention_fixed_width": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _I64, _I64,
                                                ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "kvq_decode_symbols": (_I32, [_P, ctypes.c_int, _P, _I64, _P, _P, _P]),
    "kvq_status_str": (ctypes.c_char_p, [_I32]),
    "kvq_timing_enable": (_I32, [ctypes.c_int]),
    "kvq_timing_collect": (_I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
}


def lib():
    """Loads libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_entropy_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise KvqError(fn, status)


def _ptr(t, need=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor holding at least `need` bytes.
    The C ABI takes bare pointers, so this is the only place where a host
    tensor or a short buffer can be caught before a kernel touches it."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        # kernels launch on the current device and would fault on another's memory
        raise ValueError(f"{name}: on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if need is not None and t.numel() * t.element_size() < need:
        raise ValueError(f"{name}: holds {t.numel() * t.element_size()} bytes, needs {need}")
    return ctypes.c_void_p(t.data_ptr())


def _cache_ptrs(plan, S, rows, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale):
    """Pointers of the six cache arrays for S sequences of `rows` token rows."""
    p = plan.params
    nW = rows // p.mean_window
    cr = plan.cache_rows(rows)
    return (_ptr(k_cont, S * cr * plan.stored_bytes(0), "k_cont"),
            _ptr(v_cont, S * cr * plan.stored_bytes(1), "v_cont"),
            _ptr(k_so, S * rows * 4, "k_so"), _ptr(v_so, S * rows * 4, "v_so"),
            _ptr(k_mean_q, S * nW * plan.n, "k_mean_q"), _ptr(k_mean_scale, S * nW * 2, "k_mean_scale"))


def _kv_ptrs(plan, k, v):
    """(dtype code, S, T, k pointer, v pointer) of K/V inputs [S, T, Hkv, d] or [S, T, n]."""
    if k.dtype != v.dtype or k.shape != v.shape:
        raise ValueError("k and v must have the same dtype and shape")
    dt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}.get(k.dtype)
    if dt is None:
        raise TypeError("k/v must be float32 or bfloat16")
    S, T = int(k.shape[0]), int(k.shape[1])
    if k.numel() != S * T * plan.n:
        raise ValueError(f"k/v must hold [S, T, {plan.n}] values")
    return dt, S, T, _ptr(k, name="k"), _ptr(v, name="v")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError(f"stream: on {stream.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Owns a kvq_plan (host-side tables of one cache format)."""

    def __init__(self, n_kv_heads, head_dim, levels_k=8, levels_v=6, container_bytes_k=331,
                 container_bytes_v=231, mean_window=128, sharpen_alpha=1.4, values_k=None, values_v=None,
                 layout=KVQ_LAYOUT_ROWS):
        self.params = kvq_params(n_kv_heads, head_dim, levels_k, levels_v, container_bytes_k,
                                 container_bytes_v, mean_window, sharpen_alpha, layout)
        h = ctypes.c_void_p()
        if values_k is None and values_v is None:
            _check("kvq_plan_create", lib().kvq_plan_create(ctypes.byref(self.params), ctypes.byref(h)))
        else:
            arr = lambda vals: None if vals is None else (ctypes.c_float * len(vals))(*vals)
            _check("kvq_plan_create_levels", lib().kvq_plan_create_levels(
                ctypes.byref(self.params), arr(values_k), arr(values_v), ctypes.byref(h)))
        self.handle = h

    @property
    def tiles(self):
        return self.params.container_layout == KVQ_LAYOUT_TILES

    def stored_bytes(self, side):
        """Bytes a container of side 0 (K) / 1 (V) occupies in the cache."""
        C = self.params.container_bytes_k if side == 0 else self.params.container_bytes_v
        return (C + 3) // 4 * 4 if self.tiles else C

    def cache_rows(self, tokens):
        """Token rows a cache of `tokens` tokens per sequence holds (whole 64-token
        tiles in the tile layout)."""
        return (tokens + 63) // 64 * 64 if self.tiles else tokens

    def levels(self, side):
        """Level values v_m as stored (floats) for side 0 (K) / 1 (V)."""
        out = (ctypes.c_float * 16)()
        _check("kvq_plan_levels", lib().kvq_plan_levels(self.handle, side, out))
        M = self.params.levels_k if side == 0 else self.params.levels_v
        return list(out)[:M]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.kvq_plan_destroy(h)
            self.handle = None

    @property
    def n(self):
        return self.params.n_kv_heads * self.params.head_dim

    def tables(self, side):
        """(freq, cum, rate_fx) lists of length `levels` for side 0 (K) / 1 (V)."""
        f = (ctypes.c_uint16 * 16)()
        c = (ctypes.c_uint16 * 16)()
        r = (ctypes.c_int32 * 16)()
        _check("kvq_plan_tables", lib().kvq_plan_tables(self.handle, side, f, c, r))
        M = self.params.levels_k if side == 0 else self.params.levels_v
        return list(f)[:M], list(c)[:M], list(r)[:M]

    def lambda_grid(self):
        g = (ctypes.c_float * 512)()
        _check("kvq_plan_lambda_grid", lib().kvq_plan_lambda_grid(self.handle, g))
        return list(g)

    def bits_per_elem(self, metadata=True):
        return lib().kvq_bits_per_elem(ctypes.byref(self.params), int(bool(metadata)))

    def workspace_bytes(self, op, n_seqs, seq_len, n_q_heads):
        b = ctypes.c_size_t()
        _check("kvq_workspace_bytes", lib().kvq_workspace_bytes(
            self.handle, op, n_seqs, seq_len, n_q_heads, ctypes.byref(b)))
        return b.value


def kvq_model_probs(levels, n, alpha=1.0):
    """Model probabilities of the `levels` symbols (list of floats)."""
    out = (ctypes.c_double * levels)()
    _check("kvq_model_probs", lib().kvq_model_probs(levels, n, float(alpha), out))
    return list(out)


def kvq_containers_for_budget(bits_per_elem, n_kv_heads, head_dim, mean_window):
    ck, cv = _I32(), _I32()
    _check("kvq_containers_for_budget", lib().kvq_containers_for_budget(
        bits_per_elem, n_kv_heads, head_dim, mean_window, ctypes.byref(ck), ctypes.byref(cv)))
    return ck.value, cv.value


def kvq_encode_streams(plan, k, v, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale,
                       stats=None, stream=None):
    """k, v: [S, T, Hkv, d] (or [S, T, n]) fp32/bf16 CUDA tensors; outputs as in kvq.h."""
    dt, S, T, kp, vp = _kv_ptrs(plan, k, v)
    cp = _cache_ptrs(plan, S, T, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale)
    _check("kvq_encode_streams", lib().kvq_encode_streams(
        plan.handle, kp, vp, dt, S, T, *cp, _ptr(stats, 64, "stats"), _stream(stream)))


def kvq_decode_attention(plan, q, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, out,
                         workspace, out_f32=None, softmax_scale=0.0, stream=None):
    """q: [S, Hq, d] bf16; out: [S, Hq, d] bf16; workspace: uint8 CUDA tensor."""
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("q and out must be bfloat16")
    S, Hq = int(q.shape[0]), int(q.shape[1])
    T = int(k_cont.shape[1])
    d = plan.params.head_dim
    cp = _cache_ptrs(plan, S, T, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale)
    _check("kvq_decode_attention", lib().kvq_decode_attention(
        plan.handle, _ptr(q, S * Hq * d * 2, "q"), Hq, *cp, S, T, float(softmax_scale),
        _ptr(out, S * Hq * d * 2, "out"), _ptr(out_f32, S * Hq * d * 4, "out_f32"),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 72 << 20     # KVQ_NOALLOC_SCRATCH_BYTES


def kvq_decode_attention_noalloc(plan, q, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, out,
                                 out_f32=None, softmax_scale=0.0, stream=None):
    """kvq_decode_attention without a workspace: the library's fixed scratch
    array of NOALLOC_SCRATCH_BYTES per GPU takes its place."""
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("q and out must be bfloat16")
    S, Hq = int(q.shape[0]), int(q.shape[1])
    T = int(k_cont.shape[1])
    d = plan.params.head_dim
    cp = _cache_ptrs(plan, S, T, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale)
    _check("kvq_decode_attention_noalloc", lib().kvq_decode_attention_noalloc(
        plan.handle, _ptr(q, S * Hq * d * 2, "q"), Hq, *cp, S, T, float(softmax_scale),
        _ptr(out, S * Hq * d * 2, "out"), _ptr(out_f32, S * Hq * d * 4, "out_f32"), _stream(stream)))


def kvq_encode_append(plan, k, v, cache, token_offset, stats=None, stream=None):
    """Encodes k, v [S, T', Hkv, d] into rows [token_offset, token_offset + T') of `cache`
    (the dict of alloc_cache; the capacity is the second dimension of its k_so)."""
    dt, S, T, kp, vp = _kv_ptrs(plan, k, v)
    cap = int(cache["k_so"].shape[1])           # the capacity (container arrays may round it up)
    cp = _cache_ptrs(plan, S, cap, cache["k_cont"], cache["v_cont"], cache["k_so"], cache["v_so"],
                     cache["k_mean_q"], cache["k_mean_scale"])
    _check("kvq_encode_append", lib().kvq_encode_append(
        plan.handle, kp, vp, dt, S, T, cap, int(token_offset), *cp, _ptr(stats, 64, "stats"),
        _stream(stream)))


def kvq_decode_attention_ex(plan, q, cache, n_tokens, res_k, res_v, res_len, out, workspace,
                            out_f32=None, softmax_scale=0.0, stream=None):
    """Attention over rows [0, n_tokens) of `cache` (capacity = k_so's second dimension;
    may be None when n_tokens == 0) and rows [0, res_len) of res_k / res_v
    [S, R_cap, Hkv, d] bf16 (may be None when res_len == 0)."""
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("q and out must be bfloat16")
    S, Hq = int(q.shape[0]), int(q.shape[1])
    c = cache or {}
    cap = int(c["k_so"].shape[1]) if cache is not None else 0
    rcap = int(res_k.shape[1]) if res_k is not None else 0
    if res_k is not None and (res_k.dtype != torch.bfloat16 or res_v.dtype != torch.bfloat16):
        raise TypeError("res_k and res_v must be bfloat16")
    d = plan.params.head_dim
    cp = _cache_ptrs(plan, S, cap, c.get("k_cont"), c.get("v_cont"), c.get("k_so"), c.get("v_so"),
                     c.get("k_mean_q"), c.get("k_mean_scale"))
    rbytes = S * rcap * plan.n * 2
    _check("kvq_decode_attention_ex", lib().kvq_decode_attention_ex(
        plan.handle, _ptr(q, S * Hq * d * 2, "q"), Hq, *cp, S, cap, int(n_tokens),
        _ptr(res_k, rbytes, "res_k"), _ptr(res_v, rbytes, "res_v"), rcap, int(res_len),
        float(softmax_scale), _ptr(out, S * Hq * d * 2, "out"), _ptr(out_f32, S * Hq * d * 4, "out_f32"),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def kvq_fixed_width_container_bytes(levels, n):
    b = _I32()
    _check("kvq_fixed_width_container_bytes", lib().kvq_fixed_width_container_bytes(levels, n, ctypes.byref(b)))
    return b.value


def kvq_encode_fixed_width(plan, k, v, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, stream=None):
    """As kvq_encode_streams, in the fixed-width comparator format."""
    dt, S, T, kp, vp = _kv_ptrs(plan, k, v)
    cp = _cache_ptrs(plan, S, T, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale)
    _check("kvq_encode_fixed_width", lib().kvq_encode_fixed_width(
        plan.handle, kp, vp, dt, S, T, *cp, _stream(stream)))


def kvq_decode_attention_fixed_width(plan, q, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, out,
                                     workspace, out_f32=None, softmax_scale=0.0, stream=None):
    """As kvq_decode_attention, over fixed-width containers."""
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("q and out must be bfloat16")
    S, Hq = int(q.shape[0]), int(q.shape[1])
    T = int(k_cont.shape[1])
    d = plan.params.head_dim
    cp = _cache_ptrs(plan, S, T, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale)
    _check("kvq_decode_attention_fixed_width", lib().kvq_decode_attention_fixed_width(
        plan.handle, _ptr(q, S * Hq * d * 2, "q"), Hq, *cp, S, T, float(softmax_scale),
        _ptr(out, S * Hq * d * 2, "out"), _ptr(out_f32, S * Hq * d * 4, "out_f32"),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def kvq_decode_symbols(plan, side, cont, symbols, end_ok=None, stream=None):
    """cont: [..., C] uint8; symbols: [..., n] uint8; end_ok: nullable int32/uint32-sized."""
    C = plan.stored_bytes(side)
    if cont.shape[-1] != C:
        raise ValueError(f"cont: last dimension must be the stored container size {C}")
    n_streams = cont.numel() // C
    _check("kvq_decode_symbols", lib().kvq_decode_symbols(
        plan.handle, side, _ptr(cont, name="cont"), n_streams, _ptr(symbols, n_streams * plan.n, "symbols"),
        _ptr(end_ok, n_streams * 4, "end_ok"), _stream(stream)))


def kvq_timing_enable(on):
    _check("kvq_timing_enable", lib().kvq_timing_enable(int(bool(on))))


def kvq_timing_collect():
    """(total milliseconds, launches) of the timed attention kernels."""
    ms, n = ctypes.c_double(), _I64()
    _check("kvq_timing_collect", lib().kvq_timing_collect(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def alloc_cache(plan, n_seqs, seq_len, device="cuda"):
    """Empty output tensors for kvq_encode_streams (plumbing only)."""
    p = plan.params
    nW = seq_len // p.mean_window
    e = lambda *shape, dtype: torch.empty(*shape, dtype=dtype, device=device)
    rows = plan.cache_rows(seq_len)
    return {
        "k_cont": e(n_seqs, rows, plan.stored_bytes(0), dtype=torch.uint8),
        "v_cont": e(n_seqs, rows, plan.stored_bytes(1), dtype=torch.uint8),
        "k_so": e(n_seqs, seq_len, 2, dtype=torch.int16),
        "v_so": e(n_seqs, seq_len, 2, dtype=torch.int16),
        "k_mean_q": e(n_seqs, nW, plan.n, dtype=torch.int8),
        "k_mean_scale": e(n_seqs, nW, dtype=torch.int16),
    }


def container_rows(plan, side, cont, n_tokens):
    """The containers of a cache array as [S, n_tokens, C] rows (a copy; for
    inspection and tests, not the read path): in the tile layout, dword k of
    token g sits at dword (g / 64) 64 Cp / 4 + k 64 + g mod 64 of the array."""
    C = plan.params.container_bytes_k if side == 0 else plan.params.container_bytes_v
    if not plan.tiles:
        return cont[:, :n_tokens, :C]
    S, rows, Cp = int(cont.shape[0]), int(cont.shape[1]), int(cont.shape[2])
    t = cont.reshape(S, rows // 64, Cp // 4, 64, 4).permute(0, 1, 3, 2, 4).reshape(S, rows, Cp)
    return t[:, :n_tokens, :C].contiguous()
