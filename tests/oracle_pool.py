"""Runs the oracle over window-aligned token chunks in spawned worker
processes (the chunks are independent: every key-mean window lies inside
one).  Test/baseline helper only; the arithmetic is oracle.encode_cache."""

import multiprocessing as mp
import os

import numpy as np

import oracle as O


_WORKER_PARAMS = {}


def _init_worker(pdict):
    """Builds the coding tables once per worker process (outside any timing)."""
    p = O.OracleParams(**pdict)
    p.table("k")
    p.table("v")
    _WORKER_PARAMS[tuple(sorted(pdict.items()))] = p


def _encode_chunk(args):
    k, v, pdict = args
    p = _WORKER_PARAMS.get(tuple(sorted(pdict.items()))) or O.OracleParams(**pdict)
    r = O.encode_cache(k, v, p)
    keep = ("k_cont", "v_cont", "k_so", "v_so", "k_mean_q", "k_mean_scale", "mu_hat",
            "k_sym", "v_sym", "stats")
    return {key: r[key] for key in keep}


def _param_dict(p):
    """OracleParams fields a worker needs to rebuild the same parameters."""
    return dict(n_kv_heads=p.n_kv_heads, head_dim=p.head_dim, levels_k=p.levels_k,
                levels_v=p.levels_v, container_bytes_k=p.container_bytes_k,
                container_bytes_v=p.container_bytes_v, mean_window=p.mean_window, alpha=p.alpha,
                values_k=None if p.values_k is None else tuple(float(x) for x in p.values_k),
                values_v=None if p.values_v is None else tuple(float(x) for x in p.values_v))


def n_workers():
    return max(1, min(16, os.cpu_count() or 1))


def encode_cache_parallel(k, v, p, procs=None, chunk_windows=1):
    """oracle.encode_cache of one sequence (k, v float32 [T, n]) in parallel."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    T = k.shape[0]
    step = p.mean_window * chunk_windows
    pdict = _param_dict(p)
    jobs = [(k[t:t + step], v[t:t + step], pdict) for t in range(0, T, step)]
    procs = procs or n_workers()
    if procs == 1 or len(jobs) == 1:
        _init_worker(pdict)
        parts = [_encode_chunk(j) for j in jobs]
    else:
        with mp.get_context("spawn").Pool(min(procs, len(jobs)), initializer=_init_worker,
                                          initargs=(pdict,)) as pool:
            parts = pool.map(_encode_chunk, jobs, chunksize=1)
    out = {}
    for key in parts[0]:
        if key == "stats":
            out[key] = np.sum([pp[key] for pp in parts], axis=0).astype(np.uint64)
        else:
            out[key] = np.concatenate([pp[key] for pp in parts])
    return out


def _decode_attention_job(job):
    """Oracle read side for one sequence: Algorithm 2 on every container, then
    the factored float64 attention of Eqs. (8)-(9)."""
    r, q, pdict = job
    p = _WORKER_PARAMS.get(tuple(sorted(pdict.items()))) or O.OracleParams(**pdict)
    fk, ck, _ = p.table("k")
    fv, cv, _ = p.table("v")
    k_sym, _, _ = O.rans_decode(r["k_cont"], fk, ck, p.n)
    v_sym, _, _ = O.rans_decode(r["v_cont"], fv, cv, p.n)
    mu_tok = np.repeat(r["mu_hat"], p.mean_window, axis=0)
    kv = None if p.values_k is None else p.vals("k")
    vv = None if p.values_v is None else p.vals("v")
    return O.attention_factored_f64(q, k_sym, r["k_so"], mu_tok, v_sym, r["v_so"],
                                    p.n_kv_heads, p.head_dim, k_vals=kv, v_vals=vv)


def time_decode_attention(refs, qs, p, procs, repeats=1, target_s=None):
    """Wall time of the oracle read side over independent sequences run in
    `procs` worker processes (one sequence per task).  With target_s, the task
    list is repeated until one timed pass is expected to take about that long.
    Returns (seconds, tasks timed, outputs of the first len(refs) tasks)."""
    import time
    pdict = _param_dict(p)
    slim = [{k: r[k] for k in ("k_cont", "v_cont", "k_so", "v_so", "mu_hat")} for r in refs]
    base = [(slim[i], qs[i], pdict) for i in range(len(refs))]
    with mp.get_context("spawn").Pool(procs, initializer=_init_worker, initargs=(pdict,)) as pool:
        warm = base * max(1, procs // len(base))
        pool.map(_decode_attention_job, warm, chunksize=1)      # workers up and warm
        t0 = time.perf_counter()
        pool.map(_decode_attention_job, warm, chunksize=1)
        per_task = (time.perf_counter() - t0) * min(procs, len(warm)) / len(warm)
        if target_s:
            repeats = max(repeats, int(target_s * procs / max(per_task, 1e-6) / len(base)) + 1)
        jobs = base * repeats
        t0 = time.perf_counter()
        outs = pool.map(_decode_attention_job, jobs, chunksize=1)
        dt = time.perf_counter() - t0
    return dt, len(jobs), outs[:len(refs)]
