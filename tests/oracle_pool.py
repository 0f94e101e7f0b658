"""Runs the oracle over window-aligned token chunks in spawned worker
processes (the chunks are independent: every key-mean window lies inside
one).  Test/baseline helper only; the arithmetic is oracle.encode_cache."""

import multiprocessing as mp
import os

import numpy as np

import oracle as O


def _encode_chunk(args):
    k, v, pdict = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    p = O.OracleParams(**pdict)
    r = O.encode_cache(k, v, p)
    keep = ("k_cont", "v_cont", "k_so", "v_so", "k_mean_q", "k_mean_scale", "mu_hat",
            "k_sym", "v_sym", "stats")
    return {key: r[key] for key in keep}


def n_workers():
    return max(1, min(16, os.cpu_count() or 1))


def encode_cache_parallel(k, v, p, procs=None, chunk_windows=1):
    """oracle.encode_cache of one sequence (k, v float32 [T, n]) in parallel."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    T = k.shape[0]
    step = p.mean_window * chunk_windows
    pdict = dict(n_kv_heads=p.n_kv_heads, head_dim=p.head_dim, levels_k=p.levels_k,
                 levels_v=p.levels_v, container_bytes_k=p.container_bytes_k,
                 container_bytes_v=p.container_bytes_v, mean_window=p.mean_window, alpha=p.alpha)
    jobs = [(k[t:t + step], v[t:t + step], pdict) for t in range(0, T, step)]
    procs = procs or n_workers()
    if procs == 1 or len(jobs) == 1:
        parts = [_encode_chunk(j) for j in jobs]
    else:
        with mp.get_context("spawn").Pool(min(procs, len(jobs))) as pool:
            parts = pool.map(_encode_chunk, jobs)
    out = {}
    for key in parts[0]:
        if key == "stats":
            out[key] = np.sum([pp[key] for pp in parts], axis=0).astype(np.uint64)
        else:
            out[key] = np.concatenate([pp[key] for pp in parts])
    return out
