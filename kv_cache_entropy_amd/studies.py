"""Synthetic rate-distortion and drift studies on the GPU path.

    python -m kv_cache_entropy_amd.studies [--seqs 16] [--tokens 1024] [--json out.json]

Analogues, on seeded synthetic KV, of the measurements of the page
"D-Quant: Driftable Entropy Coding for KV Cache Quantization":
  * §3.2 Table 1: NMSE, coding gain (log2 M - H) and normal gap (CE - H) of
    8-level per-token grids after rotation and key-mean removal;
  * §3.2 Table 2: NMSE against the alphabet size at fixed K / V containers
    (2.68 / 1.84 bits per value);
  * §5.4 Figure 4 (middle, right): error against the storage budget at 8/6
    levels, and against the K/V split of a fixed 2.26-bit budget;
  * Appendix C, Figure 6: the largest feasible alphabet against the payload,
    beside equal-rate fixed-width coding (left); the measured symbol
    distributions against the analytic model and the coding table (middle);
    the distribution of the container budget left after drift, and the
    fractions of symbols drift changed (right).
Containers are written and read by libkvq (the same kernels the tests check
bit-exactly against the oracle); torch only measures errors and histograms.
The inputs are the Llama-shaped GQA workload's distribution (per-channel key
means, unit-variance values), not captured KV: the numbers characterise the
coder on near-Gaussian data and are not the page's model-accuracy results.
"""

import argparse
import json
import math
import sys

import torch

from . import kvq, synth


def hadamard(d, device):
    H = torch.ones(1, 1, dtype=torch.float64)
    while H.shape[0] < d:
        H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
    return (H / math.sqrt(d)).to(device)


class Sample:
    """Seeded K, V, q of a few sequences, plus exact references."""

    def __init__(self, seqs, tokens, device="cuda"):
        self.w = synth.WORKLOADS["gqa"]
        self.seqs = list(range(seqs))
        self.k, self.v = synth.cache_inputs(self.w, device, self.seqs, (0, tokens))
        self.q = synth.queries(self.w, device, self.seqs)
        self.S, self.T = len(self.seqs), tokens
        w = self.w
        H = hadamard(w.head_dim, device)
        rot = lambda x: (x.double().reshape(self.S, self.T, w.n_kv_heads, w.head_dim) @ H).reshape(
            self.S, self.T, w.n)
        self.k_rot, self.v_rot = rot(self.k), rot(self.v)
        self.H = H
        self.exact = self.attention(self.k.double(), self.v.double())

    def attention(self, K, V):
        w = self.w
        G = w.n_q_heads // w.n_kv_heads
        q = self.q.double().reshape(self.S, w.n_kv_heads, G, w.head_dim)
        K = K.reshape(self.S, self.T, w.n_kv_heads, w.head_dim).permute(0, 2, 1, 3)
        V = V.reshape(self.S, self.T, w.n_kv_heads, w.head_dim).permute(0, 2, 1, 3)
        a = torch.softmax(q @ K.transpose(-1, -2) / math.sqrt(w.head_dim), dim=-1)
        return (a @ V).reshape(self.S, w.n_q_heads, w.head_dim)


def lloyd_max_levels(M, n, streams=4000, iters=60, seed=0):
    """Non-affine reconstruction levels in grid units for min-max normalised
    N(0,1) streams of length n: Lloyd-Max iteration (start at the quantiles,
    then alternate nearest-level assignment and centroid update), as
    KVQuant-style non-uniform quantisers do.  Every stream puts its minimum at
    0 and its maximum at M - 1, so those two levels stay pinned and only the
    interior ones move.  Returns a tuple of M floats."""
    import numpy as np
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((streams, n))
    u = (x - x.min(1, keepdims=True)) / (x.max(1, keepdims=True) - x.min(1, keepdims=True)) * (M - 1)
    u = np.sort(u.ravel())
    lv = np.quantile(u, (np.arange(M) + 0.5) / M)
    lv[0], lv[-1] = 0.0, M - 1.0
    for _ in range(iters):
        cut = np.searchsorted(u, (lv[1:] + lv[:-1]) / 2)
        for m in range(1, M - 1):
            seg = u[cut[m - 1]:cut[m]]
            if seg.size:
                lv[m] = seg.mean()
    return tuple(float(v) for v in lv)


def run_config(sm, mk, mv, ck, cv, attention=True, values=(None, None)):
    """Encodes the sample with one format; returns errors and symbol statistics.
    values: optional non-affine levels (grid units) for K and V."""
    w = sm.w
    try:
        plan = kvq.Plan(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, 128, 1.4,
                        values_k=values[0], values_v=values[1])
    except kvq.KvqError as e:
        if e.status == -2:            # KVQ_EINFEASIBLE: the alphabet does not fit
            return None
        raise
    c = kvq.alloc_cache(plan, sm.S, sm.T)
    stats = torch.zeros(8, dtype=torch.int64, device="cuda")
    kvq.kvq_encode_streams(plan, sm.k, sm.v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                           c["k_mean_q"], c["k_mean_scale"], stats=stats)
    out = {"levels": [mk, mv], "containers": [ck, cv], "bits_per_elem": plan.bits_per_elem(True)}
    st = stats.cpu().tolist()
    nsym = sm.S * sm.T * w.n
    out["changed_k"], out["changed_v"] = st[2] / nsym, st[6] / nsym
    out["fallbacks"] = st[0] + st[1] + st[4] + st[5]
    mu = (c["k_mean_q"].double() * c["k_mean_scale"].view(torch.float16).double()[..., None])
    mu_tok = mu.repeat_interleave(128, dim=1)
    for side, key, so_key, ref in ((0, "k_cont", "k_so", sm.k_rot), (1, "v_cont", "v_so", sm.v_rot)):
        sym = torch.empty(sm.S, sm.T, w.n, dtype=torch.uint8, device="cuda")
        kvq.kvq_decode_symbols(plan, side, c[key], sym)
        so = c[so_key].view(torch.float16).double()
        lv = torch.tensor(plan.levels(side), dtype=torch.float64, device="cuda")
        rec = so[..., 0:1] * lv[sym.long()] + so[..., 1:2]
        if side == 0:
            rec = rec + mu_tok
        name = "k" if side == 0 else "v"
        out[f"nmse_{name}"] = float(((rec - ref) ** 2).sum() / (ref ** 2).sum())
        M = mk if side == 0 else mv
        hist = torch.bincount(sym.flatten().long(), minlength=M).double()
        ph = hist / hist.sum()
        model = torch.tensor(kvq.kvq_model_probs(M, w.n, 1.0), dtype=torch.float64, device="cuda")
        f, _, _ = plan.tables(side)
        table = torch.tensor(f, dtype=torch.float64, device="cuda") / 256.0
        nz = ph > 0
        H = float(-(ph[nz] * torch.log2(ph[nz])).sum())
        out[f"entropy_{name}"] = H
        out[f"coding_gain_{name}"] = math.log2(M) - H
        out[f"model_gap_{name}"] = (float(-(ph[nz] * torch.log2(model[nz])).sum()) - H
                                    if values[side] is None else None)
        out[f"table_gap_{name}"] = float(-(ph[nz] * torch.log2(table[nz])).sum()) - H
        out[f"hist_{name}"] = [round(float(x), 5) for x in ph]
        if side == 0:
            khat_rot = rec
        else:
            vhat_rot = rec
    if attention and mk <= 9 and mv <= 8:
        o = torch.empty(sm.S, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
        o32 = torch.empty_like(o, dtype=torch.float32)
        ws = torch.empty(plan.workspace_bytes(1, sm.S, sm.T, w.n_q_heads), dtype=torch.uint8, device="cuda")
        kvq.kvq_decode_attention(plan, sm.q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                                 c["k_mean_q"], c["k_mean_scale"], o, ws, out_f32=o32)
        err = (o32.double() - sm.exact).norm(dim=-1) / sm.exact.norm(dim=-1)
        out["attn_rel_err"] = float(err.mean())
        # the same attention from the reconstructed cache in float64 (isolates the
        # kernel's own arithmetic from the quantisation error)
        kh = (khat_rot.reshape(sm.S, sm.T, w.n_kv_heads, w.head_dim) @ sm.H).reshape(sm.S, sm.T, w.n)
        vh = (vhat_rot.reshape(sm.S, sm.T, w.n_kv_heads, w.head_dim) @ sm.H).reshape(sm.S, sm.T, w.n)
        ref_q = sm.attention(kh, vh)
        out["attn_kernel_vs_dequant"] = float(((o32.double() - ref_q).norm(dim=-1) / ref_q.norm(dim=-1)).max())
    torch.cuda.synchronize()
    return out


RATE_ONE = 1 << 16          # the plan's rates r_fx are bits in this fixed point
STATE_BITS = 32             # sigma: the final rANS state at the head of a container


def budget_fx(container_bytes):
    """B = 8 C - sigma bits ([D-Quant] §4.2 Eq. (3)) in the rates' fixed point."""
    return (8 * int(container_bytes) - STATE_BITS) * RATE_ONE


def max_alphabet(n_kv_heads, head_dim, payload_bits, alpha=1.4, max_levels=16):
    """Figure 6 (left) analogue.  For each payload b (bits per value), the
    container C = ceil((b n + sigma) / 8) bytes, its actual payload
    b' = (8 C - sigma) / n, and the largest alphabet M (2..max_levels) whose
    plan is feasible: every value of a stream fits at the cheapest level,
    n r_min <= B (the criterion of Table 2's dashes).  Fixed-width coding at
    the same rate holds M <= 2^b' levels when charged the ideal log2 M bits
    per symbol (as in Appendix B) and 2^floor(b') at whole bits per symbol.
    Returns rows {payload_bits, container_bytes, feasible: [M...], ...}."""
    n = n_kv_heads * head_dim
    rows = []
    for b in payload_bits:
        C = int(math.ceil((b * n + STATE_BITS) / 8))
        bb = (8 * C - STATE_BITS) / n
        feasible = []
        for M in range(2, max_levels + 1):
            try:
                # the key side decides; the value side gets room to spare
                kvq.Plan(n_kv_heads, head_dim, M, 2, C, 8192, 128, alpha)
                feasible.append(M)
            except kvq.KvqError as e:
                if e.status != -2:
                    raise
        rows.append({"payload_bits": b, "container_bytes": C, "actual_payload_bits": round(bb, 6),
                     "feasible_levels": feasible, "max_levels_entropy": max(feasible) if feasible else None,
                     "max_levels_fixed_width_ideal": int(math.floor(2.0 ** bb + 1e-9)),
                     "max_levels_fixed_width_whole_bits": 1 << int(math.floor(bb + 1e-9))})
    return rows


def drift_study(plan, k, v, edges_bits=(0, 8, 16, 32, 64, 128, 256, 512, 1024, 4096)):
    """Figure 6 (right) analogue on the GPU path: encodes k, v [S, T, n] with
    the plan and returns, per side, the symbol counts, the number of symbols
    drift changed (against nearest rounding on the final grid, the encoder's
    counters), and every stream's remaining budget B - sum_i r(m_i) in the
    rates' fixed point (the quantity drift keeps non-negative, Eq. (6)), with
    a histogram over edges_bits (bits)."""
    S, T = int(k.shape[0]), int(k.shape[1])
    c = kvq.alloc_cache(plan, S, T)
    stats = torch.zeros(8, dtype=torch.int64, device="cuda")
    kvq.kvq_encode_streams(plan, k, v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                           c["k_mean_q"], c["k_mean_scale"], stats=stats)
    st = stats.cpu().tolist()
    out = {"streams_per_side": S * T, "values_per_stream": plan.n,
           "containers": [plan.params.container_bytes_k, plan.params.container_bytes_v],
           "levels": [plan.params.levels_k, plan.params.levels_v]}
    for side, key, name in ((0, "k_cont", "k"), (1, "v_cont", "v")):
        sym = torch.empty(S, T, plan.n, dtype=torch.uint8, device="cuda")
        kvq.kvq_decode_symbols(plan, side, c[key], sym)
        f, _, r = plan.tables(side)
        M = len(f)
        rate = torch.tensor(r, dtype=torch.int64, device="cuda")
        used = rate[sym.long()].sum(dim=-1).flatten()
        C = out["containers"][side]
        rem = (budget_fx(C) - used).cpu()
        counts = torch.bincount(sym.flatten().long(), minlength=M).cpu().tolist()
        rem_bits = rem.double() / RATE_ONE
        e = torch.tensor(list(edges_bits), dtype=torch.float64)
        hist = [int(((rem_bits >= e[i]) & (rem_bits < e[i + 1])).sum()) for i in range(len(e) - 1)]
        changed = st[2] if side == 0 else st[6]
        out[name] = {
            "symbol_counts": counts,
            "changed_symbols": int(changed),
            "changed_frac": changed / (S * T * plan.n),
            "fallbacks": int(st[0] + st[1]) if side == 0 else int(st[4] + st[5]),
            "overruns": int(st[3] if side == 0 else st[7]),
            "remaining_fx": [int(x) for x in rem.tolist()],
            "remaining_bits": {"min": float(rem_bits.min()), "median": float(rem_bits.median()),
                               "mean": float(rem_bits.mean()), "max": float(rem_bits.max()),
                               "below_8_bits_frac": float((rem_bits < 8).double().mean())},
            "remaining_hist": {"edges_bits": list(edges_bits), "counts": hist},
        }
    torch.cuda.synchronize()
    return out


def unpack_fw(cont, levels, n):
    """Symbols of fixed-width containers (the layout of kvq_encode_fixed_width)."""
    b = 1
    while (1 << b) < levels:
        b *= 2
    per = 8 // b
    i = torch.arange(n, device=cont.device)
    c, r = i // 4, i % 4
    byte = cont[..., (4 * (c // per) + r)].long()
    return (byte >> (b * (c % per))) & ((1 << b) - 1)


def run_fixed_width(sm, mk=6, mv=3):
    """The Appendix B comparator on the same sample: NMSE and attention error."""
    w = sm.w
    ck, cv = kvq.kvq_fixed_width_container_bytes(mk, w.n), kvq.kvq_fixed_width_container_bytes(mv, w.n)
    plan = kvq.Plan(w.n_kv_heads, w.head_dim, mk, mv, ck, cv, 128, 1.4)
    c = kvq.alloc_cache(plan, sm.S, sm.T)
    kvq.kvq_encode_fixed_width(plan, sm.k, sm.v, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                               c["k_mean_q"], c["k_mean_scale"])
    out = {"levels": [mk, mv], "containers": [ck, cv], "bits_per_elem": plan.bits_per_elem(True)}
    mu = (c["k_mean_q"].double() * c["k_mean_scale"].view(torch.float16).double()[..., None])
    mu_tok = mu.repeat_interleave(128, dim=1)
    for name, key, so_key, M, ref in (("k", "k_cont", "k_so", mk, sm.k_rot), ("v", "v_cont", "v_so", mv, sm.v_rot)):
        sym = unpack_fw(c[key], M, w.n).double()
        so = c[so_key].view(torch.float16).double()
        rec = so[..., 0:1] * sym + so[..., 1:2] + (mu_tok if name == "k" else 0.0)
        out[f"nmse_{name}"] = float(((rec - ref) ** 2).sum() / (ref ** 2).sum())
    o = torch.empty(sm.S, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty_like(o, dtype=torch.float32)
    ws = torch.empty(plan.workspace_bytes(1, sm.S, sm.T, w.n_q_heads), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attention_fixed_width(plan, sm.q, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                                         c["k_mean_q"], c["k_mean_scale"], o, ws, out_f32=o32)
    err = (o32.double() - sm.exact).norm(dim=-1) / sm.exact.norm(dim=-1)
    out["attn_rel_err"] = float(err.mean())
    torch.cuda.synchronize()
    return out


def fmt(x, spec=".4f"):
    return "—" if x is None else format(x, spec)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--seqs", type=int, default=16)
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--json", default=None)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.exit("the studies run the HIP library and need a GPU")
    sm = Sample(args.seqs, args.tokens)
    res = {"sample": f"gqa distribution, sequences 0..{args.seqs - 1}, {args.tokens} tokens each",
           "command": "python -m kv_cache_entropy_amd.studies " + " ".join(sys.argv[1:] if argv is None else argv),
           "device": torch.cuda.get_device_name(0)}
    print(f"# Synthetic studies ({res['sample']})\n")

    # Table 1 analogue: 8 levels, a container large enough that drift never acts
    t1 = run_config(sm, 8, 8, 400, 400)
    res["table1"] = t1
    print("## 8-level grids, no budget pressure (Table 1 analogue)\n")
    print("| side | NMSE | entropy H (bits) | coding gain log2 M − H | normal gap CE − H | sharpened-table gap |")
    print("|---|---:|---:|---:|---:|---:|")
    for s in ("k", "v"):
        print(f"| {s.upper()} | {t1['nmse_' + s]:.4%} | {t1['entropy_' + s]:.4f} | {t1['coding_gain_' + s]:.4f} | "
              f"{t1['model_gap_' + s]:.5f} | {t1['table_gap_' + s]:.5f} |")

    # Table 2 analogue: alphabet size at fixed containers
    print("\n## NMSE against the alphabet at K 331 B (2.68 bits/value) and V 231 B (1.84) (Table 2 analogue)\n")
    print("| levels | K NMSE | V NMSE |")
    print("|---:|---:|---:|")
    res["table2"] = []
    for M in (2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 14, 16):
        rk = run_config(sm, M, 2, 331, 231, attention=False)
        rv = run_config(sm, 2, M, 331, 231, attention=False)
        nk = rk["nmse_k"] if rk else None
        nv = rv["nmse_v"] if rv else None
        res["table2"].append({"levels": M, "nmse_k": nk, "nmse_v": nv})
        print(f"| {M} | {fmt(nk, '.4%')} | {fmt(nv, '.4%')} |")

    # Figure 4 middle analogue: budget sweep at 8/6 levels
    print("\n## Storage budget at 8/6 levels (Figure 4 middle analogue)\n")
    print("| bits/value | C_K/C_V | K NMSE | V NMSE | attention rel. error | K changed | V changed | kernel vs dequant |")
    print("|---:|---|---:|---:|---:|---:|---:|---:|")
    res["budget"] = []
    for b in (1.75, 2.0, 2.26, 2.5, 3.0, 3.5, 4.0):
        ck, cv = kvq.kvq_containers_for_budget(b, 8, 128, 128)
        r = run_config(sm, 8, 6, ck, cv)
        res["budget"].append(dict(budget=b, **(r or {})))
        if r is None:
            print(f"| {b} | {ck}/{cv} | — | — | — | — | — | — |")
            continue
        print(f"| {r['bits_per_elem']:.3f} | {ck}/{cv} | {r['nmse_k']:.4%} | {r['nmse_v']:.4%} | "
              f"{r['attn_rel_err']:.4%} | {r['changed_k']:.3%} | {r['changed_v']:.3%} | "
              f"{r['attn_kernel_vs_dequant']:.1e} |")

    # Figure 4 right analogue: K/V split at 2.26 bits per value
    print("\n## K/V split of 562 container bytes (2.26 bits/value) (Figure 4 right analogue)\n")
    print("| C_K/C_V | K NMSE | V NMSE | attention rel. error |")
    print("|---|---:|---:|---:|")
    res["split"] = []
    for ck in (251, 291, 331, 371, 411):
        cv = 562 - ck
        r = run_config(sm, 8, 6, ck, cv)
        res["split"].append(dict(ck=ck, cv=cv, **(r or {})))
        if r is None:
            print(f"| {ck}/{cv} | — | — | — |")
            continue
        print(f"| {ck}/{cv} | {r['nmse_k']:.4%} | {r['nmse_v']:.4%} | {r['attn_rel_err']:.4%} |")

    # Appendix C analogue: the default format
    d = next(r for r in res["budget"] if r["budget"] == 2.26)
    print("\n## Default format 331/231 B, 8/6 levels (Appendix C analogue)\n")
    print(f"* changed symbols after drift: K {d['changed_k']:.3%}, V {d['changed_v']:.3%}; "
          f"fallbacks {d['fallbacks']}")
    print(f"* extra rate of the analytic model over the measured symbol distribution: "
          f"K {d['model_gap_k']:.4f}, V {d['model_gap_v']:.4f} bits/value; of the sharpened "
          f"coding table: K {d['table_gap_k']:.4f}, V {d['table_gap_v']:.4f}")
    print(f"* measured K histogram {d['hist_k']}")
    print(f"* measured V histogram {d['hist_v']}")
    # Figure 6 analogues
    w = sm.w
    pay = [0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.25, 2.5, 2.75, 3.0, 3.5, 4.0]
    left = max_alphabet(w.n_kv_heads, w.head_dim, pay)
    res["figure6_left"] = left
    print("\n## Largest feasible alphabet against the payload (Figure 6 left analogue)\n")
    print("Feasible: every value of a stream fits at the cheapest level (n r_min <= 8C - 32 bits).\n")
    print("| payload bits/value | container bytes | entropy-coded max levels | fixed width, ideal log2 M | "
          "fixed width, whole bits |")
    print("|---:|---:|---:|---:|---:|")
    for r in left:
        print(f"| {r['actual_payload_bits']:.3f} | {r['container_bytes']} | {r['max_levels_entropy']} | "
              f"{r['max_levels_fixed_width_ideal']} | {r['max_levels_fixed_width_whole_bits']} |")
    res["figure6_right"] = []
    print("\n## Container budget left after drift (Figure 6 right analogue)\n")
    for ck, cv in ((331, 231), (292, 203)):
        plan = kvq.Plan(w.n_kv_heads, w.head_dim, 8, 6, ck, cv, 128, 1.4)
        ds = drift_study(plan, sm.k, sm.v)
        slim = {key: val for key, val in ds.items() if key not in ("k", "v")}
        for side in ("k", "v"):
            slim[side] = {key: val for key, val in ds[side].items() if key != "remaining_fx"}
        res["figure6_right"].append(slim)
        edges = ds["k"]["remaining_hist"]["edges_bits"]
        print(f"### {ck}/{cv} B, 8/6 levels ({plan.bits_per_elem(True):.3f} bits/value)\n")
        print("| remaining bits | " + " | ".join(f"[{edges[i]}, {edges[i + 1]})" for i in range(len(edges) - 1)) + " |")
        print("|---|" + "---:|" * (len(edges) - 1))
        for side in ("k", "v"):
            h = ds[side]["remaining_hist"]["counts"]
            tot = sum(h)
            print(f"| {side.upper()} streams | " + " | ".join(f"{x / tot:.1%}" for x in h) + " |")
        for side in ("k", "v"):
            d_ = ds[side]
            rb = d_["remaining_bits"]
            print(f"* {side.upper()}: changed symbols {d_['changed_frac']:.3%}, fallbacks {d_['fallbacks']}, "
                  f"remaining bits min {rb['min']:.2f} / median {rb['median']:.1f} / mean {rb['mean']:.1f}, "
                  f"streams with under 8 bits left {rb['below_8_bits_frac']:.1%}")
        print()
    # Appendix B analogue: the fixed-width comparator at 6/3 levels
    fw = run_fixed_width(sm)
    res["fixed_width"] = fw
    print("\n## Fixed-width comparator, nearest rounding at 6/3 levels (Appendix B analogue)\n")
    print("| format | levels | bytes K/V | stored bits/value | K NMSE | V NMSE | attention rel. error |")
    print("|---|---|---|---:|---:|---:|---:|")
    print(f"| entropy-coded | 8/6 | 331/231 | {d['bits_per_elem']:.3f} | {d['nmse_k']:.4%} | {d['nmse_v']:.4%} | "
          f"{d['attn_rel_err']:.4%} |")
    print(f"| fixed width | 6/3 | {fw['containers'][0]}/{fw['containers'][1]} | {fw['bits_per_elem']:.3f} | "
          f"{fw['nmse_k']:.4%} | {fw['nmse_v']:.4%} | {fw['attn_rel_err']:.4%} |")
    print("\n(The page charges the fixed-width format the ideal log2 6 + log2 3 bits, i.e. the same "
          "2.26 bits/value; stored at power-of-two widths it takes the bytes above.)")
    # non-affine levels: Lloyd-Max levels of min-max normalised Gaussian streams
    lk, lvv = lloyd_max_levels(8, sm.w.n), lloyd_max_levels(6, sm.w.n)
    res["non_affine"] = {"levels_k": lk, "levels_v": lvv, "rows": []}
    print("\n## Non-affine reconstruction levels (Lloyd-Max levels for min-max normalised Gaussian streams)\n")
    print(f"* K levels (grid units) {[round(x, 4) for x in lk]}")
    print(f"* V levels (grid units) {[round(x, 4) for x in lvv]}\n")
    print("| levels | C_K/C_V | K NMSE | V NMSE | attention rel. error | K changed | V changed | H_K | H_V |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|")
    for ck, cv in ((400, 400), (331, 231), (292, 203)):
        for name, vals in (("affine", (None, None)), ("Lloyd-Max", (lk, lvv))):
            r = run_config(sm, 8, 6, ck, cv, values=vals)
            res["non_affine"]["rows"].append(dict(kind=name, ck=ck, cv=cv, **(r or {})))
            if r is None:
                print(f"| {name} | {ck}/{cv} | — | — | — | — | — | — | — |")
                continue
            print(f"| {name} | {ck}/{cv} | {r['nmse_k']:.4%} | {r['nmse_v']:.4%} | {r['attn_rel_err']:.4%} | "
                  f"{r['changed_k']:.3%} | {r['changed_v']:.3%} | {r['entropy_k']:.4f} | {r['entropy_v']:.4f} |")
    if args.json:
        with open(args.json, "w") as fh:
            json.dump(res, fh, indent=1)


if __name__ == "__main__":
    main()
