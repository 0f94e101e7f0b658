"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

The page measures on KV captured from trained 8B models running long-context
benchmarks; none of that is available here, so these generators stand in for
it with the page's shapes (8 KV heads x d = 128 = one 1024-value group per
token, 32 layers, 32 query heads for the Llama-3-8B-shaped case) and the
post-preprocessing statistics it describes (near-Gaussian, plus one-coordinate
key spikes for the heavy-tailed stress case).

Every sequence s (= layer * batch + b) is generated from its own seeded torch
generator, so any subset can be regenerated on its own; values are produced
in fp32 and rounded to bf16 (round-to-nearest-even) except for the Tiny case,
which is fp32 from numpy's PCG64.
"""

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    batch: int
    layers: int
    seq_len: int
    seed: int
    dist: str
    containers: tuple = ((331, 231),)   # (C_K, C_V) per budget
    budgets: tuple = (2.26,)
    dtype: str = "bf16"

    @property
    def n_seqs(self):
        return self.layers * self.batch

    @property
    def n(self):
        return self.n_kv_heads * self.head_dim


WORKLOADS = {
    # 1 q head / 1 KV head, d = 128, 256 tokens, fp32, 36-byte containers
    "tiny": Workload("tiny", 1, 1, 128, 1, 1, 256, 0, "tiny", ((36, 36),), (2.25,), "f32"),
    # Llama-3-8B-shaped GQA decode: 32/8 heads, batch 16, 8192 tokens, 32 layers
    "gqa": Workload("gqa", 32, 8, 128, 16, 32, 8192, 1, "keymeans"),
    # long context: batch 4, 32768 tokens, 32 layers, budgets 2.0 / 2.26 / 3.0
    "long": Workload("long", 32, 8, 128, 4, 32, 32768, 2, "keymeans",
                     ((292, 203), (331, 231), (442, 309)), (2.0, 2.26, 3.0)),
    # very long context: 64/8 heads, batch 1, 131072 tokens, one layer
    "verylong": Workload("verylong", 64, 8, 128, 1, 1, 131072, 3, "gauss"),
    # heavy-tailed stress: 32/8, batch 8, 4096 tokens, one layer, budgets 2/3/4
    "heavy": Workload("heavy", 32, 8, 128, 8, 1, 4096, 4, "heavy",
                      ((292, 203), (442, 309), (593, 414)), (2.0, 3.0, 4.0)),
}

N_SPIKE_CHANNELS = 10      # round(1% of 1024 key channels)


def _gen(device, *key):
    g = torch.Generator(device=device)
    h = 0
    for k in key:
        h = (h * 1000003 + int(k) + 1) % (2 ** 62)
    g.manual_seed(h)
    return g


def _tiny_numpy(w):
    rng = np.random.default_rng(w.seed)
    mu = rng.normal(0.0, 0.5, w.n).astype(np.float32)
    k = (rng.standard_normal((w.seq_len, w.n)) + mu).astype(np.float32)
    v = rng.standard_normal((w.seq_len, w.n)).astype(np.float32)
    q = rng.standard_normal((w.n_q_heads, w.head_dim)).astype(np.float32)
    return k, v, q


def spike_channels(w, device="cpu"):
    g = _gen("cpu", w.seed, 77)
    return torch.randperm(w.n, generator=g)[:N_SPIKE_CHANNELS].to(device)


def sequence_kv(w, s, device, tokens=None):
    """K and V of sequence s as [T', n] tensors (bf16, or fp32 for Tiny).

    tokens=(t0, t1) generates the whole sequence and returns that slice (the
    values do not depend on the slice)."""
    T, n = w.seq_len, w.n
    if w.dist == "tiny":
        k, v, _ = _tiny_numpy(w)
        k, v = torch.from_numpy(k).to(device), torch.from_numpy(v).to(device)
    else:
        g = _gen(device, w.seed, s, 1)
        if w.dist == "keymeans":
            layer = s // w.batch
            gl = _gen(device, w.seed, layer, 2)
            mu = torch.randn(n, generator=gl, device=device)
            sig = 0.5 + 1.5 * torch.rand(n, generator=gl, device=device)
            k = mu + sig * torch.randn(T, n, generator=g, device=device)
            v = torch.randn(T, n, generator=g, device=device)
        elif w.dist == "gauss":
            k = torch.randn(T, n, generator=g, device=device)
            v = torch.randn(T, n, generator=g, device=device)
        elif w.dist == "heavy":
            def student_t4():
                # t(4) = z0 / sqrt((z1^2 + ... + z4^2) / 4), every step one
                # correctly rounded IEEE operation, so that the CPU generator
                # gives the same bits on every host (a library reduction may
                # group the terms differently, a vectorised sqrt may round
                # differently)
                z = torch.randn(5, T, n, generator=g, device=device)
                ss = z[1] * z[1]
                for i in (2, 3, 4):
                    ss = ss + z[i] * z[i]
                ss = ss / 4.0
                if ss.device.type == "cpu":
                    # the hardware square root (correctly rounded on every x86
                    # host); a library's vectorised sqrt need not be
                    den = torch.from_numpy(np.sqrt(ss.numpy()))
                else:
                    den = torch.sqrt(ss)
                return z[0] / den
            k = student_t4()
            v = student_t4()
            ch = spike_channels(w, device)
            pick = torch.randint(0, N_SPIKE_CHANNELS, (T,), generator=g, device=device)
            sign = torch.randint(0, 2, (T,), generator=g, device=device).float() * 2 - 1
            mag = 20.0 + 30.0 * torch.rand(T, generator=g, device=device)
            k[torch.arange(T, device=device), ch[pick]] = sign * mag
        else:
            raise ValueError(w.dist)
        k = k.to(torch.bfloat16)
        v = v.to(torch.bfloat16)
    if tokens is not None:
        k, v = k[tokens[0]:tokens[1]], v[tokens[0]:tokens[1]]
    return k.contiguous(), v.contiguous()


def queries(w, device, seqs=None):
    """Decode queries [S', Hq, d] bf16 for the given sequences (default all)."""
    seqs = range(w.n_seqs) if seqs is None else seqs
    if w.dist == "tiny":
        _, _, q = _tiny_numpy(w)
        return torch.from_numpy(q)[None].to(torch.bfloat16).to(device)
    out = []
    for s in seqs:
        g = _gen(device, w.seed, s, 3)
        out.append(torch.randn(w.n_q_heads, w.head_dim, generator=g, device=device))
    return torch.stack(out).to(torch.bfloat16).contiguous()


def cache_inputs(w, device, seqs=None, tokens=None):
    """Stacked K, V [S', T', n] for the given sequences."""
    seqs = range(w.n_seqs) if seqs is None else seqs
    ks, vs = zip(*(sequence_kv(w, s, device, tokens) for s in seqs))
    return torch.stack(ks).contiguous(), torch.stack(vs).contiguous()
