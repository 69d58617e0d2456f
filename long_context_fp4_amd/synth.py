"""Seeded synthetic inputs for the cache-write and decode workloads.

This module only draws random inputs; it holds none of the cache method's
arithmetic (no merge, quantization, scoring, selection or attention). The
same arrays feed the HIP library and the CPU checker.

Draw order per workload seed (numpy ``default_rng``): merge weights of the
latent, merge weights of the indexer key, outlier channels, then per-layer
queries (latent query, indexer query, indexer head weights, Reuse noise).
Hidden states are drawn either on the host (numpy, small workloads) or on
the GPU with a seeded torch generator (large workloads); both are float32
N(0, 1) rounded to bfloat16 nearest-even.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

LATENT_CH = 512
INDEXER_CH = 128
BASE_SEED = 20261203


def bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def merge_weights(rng, m, channels):
    """Per-channel merge weights U(0,1), normalised over the m positions (float32)."""
    u = rng.random((m, channels), dtype=np.float32)
    total = u[0].copy()
    for j in range(1, m):
        total = total + u[j]
    return (u / total).astype(np.float32)


def outlier_channels(rng, channels, frac=0.01):
    n = int(round(frac * channels))
    return np.sort(rng.permutation(channels)[:n])


def hidden_host(rng, shape, outliers=None, scale=20.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if outliers is not None and len(outliers):
        x[..., outliers] *= np.float32(scale)
    return bf16_bits(x)


def hidden_device(gen, shape, outliers=None, scale=20.0):
    """Same distribution drawn on the GPU (torch is only the RNG and memory here)."""
    import torch
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    if outliers is not None and len(outliers):
        idx = torch.as_tensor(np.asarray(outliers), device="cuda", dtype=torch.long)
        x[..., idx] *= scale
    return x.to(torch.bfloat16).view(torch.int16)


def latent_query(rng, heads):
    return bf16_bits(rng.standard_normal((heads, LATENT_CH), dtype=np.float32)
                     / np.float32(np.sqrt(LATENT_CH)))


def indexer_query(rng, heads):
    return bf16_bits(rng.standard_normal((heads, INDEXER_CH), dtype=np.float32)
                     / np.float32(np.sqrt(INDEXER_CH)))


def head_weights(rng, heads):
    return rng.random(heads, dtype=np.float32)


def perturb(rng, q_bits, std):
    """bf16 query + N(0, std^2) noise, added in float32 and rounded back to bf16."""
    q = (q_bits.astype(np.uint32) << 16).view(np.float32)
    return bf16_bits(q + rng.standard_normal(q.shape, dtype=np.float32) * np.float32(std))


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    m: int
    T: int = 0                       # tokens per sequence (dense workloads)
    lengths: Optional[List[int]] = None   # tokens per sequence (ragged workloads)
    outliers: bool = False
    H: int = 64
    Hi: int = 16
    score_mode: int = 1              # 0 = dot (one head), 1 = sum_h w_h ReLU(q_h . k)
    k: int = 512
    pool_k: int = 0
    modes: List[int] = field(default_factory=lambda: [0])   # 0 Full, 1 Reindex, 2 Reuse
    reuse_std: float = 0.01

    def entries(self):
        lens = self.lengths if self.lengths is not None else [self.T] * self.B
        return [t // self.m for t in lens]


def workload(name):
    """The five workloads, by name, with their seeds."""
    if name == "tiny":
        return Workload(name, BASE_SEED + 0, B=1, m=2, T=4096, H=8, Hi=1, score_mode=0)
    if name == "write128k":
        return Workload(name, BASE_SEED + 1, B=8, m=2, T=131072, outliers=True, modes=[])
    if name == "decode128k":
        return Workload(name, BASE_SEED + 2, B=32, m=2, T=131072)
    if name == "hsi1m":
        return Workload(name, BASE_SEED + 3, B=4, m=2, T=1048576, pool_k=16384,
                        modes=[0, 1, 1])
    if name == "group_ragged":
        rng = np.random.default_rng(BASE_SEED + 4 + 1000)
        lengths = [int(v) for v in rng.integers(32768, 262144, size=16, endpoint=True)]
        return Workload(name, BASE_SEED + 4, B=16, m=1, lengths=lengths, pool_k=16384,
                        modes=[0, 1, 2, 2])
    raise KeyError(name)


def params(w: Workload):
    """Small host-side parameters of a workload: merge weights, outliers, per-layer queries."""
    rng = np.random.default_rng(w.seed)
    p = {
        "w_lat": merge_weights(rng, w.m, LATENT_CH),
        "w_idx": merge_weights(rng, w.m, INDEXER_CH),
        "out_lat": outlier_channels(rng, LATENT_CH) if w.outliers else None,
        "out_idx": outlier_channels(rng, INDEXER_CH) if w.outliers else None,
        "layers": [],
    }
    prev_q = None
    for mode in w.modes:
        L = {"mode": mode, "score_mode": w.score_mode}
        if mode == 2:
            L["q"] = np.stack([perturb(rng, prev_q[b], w.reuse_std) for b in range(w.B)])
        else:
            L["q"] = np.stack([latent_query(rng, w.H) for _ in range(w.B)])
            L["q_idx"] = np.stack([indexer_query(rng, w.Hi) for _ in range(w.B)])
            L["w"] = (np.stack([head_weights(rng, w.Hi) for _ in range(w.B)])
                      if w.score_mode == 1 else None)
        prev_q = L["q"]
        p["layers"].append(L)
    return p


def hidden_states_host(w: Workload, p):
    """Host hidden states per sequence: list of (x_lat [T,512], x_idx [T,128]) bf16 bits."""
    rng = np.random.default_rng(w.seed + 500)
    lens = w.lengths if w.lengths is not None else [w.T] * w.B
    return [(hidden_host(rng, (t, LATENT_CH), p["out_lat"]),
             hidden_host(rng, (t, INDEXER_CH), p["out_idx"])) for t in lens]


def hidden_states_device(w: Workload, p, seq):
    """Device hidden states of one sequence (seeded per sequence), as int16 torch tensors."""
    import torch
    t = w.lengths[seq] if w.lengths is not None else w.T
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed * 1000 + seq)
    x_lat = hidden_device(g, (t, LATENT_CH), p["out_lat"])
    x_idx = hidden_device(g, (t, INDEXER_CH), p["out_idx"])
    return x_lat, x_idx
