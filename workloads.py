"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers: it holds none of the method's
arithmetic.  The pages measure on long-context reasoning datasets with a
Qwen3-8B model; neither is available here, so clustered-Gaussian KV caches with
that model's attention-layer shape (32 query heads, 8 KV heads, head dim 128)
stand in for them.

Recipe (one torch CPU generator per sequence, so sequences can be drawn one at
a time and any subset reproduces the same bits):
  * per (sequence, KV head): M component means ~ N(0, I_d); each token picks a
    component uniformly; key = mean + sigma * N(0, I_d); value ~ N(0, I_d);
  * optional outliers: `outlier_channels` distinct channels per KV head (by
    randperm) are multiplied by `outlier_scale` on the whole key;
  * optional drift for generated blocks: the means move by drift * N(0, I_d)
    before each appended block;
  * query of (sequence, query head): a uniformly chosen component mean of its
    KV head (before outlier scaling) + 0.1 * N(0, I_d);
  * draws are float32, rounded once to the storage dtype.
Seeds: data 1000 * config_index + b, queries 2000 * config_index + step.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                  # position in the list of configurations
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int               # prompt tokens clustered by the build
    components: int             # mixture components per KV head
    sigma: float = 0.3
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    dtype: torch.dtype = torch.bfloat16
    tokens_per_centroid: int = 16
    cluster_block: int = 8192
    build_iters: int = 10
    update_iters: int = 5
    budgets: Sequence[int] = (128,)
    steps: int = 1
    generated_blocks: int = 0   # appended blocks (online update)
    drift: float = 0.0
    coarse_tokens_per_centroid: int = 0
    coarse_candidate_tokens: int = 0

    @property
    def capacity(self) -> int:
        return self.n_tokens + self.generated_blocks * self.cluster_block

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-fp32", 0, 1, 1, 1, 128, 4096, 256, dtype=torch.float32, budgets=(128,)),
        Workload("qwen3-8b-layer-b1-32k", 1, 1, 32, 8, 128, 32768, 2048, outlier_channels=4,
                 budgets=(128, 512), steps=100),
        Workload("qwen3-8b-layer-b16-32k-s95", 2, 16, 32, 8, 128, 32768, 2048, outlier_channels=4,
                 budgets=(1638,), steps=100),
        Workload("qwen3-8b-layer-b4-online", 3, 4, 32, 8, 128, 16384, 2048, outlier_channels=4,
                 budgets=(128,), steps=10, generated_blocks=2, drift=0.2),
        Workload("qwen3-8b-layer-b4-128k-hier", 4, 4, 32, 8, 128, 131072, 2048, outlier_channels=4,
                 budgets=(512,), steps=10, coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096),
    ]
}
BY_INDEX = {w.index: w for w in WORKLOADS.values()}


@dataclass
class Sequence_:
    """One sequence's cache: K, V [Hkv][capacity][d] and the mixture means of
    each appended phase [phases][Hkv][M][d] (phase 0 = prompt)."""
    K: torch.Tensor
    V: torch.Tensor
    means: List[torch.Tensor] = field(default_factory=list)


def make_sequence(w: Workload, b: int, n_tokens: Optional[int] = None, components: Optional[int] = None
                  ) -> Sequence_:
    """Draws sequence b of workload w (prompt + appended blocks)."""
    g = torch.Generator("cpu").manual_seed(1000 * w.index + b)
    H, d = w.n_kv_heads, w.head_dim
    M = components or w.components
    n_prompt = n_tokens if n_tokens is not None else w.n_tokens
    cap = n_prompt + w.generated_blocks * w.cluster_block
    K = torch.empty(H, cap, d, dtype=torch.float32)
    V = torch.empty(H, cap, d, dtype=torch.float32)
    means = torch.randn(H, M, d, generator=g)
    scale = torch.ones(H, d)
    if w.outlier_channels:
        for h in range(H):
            ch = torch.randperm(d, generator=g)[: w.outlier_channels]
            scale[h, ch] = w.outlier_scale
    phases = [(0, n_prompt)] + [(n_prompt + k * w.cluster_block, w.cluster_block)
                                for k in range(w.generated_blocks)]
    all_means = []
    for ph, (p, L) in enumerate(phases):
        if ph > 0:
            means = means + w.drift * torch.randn(H, M, d, generator=g)
        all_means.append(means.clone())
        z = torch.randint(0, M, (H, L), generator=g)
        noise = torch.randn(H, L, d, generator=g)
        keys = torch.gather(means, 1, z.unsqueeze(-1).expand(H, L, d)) + w.sigma * noise
        K[:, p:p + L] = keys * scale[:, None, :]
        V[:, p:p + L] = torch.randn(H, L, d, generator=g)
    return Sequence_(K.to(w.dtype), V.to(w.dtype), all_means)


def make_cache(w: Workload, batch_ids: Optional[Sequence[int]] = None, n_tokens: Optional[int] = None,
               components: Optional[int] = None):
    """K, V [len(batch_ids)][Hkv][capacity][d] (storage dtype) and the list of
    per-sequence means."""
    ids = list(range(w.batch)) if batch_ids is None else list(batch_ids)
    seqs = [make_sequence(w, b, n_tokens, components) for b in ids]
    K = torch.stack([s.K for s in seqs])
    V = torch.stack([s.V for s in seqs])
    return K, V, [s.means for s in seqs]


def make_queries(w: Workload, means: List[List[torch.Tensor]], step: int, phase: int = -1,
                 group_shared: bool = False) -> torch.Tensor:
    """q [B][Hq][d]: a random component mean of the head's KV group (of the
    given mixture phase, default the latest) + 0.1 * N(0, I).  Each query
    head draws its own component; with group_shared the G heads of a group
    draw one component together (and their own noise)."""
    g = torch.Generator("cpu").manual_seed(2000 * w.index + step + (1000 if group_shared else 0))
    B = len(means)
    G = w.n_q_heads // w.n_kv_heads
    q = torch.empty(B, w.n_q_heads, w.head_dim, dtype=torch.float32)
    for b in range(B):
        mu = means[b][phase]
        M = mu.shape[1]
        m = 0
        for hq in range(w.n_q_heads):
            if not group_shared or hq % G == 0:
                m = int(torch.randint(0, M, (1,), generator=g))
            q[b, hq] = mu[hq // G, m] + 0.1 * torch.randn(w.head_dim, generator=g)
    return q.to(w.dtype)


def randn(shape, seed: int, dtype=torch.float32) -> torch.Tensor:
    """Plain seeded N(0, 1) draws (float32, then rounded to dtype)."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)
