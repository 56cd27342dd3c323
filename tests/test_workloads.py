"""The seeded input generators: reproducible, and the two query recipes
have the structure they claim (CPU only, small draws)."""
import dataclasses

import torch

import workloads


def _small(**kw):
    base = workloads.WORKLOADS["qwen3-8b-layer-b1-32k"]
    return dataclasses.replace(base, name="t", index=77, batch=2, n_tokens=512, components=8, **kw)


def test_draws_are_reproducible_and_per_sequence():
    w = _small()
    K, V, means = workloads.make_cache(w)
    K2, V2, _ = workloads.make_cache(w)
    assert torch.equal(K, K2) and torch.equal(V, V2)
    K1, _, _ = workloads.make_cache(w, batch_ids=[1])
    assert torch.equal(K1[0], K[1])
    assert torch.equal(workloads.make_queries(w, means, 3), workloads.make_queries(w, means, 3))
    assert not torch.equal(workloads.make_queries(w, means, 3), workloads.make_queries(w, means, 4))


def test_query_recipes():
    """A query lies 0.1 * N(0, I) from one component mean of its KV head;
    with group_shared all heads of a group share the component."""
    w = _small()
    _, _, means = workloads.make_cache(w)
    G = w.n_q_heads // w.n_kv_heads
    for shared in (False, True):
        q = workloads.make_queries(w, means, 0, group_shared=shared).float()
        comps = torch.empty(w.batch, w.n_q_heads, dtype=torch.long)
        for b in range(w.batch):
            for hq in range(w.n_q_heads):
                dist = (means[b][-1][hq // G] - q[b, hq]).norm(dim=-1)
                comps[b, hq] = int(dist.argmin())
                # 0.1 * chi(128) ~ 1.13, plus bf16 rounding; other means are ~16 away
                assert dist.min() < 2.0 and dist.sort().values[1] > 8.0
        same = (comps.view(w.batch, w.n_kv_heads, G) == comps.view(w.batch, w.n_kv_heads, G)[..., :1]).all(-1)
        if shared:
            assert bool(same.all())
        else:
            assert not bool(same.all())
