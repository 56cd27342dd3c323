"""The allocation-free decode (mpattn_decode_noalloc, its workspace a device
array of the library) against mpattn_decode with a caller workspace: the
same outputs on consecutive calls, a later call with a smaller input and
another layout (the array is cleared), calls repeated on one layout (the
array keeps its tags), and the split-launch and hierarchical paths."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def M():
    from sparse_long_context_means_amd import mpattn

    return mpattn


def _case(B, Hq, Hkv, N, hier=False, seed=1):
    mp = M()
    base = workloads.WORKLOADS["qwen3-8b-layer-b1-32k"]
    import dataclasses
    w = dataclasses.replace(base, name="noalloc", index=97, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_tokens=N,
                            components=max(8, N // 16))
    K, V, means = workloads.make_cache(w)
    kw = dict(coarse_tokens_per_centroid=128, coarse_candidate_tokens=2048) if hier else {}
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=2048, build_iters=3,
                  seed=seed, **kw)
    st = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, N, st)
    return mp, w, means, p, st, Kd, Vd


def _check(mp, w, means, p, st, Kd, Vd, step, T, n_total=None):
    n_total = n_total or p.capacity_tokens
    q = workloads.make_queries(w, means, step).to(DEV)
    ws = mp.Workspace().get(p, st, DEV)
    ref = mp.decode(p, q, Kd, Vd, n_total, st, T, workspace=ws).clone()
    out = torch.full_like(ref, float("nan"))
    mp.decode_noalloc(p, q, Kd, Vd, n_total, st, T, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    o, r = out.cpu().numpy(), ref.cpu().numpy()
    assert np.all(np.abs(o - r) <= 2e-3 + 1e-2 * np.abs(r)), float(np.abs(o - r).max())
    # the same kernels on the same inputs: the same bits
    assert torch.equal(out, ref)


def test_noalloc_matches_decode_on_consecutive_calls():
    mp, w, means, p, st, Kd, Vd = _case(16, 32, 8, 6000)
    assert p.decode_stages() == ["unit"]
    _check(mp, w, means, p, st, Kd, Vd, 0, 700)
    _check(mp, w, means, p, st, Kd, Vd, 1, 300)
    # a smaller input of another layout: fewer sequences and tokens
    mp2, w2, means2, p2, st2, Kd2, Vd2 = _case(8, 16, 4, 3000, seed=2)
    assert p2.decode_stages() == ["unit"]
    _check(mp2, w2, means2, p2, st2, Kd2, Vd2, 2, 200)
    _check(mp2, w2, means2, p2, st2, Kd2, Vd2, 3, 200)
    # back to the first layout
    _check(mp, w, means, p, st, Kd, Vd, 4, 1000)


def test_noalloc_split_and_hierarchical_paths():
    mp, w, means, p, st, Kd, Vd = _case(1, 8, 2, 5000)
    assert p.decode_stages() == ["score", "select", "attend", "merge"]
    _check(mp, w, means, p, st, Kd, Vd, 0, 400)
    mph, wh, meansh, ph, sth, Kdh, Vdh = _case(4, 32, 8, 8192, hier=True)
    assert ph.decode_stages() == ["hier_unit"]
    _check(mph, wh, meansh, ph, sth, Kdh, Vdh, 1, 512)
    _check(mph, wh, meansh, ph, sth, Kdh, Vdh, 2, 300)
    _check(mp, w, means, p, st, Kd, Vd, 3, 100)


def test_noalloc_serves_the_batch16_32k_layout():
    """The layout of a Qwen3-8B-shaped layer at batch 16 and 32768 tokens
    (128 units of 2048 clusters, about 39 MiB of decode workspace) fits the
    library's array: the same bits as mpattn_decode on two steps."""
    mp, w, means, p, st, Kd, Vd = _case(16, 32, 8, 32768)
    assert p.decode_stages() == ["unit"]
    import ctypes
    need = mp.lib.mpattn_workspace_bytes(ctypes.byref(p.c()), st.capacity_clusters, st.capacity_coarse,
                                         mp.OP_DECODE)
    assert 32 << 20 < need <= mp.lib.mpattn_decode_noalloc_max_bytes()
    _check(mp, w, means, p, st, Kd, Vd, 0, 1638)
    _check(mp, w, means, p, st, Kd, Vd, 1, 1638)
