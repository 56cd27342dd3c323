"""The teacher-forced check of the hierarchy's coarse level (the one the GPU
tests apply to the GPU's coarse build) accepts the oracle's own coarse
rounds and rejects the mistakes a coarse build could make: an unweighted
value-centroid mean, a wrong parent, a stored centroid off by one unit in
the last place, a wrong coarse size, a wrong member order.  CPU only: the
"GPU state" here is the oracle's state held in float64 tensors."""
import copy
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from gpu_util import check_coarse_round

N, BC, TPC, CTPC, K_ITERS = 4096, 2048, 16, 128, 3


def _params():
    return SimpleNamespace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, dtype=torch.bfloat16,
                           capacity_tokens=N, tokens_per_centroid=TPC, cluster_block=BC,
                           coarse_tokens_per_centroid=CTPC, hierarchical=True)


def _fake_state(st):
    """An oracle UnitState in the layout of a device ClusterState (float64
    tensors, so nothing is rounded on the way)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    C, D = st.n_clusters, st.n_coarse
    return SimpleNamespace(
        n_clusters=C, n_clustered=st.n_clustered, n_coarse=D, capacity_clusters=st.capacity_clusters,
        key_centroids=t(st.kbar), value_centroids=t(st.vbar), key_centroids_f32=t(st.mu),
        sizes=t(st.sizes), offsets=t(st.offsets), token_ids=t(st.token_ids), assign=t(st.assign),
        coarse_key_centroids=t(st.ckbar), coarse_value_centroids=t(st.cvbar), coarse_key_centroids_f32=t(st.cmu),
        coarse_sizes=t(st.csizes), coarse_offsets=t(st.coffsets), coarse_members=t(st.cmembers),
        parent=t(st.parent))


@pytest.fixture(scope="module")
def states():
    K = workloads.randn((N, 128), 31)
    means = workloads.randn((64, 128), 32)
    K = (means[torch.randint(0, 64, (N,), generator=torch.Generator().manual_seed(33))] + 0.3 * K)
    K = K.to(torch.bfloat16)
    V = workloads.randn((N, 128), 34).to(torch.bfloat16)
    out = {}
    for iters in (1, K_ITERS - 1, K_ITERS):
        st = O.build_unit(K, V, N, tokens_per_centroid=TPC, cluster_block_size=BC, iters=3, storage=O.BF16, seed=5)
        O.build_coarse(st, coarse_tokens_per_centroid=CTPC, iters=iters, seed=5, unit=0)
        out[iters] = st
    return out


def test_accepts_the_oracles_rounds(states):
    p = _params()
    check_coarse_round(p, _fake_state(states[K_ITERS - 1]), _fake_state(states[K_ITERS]), 0, 0, seed=5)
    check_coarse_round(p, None, _fake_state(states[1]), 0, 0, seed=5, from_init=True)


def _planted(states, mutate):
    cur = copy.deepcopy(states[K_ITERS])
    mutate(cur)
    return _fake_state(cur)


def test_rejects_an_unweighted_value_mean(states):
    def unweighted(st):
        for g in range(st.n_coarse):
            mem = st.cmembers[st.coffsets[g]:st.coffsets[g + 1]]
            if len(mem):
                st.cvbar[g] = O.round_storage(st.vbar[mem].mean(0), O.BF16)
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), _fake_state(states[K_ITERS - 1]), _planted(states, unweighted), 0, 0, seed=5)


def test_rejects_a_wrong_parent(states):
    def move(st):
        i = int(np.nonzero(st.parent >= 0)[0][7])
        g = st.parent[i]
        st.parent[i] = g + 1 if (g + 1) % (BC // CTPC) else g - 1
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), _fake_state(states[K_ITERS - 1]), _planted(states, move), 0, 0, seed=5)


def test_rejects_a_stored_centroid_one_ulp_off(states):
    def ulp(st):
        x = st.ckbar[3, 5]
        st.ckbar[3, 5] = x + abs(x) * 2.0 ** -7
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), _fake_state(states[K_ITERS - 1]), _planted(states, ulp), 0, 0, seed=5)


def test_rejects_a_wrong_size(states):
    def size(st):
        st.csizes[2] += 1
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), _fake_state(states[K_ITERS - 1]), _planted(states, size), 0, 0, seed=5)


def test_rejects_a_wrong_member_order(states):
    def order(st):
        a, b = st.coffsets[4], st.coffsets[5]
        assert b - a >= 2
        st.cmembers[a], st.cmembers[a + 1] = st.cmembers[a + 1], st.cmembers[a]
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), _fake_state(states[K_ITERS - 1]), _planted(states, order), 0, 0, seed=5)


def test_rejects_a_wrong_init(states):
    with pytest.raises(AssertionError):
        check_coarse_round(_params(), None, _fake_state(states[1]), 0, 0, seed=6, from_init=True)
