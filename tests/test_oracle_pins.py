"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test ties the oracle to something other than itself: published generator
outputs, hand-derived values (tests/golden), library routines (torch's
float32->bfloat16 conversion, scipy's nearest-centroid search, scikit-learn's
Lloyd k-means, torch's scaled-dot-product attention), closed forms, invariants
and brute force on tiny inputs.  No GPU is needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# generator and rounding
# ---------------------------------------------------------------------------

def test_splitmix64_published_outputs(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "splitmix64.json")))
    for case in g["cases"]:
        for t, v in enumerate(case["outputs"]):
            assert O.sm64_draw(case["state"], t) == int(v, 0)


@pytest.mark.parametrize("n,count", [(1, 1), (7, 7), (100, 13), (8192, 512), (4096, 256)])
def test_init_indices_distinct_in_range(n, count):
    for seed in range(5):
        idx = O.init_indices(O.block_stream(seed, 3, 1), n, count)
        assert len(set(idx.tolist())) == count
        assert idx.min() >= 0 and idx.max() < n
        if count == n:
            assert sorted(idx.tolist()) == list(range(n))


def test_init_indices_roughly_uniform():
    # first pick of a 10-way draw over 20000 streams: chi-square with 9 dof
    n, trials = 10, 20000
    hist = np.zeros(n)
    for s in range(trials):
        hist[O.init_indices(O.block_stream(s, 0, 0), n, 1)[0]] += 1
    exp = trials / n
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 27.9  # p ~ 0.001


def test_block_streams_differ():
    keys = {O.block_stream(0, u, j, lv) for u in range(4) for j in range(4) for lv in range(2)}
    assert len(keys) == 32


def test_bf16_rounding_matches_torch():
    r = _rng(0)
    x = (r.standard_normal(20000) * np.exp(r.uniform(-30, 30, 20000))).astype(np.float32)
    # exact ties: low 16 bits equal to 0x8000 (round half to even)
    bits = r.integers(0, 2**31, 4000, dtype=np.int64).astype(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    sub = (r.standard_normal(2000) * 1e-39).astype(np.float32)  # binary32 subnormals
    for arr in (x, ties, sub):
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        got = O.round_storage(arr.astype(np.float64), O.BF16)
        np.testing.assert_array_equal(got, want)


def test_f32_rounding_matches_numpy():
    x = _rng(1).standard_normal(10000) * 1e3
    np.testing.assert_array_equal(O.round_storage(x, O.F32), x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(O.round_storage(x, O.EXACT), x)


# ---------------------------------------------------------------------------
# k-means
# ---------------------------------------------------------------------------

def test_assign_matches_scipy_vq():
    from scipy.cluster.vq import vq

    r = _rng(2)
    x = r.standard_normal((500, 16))
    mu = r.standard_normal((37, 16))
    a, bd, J = O.assign_step(x, mu)
    codes, dist = vq(x, mu)
    np.testing.assert_array_equal(a, codes)
    np.testing.assert_allclose(bd, dist ** 2, rtol=1e-12)
    assert abs(J - (dist ** 2).sum()) < 1e-9 * J


def test_assign_ties_go_to_lowest_index():
    x = np.array([[0.0, 0.0], [1.0, 1.0]])
    mu = np.array([[5.0, 5.0], [1.0, 1.0], [1.0, 1.0], [-1.0, -1.0]])
    a, _, _ = O.assign_step(x, mu)
    # point 0 is equidistant from centroids 1, 2 and 3 -> 1; point 1 sits on 1 and 2 -> 1
    assert a.tolist() == [1, 1]


def test_lloyd_hand_worked_trace(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_lloyd.json")))
    x = np.array(g["points"], dtype=np.float64)
    mu, mu_s, a, counts, J = O.kmeans(x, g["clusters"], g["iters"], O.EXACT, g["init_indices"])
    np.testing.assert_allclose(J, g["objective"], rtol=1e-14)
    assert a.tolist() == g["assign_after"]
    np.testing.assert_allclose(mu, g["centroids_after"], rtol=1e-14)
    np.testing.assert_array_equal(mu, mu_s)


@pytest.mark.parametrize("iters", [1, 3, 12])
def test_lloyd_matches_sklearn(iters):
    from sklearn.cluster import KMeans

    for seed in range(20):
        r = _rng(100 + seed)
        centers = r.standard_normal((6, 8)) * 3
        x = np.concatenate([c + r.standard_normal((40, 8)) for c in centers])
        init = r.choice(len(x), 6, replace=False).astype(np.int32)
        # skip draws in which some cluster empties (scikit-learn relocates those)
        mu_s = x[init].copy()
        mu = mu_s.copy()
        ok = True
        for _ in range(iters):
            a, _, _ = O.assign_step(x, mu_s)
            mu, mu_s, counts = O.update_step(x, a, mu, mu_s, O.EXACT)
            ok &= bool((counts > 0).all())
        if not ok:
            continue
        got, _, _, _, _ = O.kmeans(x, 6, iters, O.EXACT, init)
        km = KMeans(n_clusters=6, init=x[init], n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd").fit(x)
        np.testing.assert_allclose(got, km.cluster_centers_, rtol=1e-10, atol=1e-10)
        return
    pytest.fail("no draw without empty clusters")


def test_objective_non_increasing_exact():
    for seed in range(10):
        r = _rng(200 + seed)
        x = r.standard_normal((300, 12))
        C = 40  # many clusters: some empty out and keep their centroid
        init = O.init_indices(O.block_stream(seed, 0, 0), 300, C)
        _, _, _, _, J = O.kmeans(x, C, 15, O.EXACT, init)
        assert np.all(np.diff(J) <= 1e-12 * J[:-1])


def test_objective_bf16_rounding_bound():
    # J_{t+1} <= J_t + sum_i (2 |k_i - mu_a| |delta_a| + |delta_a|^2), delta = stored - exact mean
    r = _rng(3)
    x = O.round_storage(r.standard_normal((400, 16)) * 4, O.BF16)
    C = 30
    init = O.init_indices(O.block_stream(1, 0, 0), 400, C)
    mu_s = x[init].copy()
    mu = mu_s.copy()
    a, _, J_prev = O.assign_step(x, mu_s)
    for _ in range(10):
        mu, mu_s, counts = O.update_step(x, a, mu, mu_s, O.BF16)
        delta = np.linalg.norm(mu_s - mu, axis=1)
        dist = np.linalg.norm(x - mu[a], axis=1)
        bound = J_prev + (2 * dist * delta[a] + delta[a] ** 2).sum()
        a, _, J = O.assign_step(x, mu_s)
        assert J <= bound * (1 + 1e-12)
        J_prev = J


def test_bruteforce_global_optimum_tiny():
    # all 3^9 labelings of 9 points into 3 non-empty groups
    r = _rng(4)
    groups = np.array([[0, 0], [10, 0], [0, 10]], dtype=np.float64)
    x = np.concatenate([g + 0.3 * r.standard_normal((3, 2)) for g in groups])
    best = math.inf
    for lab in itertools.product(range(3), repeat=len(x)):
        lab = np.array(lab)
        if len(set(lab.tolist())) < 3:
            continue
        J = sum(((x[lab == c] - x[lab == c].mean(0)) ** 2).sum() for c in range(3))
        best = min(best, J)
    # Lloyd from any seeding is at least the optimum; seeded one per group it reaches it
    for init in ([0, 3, 6], [0, 1, 2], [2, 5, 8], [4, 5, 7]):
        mu, _, a, counts, J = O.kmeans(x, 3, 20, O.EXACT, init)
        final = sum(((x[a == c] - mu[c]) ** 2).sum() for c in range(3) if counts[c] > 0)
        assert final >= best - 1e-9
        if init in ([0, 3, 6], [2, 5, 8]):
            assert abs(final - best) < 1e-9
        # fixed point: every point sits at its nearest final centroid
        a2, _, _ = O.assign_step(x, mu)
        np.testing.assert_array_equal(a2, a)


def test_permutation_invariance_kmeans():
    r = _rng(5)
    x = r.standard_normal((200, 8))
    init = O.init_indices(O.block_stream(2, 0, 0), 200, 12)
    mu, mu_s, a, counts, J = O.kmeans(x, 12, 8, O.BF16, init)
    perm = r.permutation(200)
    inv = np.argsort(perm)
    mu2, mu_s2, a2, counts2, J2 = O.kmeans(x[perm], 12, 8, O.BF16, inv[init])
    np.testing.assert_allclose(mu2, mu, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(a2, a[perm])
    np.testing.assert_array_equal(counts2, counts)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def test_selection_is_longest_fitting_prefix():
    r = _rng(6)
    for trial in range(200):
        C = int(r.integers(1, 60))
        key = np.round(r.standard_normal(C), 1)  # many exact ties
        sizes = r.integers(0, 6, C).astype(np.int32)
        T = int(r.integers(0, 60))
        sel, taken = O.select(key, sizes, T)
        live = np.nonzero(sizes > 0)[0]
        order = live[np.lexsort((live, -key[live]))]  # key desc, id asc
        cum = np.cumsum(sizes[order])
        k = int(np.searchsorted(cum, T, side="right"))  # longest prefix with sum <= T
        want = np.zeros(C, np.int32)
        want[order[:k]] = 1
        np.testing.assert_array_equal(sel, want)
        assert taken == (cum[k - 1] if k else 0) <= T


def test_selection_stops_at_first_overflow():
    key = np.array([3.0, 2.0, 1.0])
    sizes = np.array([2, 5, 1], np.int32)
    sel, taken = O.select(key, sizes, 4)
    assert sel.tolist() == [1, 0, 0] and taken == 2  # cluster 2 would fit but comes after the overflow


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _state_from(kbar, vbar, sizes, assign, n_tokens, d):
    C = len(sizes)
    st = O.empty_state(d, n_tokens, C, O.EXACT)
    st.kbar[:] = kbar
    st.vbar[:] = vbar
    st.sizes[:] = sizes
    st.assign[:n_tokens] = assign
    st.n_clusters = C
    st.n_clustered = n_tokens
    return st


def _sdpa(q, K, V):
    qt = torch.from_numpy(q)[None, :, None, :]   # [1][G][1][d]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], *K.shape)
    vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], *V.shape)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


@pytest.mark.parametrize("d", [2, 128])
def test_hand_derived_decode(golden_dir, d):
    g = json.load(open(os.path.join(golden_dir, "tiny_decode.json")))

    def pad(rows):
        a = np.zeros((len(rows), d))
        a[:, :2] = rows
        return a

    K, V = pad(g["keys"]), pad(g["values"])
    q = np.zeros((1, d))
    q[0, :2] = math.sqrt(d) * np.array([math.log(2), math.log(3)])
    st = _state_from(pad(g["key_centroids"]), pad(g["value_centroids"]), g["sizes"], g["assign"], 4, d)
    for case in g["cases"]:
        res = O.decode_unit(q, K, V, 4, st, case["budget"])
        assert res.selected.tolist() == case["selected"]
        np.testing.assert_allclose(res.out[0, :2], case["out"], rtol=1e-14, atol=1e-15)
        assert np.all(res.out[0, 2:] == 0)


def test_full_budget_is_dense_attention():
    r = _rng(7)
    N, d, G = 700, 32, 4
    K = O.round_storage(r.standard_normal((N, d)), O.BF16)
    V = O.round_storage(r.standard_normal((N, d)), O.BF16)
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=256, iters=4, storage=O.BF16, seed=1)
    q = r.standard_normal((G, d))
    res = O.decode_unit(q, K, V, N, st, budget=N)
    assert res.selected.sum() == (st.sizes[:st.n_clusters] > 0).sum()
    np.testing.assert_allclose(res.out, _sdpa(q, K, V), rtol=1e-12, atol=1e-13)


def test_singleton_clusters_are_dense_for_every_budget():
    r = _rng(8)
    N, d, G = 120, 16, 2
    K = O.round_storage(r.standard_normal((N, d)), O.BF16)
    V = O.round_storage(r.standard_normal((N, d)), O.BF16)
    st = O.build_unit(K, V, N, tokens_per_centroid=1, cluster_block_size=64, iters=3, storage=O.BF16, seed=3)
    assert (st.sizes[:st.n_clusters] == 1).all()
    # centroid equals its key, value centroid equals its value
    tok = st.token_ids[st.offsets[:st.n_clusters]]
    np.testing.assert_array_equal(st.kbar[:st.n_clusters], K[tok])
    np.testing.assert_array_equal(st.vbar[:st.n_clusters], V[tok])
    q = r.standard_normal((G, d))
    want = O.dense(q, K, V)
    for T in [0, 1, 7, 60, 119, 120, 500]:
        res = O.decode_unit(q, K, V, N, st, budget=T)
        np.testing.assert_allclose(res.out, want, rtol=1e-12, atol=1e-13)


def test_zero_variance_clusters_are_dense_for_every_budget():
    r = _rng(9)
    d, G = 24, 3
    sizes = np.array([1, 4, 2, 7, 3, 5], np.int32)
    centers = r.standard_normal((len(sizes), d))
    assign = np.repeat(np.arange(len(sizes)), sizes).astype(np.int32)
    perm = r.permutation(len(assign))
    assign = assign[perm]
    K = centers[assign]
    V = r.standard_normal((len(assign), d))
    vbar = np.stack([V[assign == c].mean(0) for c in range(len(sizes))])
    st = _state_from(centers, vbar, sizes, assign, len(assign), d)
    q = r.standard_normal((G, d)) * 2
    want = O.dense(q, K, V)
    for T in range(0, 24):
        np.testing.assert_allclose(O.decode_unit(q, K, V, len(assign), st, T).out, want, rtol=1e-12, atol=1e-13)


def test_zero_query_returns_value_mean():
    # q = 0: every logit is 0, so each cluster weighs n_c and n_c * vbar_c is its value sum
    r = _rng(10)
    N, d = 333, 16
    K, V = r.standard_normal((N, d)), r.standard_normal((N, d))
    st = O.build_unit(K, V, N, tokens_per_centroid=8, cluster_block_size=100, iters=3, storage=O.EXACT, seed=5)
    for T in [0, 10, 100, 333]:
        res = O.decode_unit(np.zeros((2, d)), K, V, N, st, T)
        np.testing.assert_allclose(res.out, np.tile(V.mean(0), (2, 1)), rtol=1e-12, atol=1e-13)


def test_zero_budget_closed_form():
    r = _rng(11)
    N, d = 300, 16
    K, V = r.standard_normal((N, d)), r.standard_normal((N, d))
    st = O.build_unit(K, V, N, tokens_per_centroid=10, cluster_block_size=300, iters=3, storage=O.EXACT, seed=2)
    q = r.standard_normal((1, d))
    C = st.n_clusters
    live = st.sizes[:C] > 0
    w = st.sizes[:C][live] * np.exp(st.kbar[:C][live] @ q[0] / math.sqrt(d))
    want = (w[:, None] * st.vbar[:C][live]).sum(0) / w.sum()
    np.testing.assert_allclose(O.decode_unit(q, K, V, N, st, 0).out[0], want, rtol=1e-12)


def test_output_is_convex_combination():
    r = _rng(12)
    N, d, G = 500, 16, 4
    K = r.standard_normal((N, d))
    V = r.standard_normal((N, d))
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=256, iters=3, storage=O.BF16, seed=4)
    q = r.standard_normal((G, d)) * 3
    for T in [0, 50, 200]:
        res = O.decode_unit(q, K, V, N, st, T)
        sel = res.selected.astype(bool)
        used = [V[sel[st.assign[:N]]], st.vbar[:st.n_clusters][~sel & (st.sizes[:st.n_clusters] > 0)]]
        used = np.concatenate(used)
        assert np.all(res.out <= used.max(0) + 1e-12) and np.all(res.out >= used.min(0) - 1e-12)


def test_group_of_identical_queries_matches_single_head():
    r = _rng(13)
    N, d = 400, 16
    K, V = r.standard_normal((N, d)), r.standard_normal((N, d))
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=200, iters=3, storage=O.BF16, seed=6)
    q1 = r.standard_normal((1, d)) * 2
    one = O.decode_unit(q1, K, V, N, st, 64)
    four = O.decode_unit(np.repeat(q1, 4, 0), K, V, N, st, 64)
    np.testing.assert_array_equal(four.selected, one.selected)
    for g in range(4):
        np.testing.assert_allclose(four.out[g], one.out[0], rtol=1e-13)


def test_tail_tokens_are_attended_exactly():
    r = _rng(14)
    N, n_cl, d = 500, 384, 16
    K, V = r.standard_normal((N, d)), r.standard_normal((N, d))
    st = O.build_unit(K, V, n_cl, tokens_per_centroid=16, cluster_block_size=128, iters=3, storage=O.EXACT,
                      seed=7, capacity_tokens=N)
    q = r.standard_normal((2, d))
    np.testing.assert_allclose(O.decode_unit(q, K, V, N, st, n_cl).out, O.dense(q, K, V), rtol=1e-12)


def test_omit_mode_reduces_to_dense_and_to_selected_only():
    r = _rng(15)
    N, d = 256, 16
    K, V = r.standard_normal((N, d)), r.standard_normal((N, d))
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=256, iters=3, storage=O.EXACT, seed=8)
    q = r.standard_normal((1, d))
    np.testing.assert_allclose(O.decode_unit(q, K, V, N, st, N, mode=1).out, O.dense(q, K, V), rtol=1e-12)
    res = O.decode_unit(q, K, V, N, st, 64, mode=1)
    keep = res.selected.astype(bool)[st.assign[:N]]
    np.testing.assert_allclose(res.out, O.dense(q, K[keep], V[keep]), rtol=1e-12)


# ---------------------------------------------------------------------------
# build, online update, hierarchy
# ---------------------------------------------------------------------------

def test_build_state_invariants():
    r = _rng(16)
    N, d = 1000, 8
    K = O.round_storage(r.standard_normal((N, d)), O.BF16)
    V = O.round_storage(r.standard_normal((N, d)), O.BF16)
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=384, iters=4, storage=O.BF16, seed=9)
    assert [b.L for b in st.blocks] == [384, 384, 232]
    assert st.n_clusters == 24 + 24 + 15
    C = st.n_clusters
    assert st.sizes[:C].sum() == N and st.offsets[0] == 0 and st.offsets[C] == N
    for c in range(C):
        ids = st.token_ids[st.offsets[c]:st.offsets[c + 1]]
        assert len(ids) == st.sizes[c] and np.all(np.diff(ids) > 0)
        assert np.all(st.assign[ids] == c)
        if len(ids):
            np.testing.assert_array_equal(st.mu[c], K[ids].mean(0))
            np.testing.assert_array_equal(st.kbar[c], O.round_storage(K[ids].mean(0), O.BF16))
            np.testing.assert_array_equal(st.vbar[c], O.round_storage(V[ids].mean(0), O.BF16))
    for b in st.blocks:  # tokens only join clusters of their own block
        a = st.assign[b.p:b.p + b.L]
        assert a.min() >= b.c0 and a.max() < b.c0 + b.C


def test_build_then_update_equals_one_build():
    r = _rng(17)
    N, d, B = 1024, 8, 256
    K = O.round_storage(r.standard_normal((N, d)), O.BF16)
    V = O.round_storage(r.standard_normal((N, d)), O.BF16)
    whole = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=B, iters=5, seed=11, unit=3)
    part = O.build_unit(K, V, 2 * B, tokens_per_centroid=16, cluster_block_size=B, iters=5, seed=11, unit=3,
                        capacity_tokens=N, capacity_clusters=whole.capacity_clusters)
    assert O.update_unit(part, K, V, 2 * B + B - 1, cluster_block_size=B, iters=5, seed=11, unit=3) == 0
    assert O.update_unit(part, K, V, N, cluster_block_size=B, iters=5, seed=11, unit=3) == 2
    for name in ("mu", "kbar", "vbar", "sizes", "offsets", "token_ids", "assign"):
        np.testing.assert_array_equal(getattr(part, name), getattr(whole, name))


def test_hierarchy_structure_and_reductions():
    r = _rng(18)
    N, d, G = 2048, 16, 2
    K = O.round_storage(r.standard_normal((N, d)) * 2, O.BF16)
    V = O.round_storage(r.standard_normal((N, d)), O.BF16)
    st = O.build_unit(K, V, N, tokens_per_centroid=16, cluster_block_size=1024, iters=4, seed=12)
    O.build_coarse(st, coarse_tokens_per_centroid=128, iters=6, seed=12)
    assert st.n_coarse == 16
    C, D = st.n_clusters, st.n_coarse
    live = st.sizes[:C] > 0
    assert np.all(st.parent[:C][live] >= 0) and np.all(st.parent[:C][~live] == -1)
    for b_i, b in enumerate(st.blocks):  # nesting stays inside a block
        par = st.parent[b.c0:b.c0 + b.C]
        par = par[par >= 0]
        assert par.min() >= 8 * b_i and par.max() < 8 * (b_i + 1)
    for g in range(D):
        mem = st.cmembers[st.coffsets[g]:st.coffsets[g + 1]]
        assert st.csizes[g] == st.sizes[mem].sum()
        assert np.all(st.parent[mem] == g)
        if len(mem):
            w = st.sizes[mem].astype(np.float64)
            np.testing.assert_allclose(st.cvbar[g], O.round_storage((w[:, None] * st.vbar[mem]).sum(0) / w.sum(),
                                                                    O.BF16))
    for J in st.cJ:  # weighted k-means objective, rounding aside, does not climb far
        assert J[-1] <= J[0]
    q = r.standard_normal((G, d))
    flat = O.decode_unit(q, K, V, N, st, 128)
    allcand = O.decode_unit_hier(q, K, V, N, st, 128, cand_budget=N)
    assert allcand.candidates.all()
    np.testing.assert_array_equal(allcand.selected, flat.selected)
    np.testing.assert_allclose(allcand.out, flat.out, rtol=1e-12)
    np.testing.assert_allclose(O.decode_unit_hier(q, K, V, N, st, N, cand_budget=N).out, O.dense(q, K, V),
                               rtol=1e-12)
    # no candidate at all: every coarse cluster is approximated
    none = O.decode_unit_hier(q, K, V, N, st, 128, cand_budget=0)
    w = st.csizes[:D] * np.exp(st.ckbar[:D] @ q.T / math.sqrt(d)).T
    np.testing.assert_allclose(none.out, (w @ st.cvbar[:D]) / w.sum(1, keepdims=True), rtol=1e-12)


def test_hierarchy_exact_weighted_objective_monotone():
    r = _rng(19)
    x = r.standard_normal((200, 6))
    w = r.integers(1, 20, 200).astype(np.float64)
    init = O.init_indices(O.block_stream(0, 0, 0, 1), 200, 10)
    _, _, _, _, J = O.kmeans(x, 10, 12, O.EXACT, init, w=w)
    assert np.all(np.diff(J) <= 1e-12 * J[:-1])
    mu, _, a, counts, _ = O.kmeans(x, 10, 1, O.EXACT, init, w=w)
    for c in range(10):
        if counts[c]:
            np.testing.assert_allclose(mu[c], (w[a == c, None] * x[a == c]).sum(0) / w[a == c].sum(), rtol=1e-13)


# ---------------------------------------------------------------------------
# fp8 (E4M3) centroid codes with a power-of-two scale per 32 values
# ---------------------------------------------------------------------------
def test_e4m3_table_from_the_format_definition():
    from oracle import centroid_codes as F
    v = F.VALUES
    assert len(v) == 127 and v[0] == 0.0
    assert v[1] == 2.0 ** -9 and v[7] == 7 * 2.0 ** -9          # subnormals 0.m x 2^-6
    assert v[8] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    assert np.all(np.diff(v) > 0)                                # codes ordered by magnitude
    # spacing doubles once per binade of 8 codes above the subnormals
    for e in range(1, 15):
        assert np.allclose(np.diff(v[8 * e:8 * e + 8]), 2.0 ** (e - 10))


def test_e4m3_hand_derived_blocks(golden_dir):
    from oracle import centroid_codes as F
    g = json.load(open(os.path.join(golden_dir, "fp8_blocks.json")))
    for case in g["cases"]:
        codes, E = F.encode_block(case["x"])
        assert E == case["E"], case["derivation"]
        assert [int(c) for c in codes] == [int(c, 16) for c in case["codes"]], case["derivation"]


def test_e4m3_every_value_round_trips_and_ties_go_even():
    from oracle import centroid_codes as F
    v = F.VALUES
    # all 127 finite magnitudes, both signs, in blocks whose largest value is
    # 448 (scale 2^0): each encodes to its own code
    xs = np.concatenate([v, -v[1:]])
    for s in range(0, len(xs), 31):
        blk = np.zeros(32)
        blk[:len(xs[s:s + 31])] = xs[s:s + 31]
        blk[31] = 448.0
        codes, E = F.encode_block(blk)
        assert E == 0
        assert np.array_equal(F.decode_rows(codes[None].astype(np.uint8), np.array([[127]]))[0], blk)
    # midpoints go to the even code, anything above a midpoint goes up
    for c in range(126):
        mid = (v[c] + v[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert F.encode_magnitude(mid) == even
        assert F.encode_magnitude(np.nextafter(mid, np.inf)) == c + 1
        assert F.encode_magnitude(np.nextafter(mid, -np.inf)) == c


def test_e4m3_scale_rule_and_error_bound():
    from oracle import centroid_codes as F
    assert F.scale_exponent(448.0) == 0 and F.scale_exponent(448.0001) == 1
    assert F.scale_exponent(1.0) == -8 and F.scale_exponent(1.75) == -8 and F.scale_exponent(1.76) == -7
    assert F.scale_exponent(0.0) == -126 and F.scale_exponent(2.0 ** -140) == -126
    rng = np.random.default_rng(3)
    X = rng.standard_normal((40, 128)) * np.exp2(rng.integers(-20, 20, (40, 1)))
    X[3, 5:9] = 0.0
    X[4, 32:64] *= 1e-45                              # below the floor of the scale
    codes, scales = F.encode_rows(X)
    Y = F.decode_rows(codes, scales)
    E = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    a = np.abs(X) * np.exp2(-E)                       # magnitudes in code units
    assert np.all(a <= 448.0)
    # E is the least such exponent unless the floor -126 holds it
    above = scales > 1
    assert np.all((np.abs(X).reshape(40, 4, 32).max(-1) * np.exp2(-(scales.astype(np.int64) - 128)))[above] > 448.0)
    assert not np.all(above)
    err = np.abs(Y - X) * np.exp2(-E)
    normal = a >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * a[normal])  # half an ulp of 3 mantissa bits
    assert np.all(err[~normal] <= 2.0 ** -10)            # half the subnormal step
    assert np.array_equal(np.signbit(Y[X != 0]), np.signbit(X[X != 0]))
