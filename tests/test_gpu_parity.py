"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Teacher forcing: every step the oracle checks starts from the GPU's own
previous state (assignment from the GPU's stored centroids, update from the
GPU's assignment, decode from the GPU's cluster state), so each kernel is
compared on identical inputs.  Integer decisions must match exactly outside
the fp32 rounding windows of tests/gpu_util.py; floating-point results within
the stated tolerances.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from gpu_util import (assign_tie_violations, check_coarse_round, close, gamma, load_oracle_states,
                      oracle_state_from_gpu, rank_tolerance, selection_is_valid, storage_of, U32)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def M():
    from sparse_long_context_means_amd import mpattn

    return mpattn


def small_workload(B, Hq, Hkv, n, components, dtype=torch.bfloat16, outliers=0, index=90):
    base = workloads.WORKLOADS["qwen3-8b-layer-b1-32k"]
    return dataclasses.replace(base, name="test", index=index, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_tokens=n,
                               components=components, dtype=dtype, outlier_channels=outliers)


def queries(w, means, step):
    return workloads.make_queries(w, means, step)


# ---------------------------------------------------------------------------
# decode from an oracle-built state (teacher-forced state)
# ---------------------------------------------------------------------------
DECODE_CASES = [
    # dtype, B, Hq, Hkv, n_clustered, n_total, block, tpc, budgets, sorted copy, splits
    ("bf16", 2, 8, 2, 5000, 5000, 2048, 16, [0, 1, 100, 517, 5000], True, 0),
    ("bf16", 1, 8, 2, 3000, 3333, 1024, 16, [64, 3000], False, 3),
    ("fp32", 1, 1, 1, 4096, 4096, 8192, 16, [128], True, 0),
    ("bf16", 1, 8, 1, 2000, 2000, 512, 8, [200], True, 0),
    ("bf16", 1, 2, 1, 777, 777, 256, 4, [50, 0], False, 0),
    # many units: the whole step of a unit in one workgroup
    ("bf16", 16, 32, 8, 2048, 2048, 1024, 16, [0, 40, 300, 2048], True, 0),
    ("bf16", 8, 16, 8, 3000, 3300, 1024, 16, [100, 3000], False, 0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-G{c[2] // c[3]}-N{c[5]}")
def test_decode_matches_oracle_on_oracle_state(case):
    mp = M()
    dt_name, B, Hq, Hkv, n_cl, n_tot, Bc, r, budgets, sorted_copy, splits = case
    dt = torch.bfloat16 if dt_name == "bf16" else torch.float32
    w = small_workload(B, Hq, Hkv, n_tot, max(8, n_tot // 16), dt, outliers=4 if dt_name == "bf16" else 0)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=n_tot, dtype=dt, tokens_per_centroid=r,
                  cluster_block=Bc, build_iters=3, splits=splits, seed=5)
    storage = storage_of(dt)
    units = O.parallel_map(lambda u: O.build_unit(K[u // Hkv, u % Hkv], V[u // Hkv, u % Hkv], n_cl,
                                                  tokens_per_centroid=r, cluster_block_size=Bc, iters=3,
                                                  storage=storage, seed=5, unit=u,
                                                  capacity_clusters=p.max_clusters()),
                           range(B * Hkv))
    state = mp.ClusterState(p, DEV, sorted_copy=sorted_copy)
    load_oracle_states(state, p, units, K, V)
    Kd, Vd = K.to(DEV), V.to(DEV)
    G = Hq // Hkv
    for step, T in enumerate(budgets):
        q = queries(w, means, step)
        dbg = mp.DecodeDebug.allocate(p, state, DEV)
        out = mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, T, debug=dbg).cpu().numpy()
        sel_g = dbg.selected.cpu().numpy()
        s_g = dbg.scores.cpu().numpy()
        exact_g = dbg.exact_tokens.cpu().numpy()
        for u, st in enumerate(units):
            b, h = divmod(u, Hkv)
            qu = q[b, h * G:(h + 1) * G]
            ref = O.decode_unit(qu, K[b, h], V[b, h], n_tot, st, T)
            C = st.n_clusters
            # scores within the fp32 bound of a 128-term dot product
            s64 = ref.s.T  # [C][G]
            q64 = O.f64(qu)
            bound = gamma(136) * (np.abs(q64)[:, None, :] * np.abs(st.kbar[:C])[None]).sum(-1).T / math.sqrt(128)
            assert np.all(np.abs(s_g[b, h] - s64) <= bound + 4 * U32 * np.abs(s64) + 1e-30), "scores"
            live = st.sizes[:C] > 0
            assert np.array_equal(sel_g[b, h][~live], np.zeros((~live).sum(), np.int32))
            if np.array_equal(sel_g[b, h], ref.selected):
                ok, ea, er = close(out[b, h * G:(h + 1) * G], ref.out)
                assert ok, f"unit {u} T={T}: max abs {ea:.3g} max rel {er:.3g}"
            else:
                tol = rank_tolerance(q64, st.kbar[:C])
                assert selection_is_valid(ref.r, tol, st.sizes[:C], T, sel_g[b, h]), f"unit {u}: invalid selection"
                want = O.decode_with_selection(qu, K[b, h], V[b, h], n_tot, st, sel_g[b, h])
                ok, ea, er = close(out[b, h * G:(h + 1) * G], want)
                assert ok, f"unit {u} T={T} (tie-broken selection): max abs {ea:.3g}"
            assert exact_g[b, h] == st.sizes[:C][sel_g[b, h].astype(bool)].sum()


def test_hand_derived_example_on_gpu(golden_dir):
    """The hand-worked decode of tests/golden/tiny_decode.json, padded to d = 128."""
    import json
    import os

    mp = M()
    g = json.load(open(os.path.join(golden_dir, "tiny_decode.json")))
    d = 128

    def pad(rows):
        a = np.zeros((len(rows), d))
        a[:, :2] = rows
        return a

    K = torch.from_numpy(pad(g["keys"])).float()[None, None]
    V = torch.from_numpy(pad(g["values"])).float()[None, None]
    q = torch.zeros(1, 1, d)
    q[0, 0, :2] = torch.tensor([math.log(2), math.log(3)], dtype=torch.float64) * math.sqrt(d)
    p = mp.Params(batch=1, n_q_heads=1, n_kv_heads=1, capacity_tokens=4, dtype=torch.float32, tokens_per_centroid=2,
                  cluster_block=4)
    st = O.empty_state(d, 4, p.max_clusters(), O.F32)
    st.kbar[:2] = pad(g["key_centroids"])
    st.mu[:2] = pad(g["key_centroids"])
    st.vbar[:2] = pad(g["value_centroids"])
    st.sizes[:2] = g["sizes"]
    st.offsets[:3] = [0, 2, 4]
    st.token_ids[:4] = [0, 1, 2, 3]
    st.assign[:4] = g["assign"]
    st.n_clusters, st.n_clustered = 2, 4
    st.blocks.append(O.Block(0, 4, 0, 2, 0))
    state = mp.ClusterState(p, DEV, sorted_copy=True)
    load_oracle_states(state, p, [st], K, V)
    for case in g["cases"]:
        dbg = mp.DecodeDebug.allocate(p, state, DEV)
        out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 4, state, case["budget"], debug=dbg).cpu().numpy()
        assert dbg.selected.cpu().numpy()[0, 0].tolist() == case["selected"]
        np.testing.assert_allclose(out[0, 0, :2], case["out"], rtol=1e-5, atol=1e-6)
        assert np.all(out[0, 0, 2:] == 0)


# ---------------------------------------------------------------------------
# clustering, teacher-forced round by round
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block,tpc", [(16384, 16), (16384, 8), (12000, 12)])
def test_membership_lists_follow_the_assignment(block, tpc):
    """Member lists, sizes and offsets against their definition on the GPU's
    own assignment: each block's tokens in (cluster, token) order.  The
    shapes take both list kernels: a counting sort up to 1024 clusters per
    block (16384 / 16, and 12000 / 12 = 1000), the bitonic sort beyond
    (16384 / 8 = 2048); the cache ends in a ragged block."""
    mp = M()
    B, Hq, Hkv, N = 1, 4, 2, 20000
    w = small_workload(B, Hq, Hkv, N, N // 16, outliers=4, index=77)
    K, V, _ = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, tokens_per_centroid=tpc,
                  cluster_block=block, build_iters=2, seed=5)
    st = mp.ClusterState(p, DEV, sorted_copy=False)
    mp.build_clusters(p, K.to(DEV), V.to(DEV), N, st)
    torch.cuda.synchronize()
    cfull = -(-block // tpc)
    for h in range(Hkv):
        a = st.assign[0, h, :N].cpu().numpy()
        tids = st.token_ids[0, h, :N].cpu().numpy()
        sizes = st.sizes[0, h].cpu().numpy()
        offs = st.offsets[0, h].cpu().numpy()
        for j, p0 in enumerate(range(0, N, block)):
            L = min(block, N - p0)
            c0, C = j * cfull, -(-L // tpc)
            loc = a[p0:p0 + L] - c0
            assert loc.min() >= 0 and loc.max() < C, (h, j)
            counts = np.bincount(loc, minlength=C)
            np.testing.assert_array_equal(sizes[c0:c0 + C], counts)
            np.testing.assert_array_equal(offs[c0:c0 + C], p0 + np.concatenate([[0], np.cumsum(counts)[:-1]]))
            np.testing.assert_array_equal(tids[p0:p0 + L], p0 + np.lexsort((np.arange(L), loc)))


@pytest.mark.parametrize("dt_name", ["bf16", "fp32"])
def test_build_rounds_match_oracle(dt_name):
    mp = M()
    dt = torch.bfloat16 if dt_name == "bf16" else torch.float32
    B, Hq, Hkv, N, Bc, r, seed = 1, 8, 2, 5000, 2048, 16, 3
    w = small_workload(B, Hq, Hkv, N, 300, dt, outliers=4 if dt_name == "bf16" else 0)
    K, V, _ = workloads.make_cache(w)
    storage = storage_of(dt)
    Kd, Vd = K.to(DEV), V.to(DEV)
    snaps = []
    for t in (1, 2, 3):
        p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, dtype=dt, tokens_per_centroid=r,
                      cluster_block=Bc, build_iters=t, seed=seed)
        state = mp.ClusterState(p, DEV, sorted_copy=True)
        mp.build_clusters(p, Kd, Vd, N, state)
        torch.cuda.synchronize()
        snaps.append([oracle_state_from_gpu(state, u // Hkv, u % Hkv, p) for u in range(B * Hkv)] +
                     [state.sorted_keys.cpu(), state.sorted_values.cpu()])
    n_diff_total = 0
    for u in range(B * Hkv):
        Ku, Vu = O.f64(K[0, u]), O.f64(V[0, u])
        for t in range(3):
            cur = snaps[t][u]
            for blk in cur.blocks:
                x = Ku[blk.p:blk.p + blk.L]
                if t == 0:
                    init = O.init_indices(O.block_stream(seed, u, blk.index), blk.L, blk.C)
                    mu_prev, mus_prev = x[init].copy(), O.round_storage(x[init], storage)
                else:
                    prev = snaps[t - 1][u]
                    mu_prev = prev.mu[blk.c0:blk.c0 + blk.C].copy()
                    mus_prev = prev.kbar[blk.c0:blk.c0 + blk.C].copy()
                a_ref, _, _ = O.assign_step(x, mus_prev)
                a_gpu = cur.assign[blk.p:blk.p + blk.L] - blk.c0
                nd, bad = assign_tie_violations(x, mus_prev, a_gpu, a_ref)
                n_diff_total += nd
                assert not bad, f"unit {u} round {t + 1} block {blk.index}: {len(bad)} assignments outside ties"
                # update from the GPU's assignment
                mu, mus, counts = O.update_step(x, a_gpu, mu_prev, mus_prev, storage)
                np.testing.assert_array_equal(cur.sizes[blk.c0:blk.c0 + blk.C], counts)
                live = counts > 0
                gm = cur.mu[blk.c0:blk.c0 + blk.C]
                # fp32 mean of n terms: |err| <= gamma(n + 1) * mean|x| + u |mean|
                absmean = np.stack([np.abs(x[a_gpu == c]).mean(0) if counts[c] else np.zeros(x.shape[1])
                                    for c in range(blk.C)])
                bound = gamma(counts[:, None] + 1) * absmean + U32 * np.abs(mu)
                assert np.all(np.abs(gm - mu)[live] <= bound[live] + 1e-30), "centroid means"
                np.testing.assert_array_equal(gm[~live], mu_prev[~live])  # empty clusters keep their centroid
                np.testing.assert_array_equal(cur.kbar[blk.c0:blk.c0 + blk.C], O.round_storage(gm, storage))
                # membership lists in (cluster, token) order
                order = np.lexsort((np.arange(blk.L), a_gpu))
                np.testing.assert_array_equal(cur.token_ids[blk.p:blk.p + blk.L], blk.p + order)
                starts = blk.p + np.concatenate([[0], np.cumsum(counts)[:-1]])
                np.testing.assert_array_equal(cur.offsets[blk.c0:blk.c0 + blk.C], starts)
                if t == 2:  # value centroids of the final round and the sorted copy
                    vx = Vu[blk.p:blk.p + blk.L]
                    for c in np.nonzero(live)[0][:64]:
                        m = vx[a_gpu == c].mean(0)
                        vb = gamma(counts[c] + 1) * np.abs(vx[a_gpu == c]).mean(0) + U32 * np.abs(m)
                        gv = cur.vbar[blk.c0 + c]
                        lo = O.round_storage(m - vb, storage)
                        hi = O.round_storage(m + vb, storage)
                        assert np.all((gv >= lo) & (gv <= hi)), "value centroid"
                    sk = snaps[t][-2][0, u].double().numpy()
                    np.testing.assert_array_equal(sk[blk.p:blk.p + blk.L], Ku[blk.p + order])
    print(f"assignments differing inside tie windows: {n_diff_total}")


def test_tiny_config_free_running():
    """The tiny fp32 workload end to end: well-separated components, so the
    GPU and the oracle follow the same Lloyd trajectory."""
    mp = M()
    w = workloads.WORKLOADS["tiny-fp32"]
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=1, n_q_heads=1, n_kv_heads=1, capacity_tokens=w.n_tokens, dtype=torch.float32,
                  build_iters=w.build_iters, seed=0)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, state)
    q = workloads.make_queries(w, means, 0)
    out = mp.decode(p, q.to(DEV), Kd, Vd, w.n_tokens, state, w.budgets[0]).cpu().numpy()
    ref = O.build_unit(K[0, 0], V[0, 0], w.n_tokens, iters=w.build_iters, storage=O.F32, seed=0)
    gst = oracle_state_from_gpu(state, 0, 0, p)
    assert state.n_clusters == ref.n_clusters == 256
    mism = int((gst.assign[:w.n_tokens] != ref.assign[:w.n_tokens]).sum())
    assert mism == 0, f"{mism} tokens assigned differently"
    np.testing.assert_allclose(gst.kbar[:256], ref.kbar[:256], rtol=1e-5, atol=1e-6)
    res = O.decode_unit(q[0], K[0, 0], V[0, 0], w.n_tokens, ref, w.budgets[0])
    ok, ea, er = close(out[0], res.out)
    assert ok, (ea, er)
    assert np.all(np.diff(ref.J[0]) <= 1e-9 * ref.J[0][:-1])


# ---------------------------------------------------------------------------
# reductions, determinism, split invariance
# ---------------------------------------------------------------------------

def _built(B=2, Hq=8, Hkv=2, N=4500, Bc=2048, splits=0, dt=torch.bfloat16, sorted_copy=True, iters=4, r=16,
           fmt=0):
    mp = M()
    w = small_workload(B, Hq, Hkv, N, 200, dt, outliers=4)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, dtype=dt, cluster_block=Bc,
                  build_iters=iters, splits=splits, seed=1, tokens_per_centroid=r, centroid_format=fmt)
    state = mp.ClusterState(p, DEV, sorted_copy=sorted_copy)
    mp.build_clusters(p, K.to(DEV), V.to(DEV), N, state)
    return mp, w, K, V, means, p, state


def test_dense_decode_matches_oracle():
    """The dense split-K decode (the comparison point) against textbook
    softmax attention on every head, with a token count that leaves a
    ragged last tile, and against the sparse decode at a full budget."""
    mp, w, K, V, means, p, state = _built(B=2, Hq=8, Hkv=2, N=4500)
    G = p.group
    for n_tok in (4500, 4433, 70):
        q = queries(w, means, 40 + n_tok % 7)
        out = mp.dense_decode(p, q.to(DEV), K.to(DEV), V.to(DEV), n_tok).cpu().numpy()
        for b in range(p.batch):
            for h in range(p.n_kv_heads):
                ref = O.dense(q[b, h * G:(h + 1) * G], K[b, h, :n_tok], V[b, h, :n_tok])
                ok, ea, er = close(out[b, h * G:(h + 1) * G], ref)
                assert ok, (n_tok, b, h, ea, er)
    q = queries(w, means, 50)
    od = mp.dense_decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 4500).cpu().numpy()
    of = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 4500, state, 4500).cpu().numpy()
    np.testing.assert_allclose(od, of, rtol=1e-3, atol=2e-4)


def test_full_budget_is_dense_attention():
    mp, w, K, V, means, p, state = _built()
    q = queries(w, means, 3)
    out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), p.capacity_tokens, state, p.capacity_tokens).cpu().numpy()
    G = p.group
    for b in range(p.batch):
        for h in range(p.n_kv_heads):
            ref = O.dense(q[b, h * G:(h + 1) * G], K[b, h], V[b, h])
            ok, ea, er = close(out[b, h * G:(h + 1) * G], ref)
            assert ok, (b, h, ea, er)


def test_gpu_state_decode_matches_oracle():
    """Decode on the GPU-built state, checked by the oracle on that state."""
    mp, w, K, V, means, p, state = _built(sorted_copy=False)
    G = p.group
    for step, T in enumerate([0, 128, 700]):
        q = queries(w, means, step)
        dbg = mp.DecodeDebug.allocate(p, state, DEV)
        out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), p.capacity_tokens, state, T, debug=dbg).cpu().numpy()
        for u in range(p.units):
            b, h = divmod(u, p.n_kv_heads)
            st = oracle_state_from_gpu(state, b, h, p)
            sel = dbg.selected[b, h].cpu().numpy()
            ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], p.capacity_tokens, st, T)
            if not np.array_equal(sel, ref.selected):
                tol = rank_tolerance(O.f64(q[b, h * G:(h + 1) * G]), st.kbar[:st.n_clusters])
                assert selection_is_valid(ref.r, tol, st.sizes[:st.n_clusters], T, sel)
                ref_out = O.decode_with_selection(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], p.capacity_tokens,
                                                  st, sel)
            else:
                ref_out = ref.out
            ok, ea, er = close(out[b, h * G:(h + 1) * G], ref_out)
            assert ok, (u, T, ea, er)


def test_repeatable_bitwise():
    mp, w, K, V, means, p, s1 = _built()
    s2 = mp.ClusterState(p, DEV)
    mp.build_clusters(p, K.to(DEV), V.to(DEV), p.capacity_tokens, s2)
    for name in ("key_centroids", "value_centroids", "key_centroids_f32", "sizes", "offsets", "token_ids", "assign",
                 "sorted_keys", "sorted_values"):
        assert torch.equal(getattr(s1, name), getattr(s2, name)), name
    q = queries(w, means, 1).to(DEV)
    o1 = mp.decode(p, q, K.to(DEV), V.to(DEV), p.capacity_tokens, s1, 300)
    o2 = mp.decode(p, q, K.to(DEV), V.to(DEV), p.capacity_tokens, s1, 300)
    assert torch.equal(o1, o2)


def test_split_count_does_not_change_the_result():
    mp, w, K, V, means, p, state = _built()
    q = queries(w, means, 2).to(DEV)
    outs = []
    for S in (1, 3, 16, 64):
        ps = dataclasses.replace(p, splits=S)
        outs.append(mp.decode(ps, q, K.to(DEV), V.to(DEV), p.capacity_tokens, state, 400).cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-5, atol=1e-6)


def test_omit_mode_matches_oracle():
    mp, w, K, V, means, p, state = _built(B=1)
    q = queries(w, means, 4)
    G = p.group
    for T in (0, 256):
        out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), p.capacity_tokens, state, T,
                        mode=mp.MODE_OMIT).cpu().numpy()
        for h in range(p.n_kv_heads):
            st = oracle_state_from_gpu(state, 0, h, p)
            ref = O.decode_unit(q[0, h * G:(h + 1) * G], K[0, h], V[0, h], p.capacity_tokens, st, T, mode=1)
            ok, ea, er = close(out[0, h * G:(h + 1) * G], ref.out)
            assert ok, (h, T, ea)


# ---------------------------------------------------------------------------
# the per-unit path (one workgroup per unit) against the split launches
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["multipole", "omit"])
def test_unit_path_matches_split_path_and_oracle(mode):
    mp, w, K, V, means, p, state = _built(B=16, Hq=32, Hkv=8, N=3000, Bc=1024)
    md = mp.MODE_MULTIPOLE if mode == "multipole" else mp.MODE_OMIT
    ps = dataclasses.replace(p, splits=8)
    G = p.group
    for step, T in enumerate((64, 700)):
        q = queries(w, means, 10 + step)
        du, ds = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        ou = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 3000, state, T, mode=md, debug=du).cpu().numpy()
        os_ = mp.decode(ps, q.to(DEV), K.to(DEV), V.to(DEV), 3000, state, T, mode=md, debug=ds).cpu().numpy()
        # same keys, same cut, same exact-token counts on both paths
        assert torch.equal(du.scores.cpu(), ds.scores.cpu())
        assert torch.equal(du.selected.cpu(), ds.selected.cpu())
        assert torch.equal(du.exact_tokens.cpu(), ds.exact_tokens.cpu())
        np.testing.assert_allclose(ou, os_, rtol=1e-4, atol=1e-5)
        for u in (0, 37, 127):
            b, h = divmod(u, p.n_kv_heads)
            st = oracle_state_from_gpu(state, b, h, p)
            ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], 3000, st, T,
                                mode=0 if mode == "multipole" else 1)
            ok, ea, er = close(ou[b, h * G:(h + 1) * G], ref.out)
            assert ok, (u, T, ea, er)


def test_unit_path_exact_rows_in_several_batches():
    """More exact rows per workgroup than one staged batch holds (the first
    batch starts early on the cut waves, later batches are staged by all
    waves): a budget of every clustered token with an unclustered tail is
    dense attention over all tokens, and a partial budget matches the split
    launches and the oracle."""
    mp = M()
    B, Hq, Hkv, n_cl, n_tot = 8, 16, 2, 10000, 12000
    w = small_workload(B, Hq, Hkv, n_tot, 600, outliers=4, index=96)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=n_tot, cluster_block=2048, build_iters=3,
                  seed=9)
    assert p.decode_stages() == ["unit"]
    ps = dataclasses.replace(p, splits=4)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, n_cl, state)
    G = p.group
    q = queries(w, means, 41)
    out = mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, n_cl).cpu().numpy()
    for u in (0, 7, p.units - 1):
        b, h = divmod(u, Hkv)
        ok, ea, er = close(out[b, h * G:(h + 1) * G], O.dense(q[b, h * G:(h + 1) * G], K[b, h, :n_tot], V[b, h, :n_tot]))
        assert ok, (u, ea, er)
    T = 4000
    d1, d4 = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
    o1 = mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, T, debug=d1).cpu().numpy()
    o4 = mp.decode(ps, q.to(DEV), Kd, Vd, n_tot, state, T, debug=d4).cpu().numpy()
    assert torch.equal(d1.selected.cpu(), d4.selected.cpu())
    np.testing.assert_allclose(o1, o4, rtol=1e-4, atol=1e-5)
    sel = d1.selected.cpu().numpy()
    for u in (1, 10):
        b, h = divmod(u, Hkv)
        st = oracle_state_from_gpu(state, b, h, p)
        ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], n_tot, st, T)
        want = ref.out if np.array_equal(sel[b, h], ref.selected) else O.decode_with_selection(
            q[b, h * G:(h + 1) * G], K[b, h], V[b, h], n_tot, st, sel[b, h])
        ok, ea, er = close(o1[b, h * G:(h + 1) * G], want)
        assert ok, (u, ea, er)


def test_unit_path_over_2048_clusters_matches_split_path_and_oracle():
    """The one-launch decode at more than 2048 clusters per unit (the
    4096-cluster shape, four workgroups per unit at 64 units): same keys, cut
    and exact-token counts as the split launches, outputs within tolerance of
    them and of the oracle on sampled units."""
    mp, w, K, V, means, p, state = _built(B=8, Hq=32, Hkv=8, N=10000, Bc=8192, r=4, iters=2)
    assert p.decode_stages() == ["unit"] and state.n_clusters > 2048
    ps = dataclasses.replace(p, splits=8)
    G = p.group
    for step, T in enumerate((500, 3000)):
        q = queries(w, means, 30 + step)
        du, ds = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        ou = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 10000, state, T, debug=du).cpu().numpy()
        os_ = mp.decode(ps, q.to(DEV), K.to(DEV), V.to(DEV), 10000, state, T, debug=ds).cpu().numpy()
        assert torch.equal(du.scores.cpu(), ds.scores.cpu())
        assert torch.equal(du.selected.cpu(), ds.selected.cpu())
        assert torch.equal(du.exact_tokens.cpu(), ds.exact_tokens.cpu())
        np.testing.assert_allclose(ou, os_, rtol=1e-4, atol=1e-5)
        for u in (0, 63):
            b, h = divmod(u, p.n_kv_heads)
            st = oracle_state_from_gpu(state, b, h, p)
            ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], 10000, st, T, mode=0)
            ok, ea, er = close(ou[b, h * G:(h + 1) * G], ref.out)
            assert ok, (u, T, ea, er)


@pytest.mark.parametrize("recipe", ["zero_queries", "outlier_cluster", "plain"])
def test_unit_path_cut_paths_match_split_path(recipe):
    """The one-launch cut settles most units with one pass over value bins
    and a ranking of the cut bin's clusters; a degenerate key range (zero
    queries: every key 0, ties broken by id) and a crowded cut bin (one
    cluster of huge keys stretches the range, so the bulk shares a bin) take
    the exact radix passes instead.  All three must pick exactly the clusters
    of the split launches' radix cut; at zero queries the result is also the
    oracle's (every key is exactly 0 on both sides)."""
    mp = M()
    B, Hq, Hkv, N, Bc = 16, 32, 8, 6000, 2048
    w = small_workload(B, Hq, Hkv, N, 200, torch.bfloat16, outliers=4)
    K, V, means = workloads.make_cache(w)
    q = queries(w, means, 50)
    if recipe == "outlier_cluster":
        v = torch.randn(128, generator=torch.Generator().manual_seed(5))
        v = v / v.norm()
        K[:, :, :64] = (20000.0 * v).to(K.dtype)  # 64 tokens far along v: keys in the thousands
        q = (q.float() + 3.0 * v).to(q.dtype)
    elif recipe == "zero_queries":
        q = torch.zeros_like(q)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=Bc, build_iters=3,
                  seed=1)
    assert p.decode_stages() == ["unit"]
    ps = dataclasses.replace(p, splits=8)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, N, state)
    G = p.group
    for T in (0, 100, 700, 5990):
        du, ds = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        ou = mp.decode(p, q.to(DEV), Kd, Vd, N, state, T, debug=du).cpu().numpy()
        os_ = mp.decode(ps, q.to(DEV), Kd, Vd, N, state, T, debug=ds).cpu().numpy()
        assert torch.equal(du.scores.cpu(), ds.scores.cpu()), (recipe, T)
        assert torch.equal(du.selected.cpu(), ds.selected.cpu()), (recipe, T)
        assert torch.equal(du.exact_tokens.cpu(), ds.exact_tokens.cpu()), (recipe, T)
        np.testing.assert_allclose(ou, os_, rtol=1e-4, atol=1e-5)
        if recipe == "zero_queries":
            for u in (0, 77):
                b, h = divmod(u, Hkv)
                st = oracle_state_from_gpu(state, b, h, p)
                ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], N, st, T)
                assert np.array_equal(du.selected.cpu().numpy()[b, h, :st.n_clusters], ref.selected), (u, T)
                ok, ea, er = close(ou[b, h * G:(h + 1) * G], ref.out)
                assert ok, (u, T, ea, er)


def test_unit_path_rescore_gives_the_same_result():
    """The one-launch decode splits a unit over several workgroups that take
    each other's cluster keys; the paths that score the other shares locally
    (all waves: rescore 1; one wave, as when a partner is late: rescore 2)
    must give bit-identical keys, cut and output.  Forced through the debug
    flag, at 128 units (two workgroups per unit) and 64 units (four)."""
    for B, Hkv in ((16, 8), (8, 8)):
        mp, w, K, V, means, p, state = _built(B=B, Hq=4 * Hkv, Hkv=Hkv, N=3000, Bc=1024)
        assert p.decode_stages() == ["unit"]
        ws = mp.Workspace().get(p, state, DEV)
        for step, T in enumerate((64, 700)):
            q = queries(w, means, 20 + step).to(DEV)
            outs, dbgs = [], []
            for rescore in (0, 1, 2, 0):
                d = mp.DecodeDebug.allocate(p, state, DEV)
                d.rescore = rescore
                before = mp.decode_status(ws)
                outs.append(mp.decode(p, q, K.to(DEV), V.to(DEV), 3000, state, T, debug=d, workspace=ws).cpu())
                after = mp.decode_status(ws)
                # the workspace counters: every workgroup of the forced
                # late-partner path counts one fallback; nothing is poisoned
                assert after[1] == 0
                if rescore == 2:
                    assert after[0] - before[0] >= 2 * p.units
                dbgs.append(d)
            for o, d in zip(outs[1:], dbgs[1:]):
                assert torch.equal(o, outs[0]), (B, T)
                assert torch.equal(d.scores.cpu(), dbgs[0].scores.cpu())
                assert torch.equal(d.selected.cpu(), dbgs[0].selected.cpu())
                assert torch.equal(d.exact_tokens.cpu(), dbgs[0].exact_tokens.cpu())


# ---------------------------------------------------------------------------
# per-query-head selection (the alternative reading of who selects under
# grouped-query attention): each query head is the oracle's decode of a
# one-head group over its KV head's clusters
# ---------------------------------------------------------------------------
def test_per_head_selection_matches_oracle_on_oracle_state():
    mp = M()
    B, Hq, Hkv, n_tot, Bc, r = 8, 32, 8, 3000, 1024, 16
    w = small_workload(B, Hq, Hkv, n_tot, max(8, n_tot // 16), outliers=4, index=91)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=n_tot, tokens_per_centroid=r,
                  cluster_block=Bc, build_iters=3, seed=5)
    assert p.decode_stages() == ["unit"]
    units = O.parallel_map(lambda u: O.build_unit(K[u // Hkv, u % Hkv], V[u // Hkv, u % Hkv], n_tot,
                                                  tokens_per_centroid=r, cluster_block_size=Bc, iters=3,
                                                  storage=storage_of(torch.bfloat16), seed=5, unit=u,
                                                  capacity_clusters=p.max_clusters()),
                           range(B * Hkv))
    state = mp.ClusterState(p, DEV)
    load_oracle_states(state, p, units, K, V)
    Kd, Vd = K.to(DEV), V.to(DEV)
    G = Hq // Hkv
    n_tie = 0
    for step, T in enumerate((0, 40, 300, 3000)):
        q = queries(w, means, 40 + step)
        dbg = mp.DecodeDebug.allocate(p, state, DEV, per_head=True)
        out = mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, T, mode=mp.MODE_PER_HEAD, debug=dbg).cpu().numpy()
        sel_g = dbg.selected.cpu().numpy()       # [B][Hq][C]
        s_g = dbg.scores.cpu().numpy()[..., 0]    # [B][Hq][C]
        exact_g = dbg.exact_tokens.cpu().numpy()  # [B][Hq]
        for b in range(B):
            for hq in range(Hq):
                st = units[b * Hkv + hq // G]
                C = st.n_clusters
                qu = q[b, hq:hq + 1]
                ref = O.decode_unit(qu, K[b, hq // G], V[b, hq // G], n_tot, st, T)
                q64 = O.f64(qu)
                bound = gamma(136) * (np.abs(q64) @ np.abs(st.kbar[:C]).T)[0] / math.sqrt(128)
                assert np.all(np.abs(s_g[b, hq, :C] - ref.s[0]) <= bound + 4 * U32 * np.abs(ref.s[0]) + 1e-30)
                if np.array_equal(sel_g[b, hq, :C], ref.selected):
                    want = ref.out
                else:
                    n_tie += 1
                    tol = rank_tolerance(q64, st.kbar[:C])
                    assert selection_is_valid(ref.r, tol, st.sizes[:C], T, sel_g[b, hq, :C]), (b, hq, T)
                    want = O.decode_with_selection(qu, K[b, hq // G], V[b, hq // G], n_tot, st, sel_g[b, hq, :C])
                ok, ea, er = close(out[b, hq:hq + 1], want)
                assert ok, f"head ({b}, {hq}) T={T}: max abs {ea:.3g} max rel {er:.3g}"
                assert exact_g[b, hq] == st.sizes[:C][sel_g[b, hq, :C].astype(bool)].sum()
        # the heads of a group do not all take the shared cut
        if T in (40, 300):
            shared = mp.DecodeDebug.allocate(p, state, DEV)
            mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, T, debug=shared)
            per = sel_g.reshape(B, Hkv, G, -1)
            assert np.any(per != shared.selected.cpu().numpy()[:, :, None, :])
    assert n_tie <= 4


def test_per_head_selection_with_one_head_per_group_is_the_shared_decode():
    """With G = 1 the two readings coincide: same launch shape, same bits."""
    mp, w, K, V, means, p, state = _built(B=16, Hq=8, Hkv=8, N=3000, Bc=1024)
    assert p.group == 1 and p.decode_stages() == ["unit"]
    q = queries(w, means, 50).to(DEV)
    for T in (64, 700):
        a = mp.decode(p, q, K.to(DEV), V.to(DEV), 3000, state, T).cpu()
        b = mp.decode(p, q, K.to(DEV), V.to(DEV), 3000, state, T, mode=mp.MODE_PER_HEAD).cpu()
        assert torch.equal(a, b)


def test_per_head_selection_on_gpu_state_with_tail_and_replicas():
    """GPU-built state, an unclustered tail, and few enough units that each
    query head's step is split over several workgroups."""
    mp, w, K, V, means, p, state = _built(B=2, Hq=32, Hkv=8, N=4500, Bc=1024)
    assert p.decode_stages() == ["unit"]
    G = p.group
    n_cl = state.n_clustered
    q = queries(w, means, 60)
    for T in (100, 900):
        out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 4500, state, T, mode=mp.MODE_PER_HEAD).cpu().numpy()
        for b, hq in ((0, 0), (0, 5), (1, 17), (1, 31)):
            st = oracle_state_from_gpu(state, b, hq // G, p)
            ref = O.decode_unit(q[b, hq:hq + 1], K[b, hq // G], V[b, hq // G], 4500, st, T)
            ok, ea, er = close(out[b, hq:hq + 1], ref.out)
            assert ok, (b, hq, T, ea, er, n_cl)


# ---------------------------------------------------------------------------
# fp8 centroid copies: codes bit-exact against the oracle's encoder of the
# GPU's own stored centroids; the decode against the oracle's decode of the
# decoded centroids
# ---------------------------------------------------------------------------
def _check_codes(state, b, h, lo, hi):
    from oracle import centroid_codes as F
    for src, codes, scales in ((state.key_centroids, state.key_codes, state.key_scales),
                               (state.value_centroids, state.value_codes, state.value_scales)):
        want_c, want_s = F.encode_rows(src[b, h, lo:hi].double().cpu().numpy())
        assert np.array_equal(codes[b, h, lo:hi].cpu().numpy(), want_c), (b, h)
        assert np.array_equal(scales[b, h, lo:hi].cpu().numpy(), want_s), (b, h)


def _coded_unit(state, b, h, p):
    from oracle import centroid_codes as F
    return F.coded_state(oracle_state_from_gpu(state, b, h, p))


def test_fp8_codes_match_oracle_encoder():
    mp, w, K, V, means, p, state = _built(B=16, Hq=32, Hkv=8, N=3000, Bc=1024, fmt=1)
    C = state.n_clusters
    for u in (0, 1, 77, 127):
        _check_codes(state, u // 8, u % 8, 0, C)
    # scale bytes stay in 1 .. 254 and no code is NaN
    for t in (state.key_codes, state.value_codes):
        assert not torch.any((t[:, :, :C] & 0x7F) == 0x7F)
    assert int(state.key_scales[:, :, :C].min()) >= 1 and int(state.key_scales[:, :, :C].max()) <= 254


@pytest.mark.parametrize("mode", ["multipole", "omit", "per_head"])
def test_fp8_decode_matches_oracle(mode):
    mp, w, K, V, means, p, state = _built(B=16, Hq=32, Hkv=8, N=3000, Bc=1024, fmt=1)
    ps = dataclasses.replace(p, centroid_format=0)
    assert p.decode_stages() == ["unit"]
    md = {"multipole": mp.MODE_MULTIPOLE, "omit": mp.MODE_OMIT, "per_head": mp.MODE_PER_HEAD}[mode]
    G = p.group
    n_tie = 0
    for step, T in enumerate((64, 700)):
        q = queries(w, means, 70 + step)
        dbg = mp.DecodeDebug.allocate(p, state, DEV, per_head=md == mp.MODE_PER_HEAD)
        out = mp.decode(p, q.to(DEV), K.to(DEV), V.to(DEV), 3000, state, T, mode=md, debug=dbg).cpu().numpy()
        stored = mp.decode(ps, q.to(DEV), K.to(DEV), V.to(DEV), 3000, state, T, mode=md).cpu().numpy()
        assert not np.array_equal(out, stored)  # the codes are what the decode read
        sel = dbg.selected.cpu().numpy()
        for u in (0, 37, 127):
            b, h = divmod(u, p.n_kv_heads)
            st = _coded_unit(state, b, h, p)
            heads = [(hq, hq, hq + 1) for hq in (h * G, h * G + G - 1)] if md == mp.MODE_PER_HEAD \
                else [(h, h * G, (h + 1) * G)]
            for sidx, g0, g1 in heads:
                qu = q[b, g0:g1]
                ref = O.decode_unit(qu, K[b, h], V[b, h], 3000, st, T, mode=1 if mode == "omit" else 0)
                C = st.n_clusters
                got_sel = sel[b, sidx, :C]
                if np.array_equal(got_sel, ref.selected):
                    want = ref.out
                else:
                    n_tie += 1
                    tol = rank_tolerance(O.f64(qu), st.kbar[:C])
                    assert selection_is_valid(ref.r, tol, st.sizes[:C], T, got_sel), (u, sidx, T)
                    want = O.decode_with_selection(qu, K[b, h], V[b, h], 3000, st, got_sel,
                                                   mode=1 if mode == "omit" else 0)
                ok, ea, er = close(out[b, g0:g1], want)
                assert ok, (mode, u, sidx, T, ea, er)
    assert n_tie <= 2


def test_fp8_codes_follow_the_window_update():
    """The update writes the codes of the new clusters only; the old ones
    keep theirs (the decode may read them meanwhile)."""
    mp = M()
    B, Hq, Hkv, Bc = 16, 32, 8, 1024
    w = dataclasses.replace(small_workload(B, Hq, Hkv, 3000, 150, outliers=4), generated_blocks=2, cluster_block=Bc,
                            drift=0.2)
    K, V, means = workloads.make_cache(w)
    N = w.capacity
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=Bc, build_iters=3,
                  update_iters=2, seed=2, centroid_format=mp.CENTROIDS_FP8)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, 3000, state)
    C0 = state.n_clusters
    before = state.key_codes[:, :, :C0].clone(), state.value_scales[:, :, :C0].clone()
    mp.update_window(p, Kd, Vd, N, state)
    C1 = state.n_clusters
    assert C1 > C0
    assert torch.equal(state.key_codes[:, :, :C0], before[0]) and torch.equal(state.value_scales[:, :, :C0], before[1])
    for u in (3, 100):
        _check_codes(state, u // Hkv, u % Hkv, C0, C1)
    q = queries(w, means, 80)
    T = 300
    out = mp.decode(p, q.to(DEV), Kd, Vd, N, state, T).cpu().numpy()
    G = p.group
    for u in (3, 100):
        b, h = divmod(u, Hkv)
        ref = O.decode_unit(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], N, _coded_unit(state, b, h, p), T)
        ok, ea, er = close(out[b, h * G:(h + 1) * G], ref.out)
        assert ok, (u, ea, er)


# ---------------------------------------------------------------------------
# the hierarchical decode in one launch, against the six launches and the
# oracle
# ---------------------------------------------------------------------------
HIER_CASES = [
    # B, Hq, Hkv, n_clustered, n_total, block, coarse tokens per centroid, T_cand, budgets, sorted copy
    (4, 32, 8, 16384, 16384, 4096, 128, 2048, (256, 1000), True),
    (2, 8, 2, 12000, 13000, 4096, 64, 4096, (0, 300), False),
    (1, 4, 4, 9000, 9000, 2048, 128, 512, (100, 2000), True),
    # no candidates (every coarse cluster approximated); every token a candidate
    (2, 8, 8, 6000, 6500, 2048, 128, 0, (0, 300), True),
    (2, 16, 8, 3000, 3000, 1024, 128, 4096, (0, 3000), False),
]


@pytest.mark.parametrize("case", HIER_CASES, ids=lambda c: f"B{c[0]}-G{c[1] // c[2]}-N{c[4]}-cand{c[7]}")
def test_hier_one_launch_matches_six_launches_and_oracle(case):
    mp = M()
    B, Hq, Hkv, n_cl, n_tot, Bc, ctpc, Tc, budgets, sorted_copy = case
    w = small_workload(B, Hq, Hkv, n_tot, max(8, n_tot // 16), outliers=4, index=92)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=n_tot, cluster_block=Bc, build_iters=3,
                  coarse_tokens_per_centroid=ctpc, coarse_candidate_tokens=Tc, seed=3)
    assert p.decode_stages() == ["hier_unit"]
    ps = dataclasses.replace(p, splits=4)
    state = mp.ClusterState(p, DEV, sorted_copy=sorted_copy)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, n_cl, state)
    G = p.group
    for step, T in enumerate(budgets):
        q = queries(w, means, 90 + step)
        d1, d6 = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        o1 = mp.decode(p, q.to(DEV), Kd, Vd, n_tot, state, T, debug=d1).cpu().numpy()
        o6 = mp.decode(ps, q.to(DEV), Kd, Vd, n_tot, state, T, debug=d6).cpu().numpy()
        # the same keys and cuts from the same operations: identical decisions
        assert torch.equal(d1.candidates.cpu(), d6.candidates.cpu()), T
        assert torch.equal(d1.selected.cpu(), d6.selected.cpu()), T
        assert torch.equal(d1.exact_tokens.cpu(), d6.exact_tokens.cpu()), T
        np.testing.assert_allclose(o1, o6, rtol=1e-4, atol=1e-5)
        cand, sel = d1.candidates.cpu().numpy(), d1.selected.cpu().numpy()
        for u in sorted({0, p.units // 2, p.units - 1}):
            b, h = divmod(u, Hkv)
            st = oracle_state_from_gpu(state, b, h, p)
            qu = q[b, h * G:(h + 1) * G]
            q64 = O.f64(qu)
            ref = O.decode_unit_hier(qu, K[b, h], V[b, h], n_tot, st, T, Tc)
            want = ref.out
            D, C = st.n_coarse, st.n_clusters
            if not np.array_equal(cand[b, h], ref.candidates):
                cr = (q64 @ st.ckbar[:D].T).mean(0) / np.sqrt(128)
                assert selection_is_valid(cr, rank_tolerance(q64, st.ckbar[:D]), st.csizes[:D], Tc, cand[b, h])
            if not (np.array_equal(cand[b, h], ref.candidates) and np.array_equal(sel[b, h], ref.selected)):
                forced = O.decode_unit_hier(qu, K[b, h], V[b, h], n_tot, st, T, Tc, candidates=cand[b, h])
                inside = st.sizes[:C] * (cand[b, h][np.maximum(st.parent[:C], 0)] > 0) * (st.parent[:C] >= 0)
                assert selection_is_valid(forced.r, rank_tolerance(q64, st.kbar[:C]), inside.astype(np.int32), T,
                                          sel[b, h]), (u, T)
                want = O.decode_unit_hier(qu, K[b, h], V[b, h], n_tot, st, T, Tc, candidates=cand[b, h],
                                          selected=sel[b, h]).out
            ok, ea, er = close(o1[b, h * G:(h + 1) * G], want)
            assert ok, (u, T, ea, er)
            assert st.sizes[:C][sel[b, h].astype(bool)].sum() <= T
            assert d1.exact_tokens.cpu().numpy()[b, h] == st.sizes[:C][sel[b, h].astype(bool)].sum()


def test_hier_coarse_build_rounds_match_oracle():
    """The GPU's coarse level on a hierarchical shape (4 blocks of 4096
    tokens, 32 coarse clusters each), teacher forced on three units: the
    last weighted round from the GPU's state one round earlier, the first
    round from the oracle's seeded init (parents outside tie windows,
    weighted means, exact sizes, member lists and offsets, size-weighted
    value centroids)."""
    mp = M()
    B, Hq, Hkv, N = 4, 32, 8, 16384
    w = small_workload(B, Hq, Hkv, N, N // 16, outliers=4, index=92)
    K, V, _ = workloads.make_cache(w)
    base = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=4096, build_iters=3,
                coarse_tokens_per_centroid=128, coarse_candidate_tokens=2048, seed=3)
    Kd, Vd = K.to(DEV), V.to(DEV)
    states = {}
    for it in (1, 9, 10):
        p = mp.Params(coarse_iters=it, **base)
        states[it] = mp.ClusterState(p, DEV, sorted_copy=False)
        mp.build_clusters(p, Kd, Vd, N, states[it])
    torch.cuda.synchronize()
    p = states[10].params
    for u in (0, 13, p.units - 1):
        b, h = divmod(u, Hkv)
        check_coarse_round(p, states[9], states[10], b, h, seed=3)
        check_coarse_round(p, None, states[1], b, h, seed=3, from_init=True)


def test_hier_one_launch_zero_queries_take_clusters_in_id_order():
    """Zero queries make every coarse and fine key exactly 0: both cuts of
    the one-launch kernel take their exact radix passes (a degenerate key
    range) and break the ties by id, as the six launches and the oracle do."""
    mp = M()
    B, Hq, Hkv, N = 2, 16, 8, 9000
    w = small_workload(B, Hq, Hkv, N, N // 16, outliers=4, index=94)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=2048, build_iters=3,
                  coarse_tokens_per_centroid=128, coarse_candidate_tokens=1000, seed=6)
    assert p.decode_stages() == ["hier_unit"]
    ps = dataclasses.replace(p, splits=4)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, N, state)
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16)
    G = p.group
    for T in (100, 700):
        d1, d6 = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        o1 = mp.decode(p, q.to(DEV), Kd, Vd, N, state, T, debug=d1).cpu().numpy()
        o6 = mp.decode(ps, q.to(DEV), Kd, Vd, N, state, T, debug=d6).cpu().numpy()
        assert torch.equal(d1.candidates.cpu(), d6.candidates.cpu()), T
        assert torch.equal(d1.selected.cpu(), d6.selected.cpu()), T
        np.testing.assert_allclose(o1, o6, rtol=1e-4, atol=1e-5)
        for u in (0, p.units - 1):
            b, h = divmod(u, Hkv)
            st = oracle_state_from_gpu(state, b, h, p)
            ref = O.decode_unit_hier(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], N, st, T, 1000)
            assert np.array_equal(d1.candidates.cpu().numpy()[b, h, :st.n_coarse], ref.candidates), (u, T)
            assert np.array_equal(d1.selected.cpu().numpy()[b, h, :st.n_clusters], ref.selected), (u, T)
            ok, ea, er = close(o1[b, h * G:(h + 1) * G], ref.out)
            assert ok, (u, T, ea, er)


def test_hier_one_launch_outlier_keys_match_six_launches():
    """64 tokens far along one direction that the queries share give one
    coarse and a few fine clusters keys in the thousands: the rest of each
    level then shares one value bin, so both cuts of the one-launch kernel
    take their exact radix passes over a crowded bin (192 coarse clusters,
    about 270 fine candidates per unit).  Decisions must equal the six
    launches' radix cuts."""
    mp = M()
    B, Hq, Hkv, N = 2, 16, 8, 24576
    w = small_workload(B, Hq, Hkv, N, N // 16, outliers=4, index=95)
    K, V, means = workloads.make_cache(w)
    v = torch.randn(128, generator=torch.Generator().manual_seed(5))
    v = v / v.norm()
    K[:, :, :64] = (20000.0 * v).to(K.dtype)
    q = (queries(w, means, 7).float() + 3.0 * v).to(torch.bfloat16)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=8192, build_iters=3,
                  coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096, seed=7)
    assert p.decode_stages() == ["hier_unit"]
    ps = dataclasses.replace(p, splits=4)
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, N, state)
    assert state.n_coarse > 128
    for T in (100, 700):
        d1, d6 = mp.DecodeDebug.allocate(p, state, DEV), mp.DecodeDebug.allocate(ps, state, DEV)
        o1 = mp.decode(p, q.to(DEV), Kd, Vd, N, state, T, debug=d1).cpu().numpy()
        o6 = mp.decode(ps, q.to(DEV), Kd, Vd, N, state, T, debug=d6).cpu().numpy()
        assert torch.equal(d1.candidates.cpu(), d6.candidates.cpu()), T
        assert torch.equal(d1.selected.cpu(), d6.selected.cpu()), T
        assert torch.equal(d1.exact_tokens.cpu(), d6.exact_tokens.cpu()), T
        np.testing.assert_allclose(o1, o6, rtol=1e-4, atol=1e-5)


def test_hier_one_launch_rescore_gives_the_same_result():
    """The workgroups of a unit score a share of the coarse clusters each and
    exchange the keys; scoring all of them locally (rescore 1) or falling back
    as when a partner is late (rescore 2) must give the same bits."""
    mp = M()
    B, Hq, Hkv, N = 4, 32, 8, 16384
    w = small_workload(B, Hq, Hkv, N, N // 16, outliers=4, index=93)
    K, V, means = workloads.make_cache(w)
    p = mp.Params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, capacity_tokens=N, cluster_block=4096, build_iters=3,
                  coarse_tokens_per_centroid=128, coarse_candidate_tokens=2048, seed=4)
    assert p.decode_stages() == ["hier_unit"]
    state = mp.ClusterState(p, DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    mp.build_clusters(p, Kd, Vd, N, state)
    ws = mp.Workspace().get(p, state, DEV)
    for step, T in enumerate((128, 900)):
        q = queries(w, means, 100 + step).to(DEV)
        outs, dbgs = [], []
        for rescore in (0, 1, 2, 0):
            d = mp.DecodeDebug.allocate(p, state, DEV)
            d.rescore = rescore
            before = mp.decode_status(ws)
            outs.append(mp.decode(p, q, Kd, Vd, N, state, T, debug=d, workspace=ws).cpu())
            after = mp.decode_status(ws)
            assert after[1] == 0
            if rescore == 2:
                assert after[0] - before[0] >= 3 * p.units
            dbgs.append(d)
        for o, d in zip(outs[1:], dbgs[1:]):
            assert torch.equal(o, outs[0]), T
            assert torch.equal(d.candidates.cpu(), dbgs[0].candidates.cpu())
            assert torch.equal(d.selected.cpu(), dbgs[0].selected.cpu())
            assert torch.equal(d.exact_tokens.cpu(), dbgs[0].exact_tokens.cpu())
