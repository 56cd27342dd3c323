"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle checks sampled units one by one (teacher forced:
it starts from the GPU's own state), and every unit where a check is cheap.

Workloads: tiny-fp32 (covered in test_gpu_parity), the Qwen3-8B-shaped layer
at batch 1 (budgets 128 and 512) and batch 16 (95% sparsity), the online
update at batch 4, and the two-level hierarchy at 128K context.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from gpu_util import (assign_tie_violations, check_coarse_round, close, gamma, oracle_state_from_gpu,
                      rank_tolerance, selection_is_valid, U32)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def M():
    from sparse_long_context_means_amd import mpattn

    return mpattn


def params_for(w, **kw):
    mp = M()
    base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, capacity_tokens=w.capacity,
                dtype=w.dtype, tokens_per_centroid=w.tokens_per_centroid, cluster_block=w.cluster_block,
                build_iters=w.build_iters, update_iters=w.update_iters,
                coarse_tokens_per_centroid=w.coarse_tokens_per_centroid,
                coarse_candidate_tokens=w.coarse_candidate_tokens, seed=0)
    base.update(kw)
    return mp.Params(**base)


def check_decode_units(p, state, q, K, V, n_total, T, out, sel, units, Ku=None, Vu=None):
    """Oracle decode of the given units on the GPU's state; selection within
    tie windows, outputs within 2e-3 abs + 1e-2 rel."""
    G = p.group
    diff = 0
    for u in units:
        b, h = divmod(u, p.n_kv_heads)
        st = oracle_state_from_gpu(state, b, h, p)
        qu = q[b, h * G:(h + 1) * G]
        Kh = K[b, h] if Ku is None else Ku[u]
        Vh = V[b, h] if Vu is None else Vu[u]
        ref = O.decode_unit(qu, Kh, Vh, n_total, st, T)
        C = st.n_clusters
        if np.array_equal(sel[b, h], ref.selected):
            want = ref.out
        else:
            diff += 1
            tol = rank_tolerance(O.f64(qu), st.kbar[:C])
            assert selection_is_valid(ref.r, tol, st.sizes[:C], T, sel[b, h]), f"unit {u}: selection"
            want = O.decode_with_selection(qu, Kh, Vh, n_total, st, sel[b, h])
        ok, ea, er = close(out[b, h * G:(h + 1) * G], want)
        assert ok, f"unit {u} budget {T}: max abs {ea:.3g}, max rel {er:.3g}"
    return diff


def check_last_round(p, K, V, n_tokens, unit, block, state_prev, state_last):
    """Teacher-forced check of the last Lloyd round of one (unit, block):
    assignment from the previous round's stored centroids, then the update."""
    b, h = divmod(unit, p.n_kv_heads)
    prev = oracle_state_from_gpu(state_prev, b, h, p)
    cur = oracle_state_from_gpu(state_last, b, h, p)
    blk = cur.blocks[block]
    x = O.f64(K[b, h, blk.p:blk.p + blk.L])
    mus_prev = prev.kbar[blk.c0:blk.c0 + blk.C]
    a_ref, _, _ = O.assign_step(x, mus_prev)
    a_gpu = cur.assign[blk.p:blk.p + blk.L] - blk.c0
    nd, bad = assign_tie_violations(x, mus_prev, a_gpu, a_ref)
    assert not bad, f"{len(bad)} assignments outside the tie window"
    mu, mus, counts = O.update_step(x, a_gpu, prev.mu[blk.c0:blk.c0 + blk.C], mus_prev, O.BF16)
    np.testing.assert_array_equal(cur.sizes[blk.c0:blk.c0 + blk.C], counts)
    live = counts > 0
    gm = cur.mu[blk.c0:blk.c0 + blk.C]
    absmean = np.zeros_like(mu)
    np.add.at(absmean, a_gpu, np.abs(x))
    absmean[live] /= counts[live, None]
    bound = gamma(counts[:, None] + 1) * absmean + U32 * np.abs(mu)
    assert np.all(np.abs(gm - mu)[live] <= bound[live] + 1e-30)
    np.testing.assert_array_equal(cur.kbar[blk.c0:blk.c0 + blk.C], O.round_storage(gm, O.BF16))
    return nd


@pytest.fixture(scope="module")
def layer_b1():
    w = workloads.WORKLOADS["qwen3-8b-layer-b1-32k"]
    K, V, means = workloads.make_cache(w)
    return w, K, V, means


def test_qwen3_layer_b1_full(layer_b1):
    """32K context, 8 KV heads, 10 rounds: last round teacher-forced on two
    (unit, block) samples; decode at budgets 128 and 512 on every unit."""
    mp = M()
    w, K, V, means = layer_b1
    Kd, Vd = K.to(DEV), V.to(DEV)
    p9 = params_for(w, build_iters=w.build_iters - 1)
    p = params_for(w)
    s9 = mp.ClusterState(p9, DEV, sorted_copy=False)
    s10 = mp.ClusterState(p, DEV)
    mp.build_clusters(p9, Kd, Vd, w.n_tokens, s9)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, s10)
    torch.cuda.synchronize()
    assert s10.n_clusters == 2048
    nd = sum(check_last_round(p, K, V, w.n_tokens, u, j, s9, s10) for u, j in ((0, 0), (5, 3)))
    print(f"tie-window assignment differences: {nd}")
    for step, T in enumerate(w.budgets):
        q = workloads.make_queries(w, means, step)
        dbg = mp.DecodeDebug.allocate(p, s10, DEV)
        out = mp.decode(p, q.to(DEV), Kd, Vd, w.n_tokens, s10, T, debug=dbg).cpu().numpy()
        sel = dbg.selected.cpu().numpy()
        exact = dbg.exact_tokens.cpu().numpy()
        assert np.all(exact <= T) and np.all(exact > 0)
        check_decode_units(p, s10, q, K, V, w.n_tokens, T, out, sel, range(p.units))


def test_qwen3_layer_b16_sparse95_sampled():
    """Batch 16, 32K, 95% sparsity (1638 tokens per KV head), the benchmark's
    configuration: decode of 16 sampled units checked by the oracle for two
    queries, one (unit, block) last round teacher-forced."""
    mp = M()
    w = workloads.WORKLOADS["qwen3-8b-layer-b16-32k-s95"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(DEV), V.to(DEV)
    p = params_for(w)
    p9 = params_for(w, build_iters=w.build_iters - 1)
    s10 = mp.ClusterState(p, DEV)
    s9 = mp.ClusterState(p9, DEV, sorted_copy=False)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, s10)
    mp.build_clusters(p9, Kd, Vd, w.n_tokens, s9)
    torch.cuda.synchronize()
    check_last_round(p, K, V, w.n_tokens, 77, 2, s9, s10)
    del s9
    rng = np.random.default_rng(0)
    sample = sorted(rng.choice(p.units, 16, replace=False).tolist())
    T = w.budgets[0]
    for step in range(2):
        q = workloads.make_queries(w, means, step)
        dbg = mp.DecodeDebug.allocate(p, s10, DEV)
        out = mp.decode(p, q.to(DEV), Kd, Vd, w.n_tokens, s10, T, debug=dbg).cpu().numpy()
        sel = dbg.selected.cpu().numpy()
        exact = dbg.exact_tokens.cpu().numpy()
        assert np.all(exact <= T) and exact.mean() > 0.9 * T
        check_decode_units(p, s10, q, K, V, w.n_tokens, T, out, sel, sample)


def _clone(state):
    mp = M()
    c = mp.ClusterState.__new__(mp.ClusterState)
    for k, v in state.__dict__.items():
        setattr(c, k, v.clone() if isinstance(v, torch.Tensor) else v)
    return c


def test_online_update_phases():
    """Batch 4: a 16384-token prompt is clustered, then two generated blocks
    of 8192 tokens (drifted means) arrive.  At each phase the decode (with the
    unclustered tail attended exactly) is checked on every unit; the update's
    last round is teacher-forced on a sample."""
    mp = M()
    w = workloads.WORKLOADS["qwen3-8b-layer-b4-online"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(DEV), V.to(DEV)
    p = params_for(w)
    p4 = params_for(w, update_iters=w.update_iters - 1)
    state = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, state)
    T = w.budgets[0]
    n = w.n_tokens
    step = 0
    for phase in range(w.generated_blocks):
        # generated tokens arrive in 1024-token pieces; decode sees them as tail
        for n_total in (n + 1024, n + 4096, n + w.cluster_block - 1):
            assert mp.update_window(p, Kd, Vd, n_total, state) == 0
            q = workloads.make_queries(w, means, step)
            dbg = mp.DecodeDebug.allocate(p, state, DEV)
            out = mp.decode(p, q.to(DEV), Kd, Vd, n_total, state, T, debug=dbg).cpu().numpy()
            check_decode_units(p, state, q, K, V, n_total, T, out, dbg.selected.cpu().numpy(), range(p.units))
            step += 1
        n_total = n + w.cluster_block
        before = _clone(state)
        prev = _clone(state)
        assert mp.update_window(p4, Kd, Vd, n_total, prev) == 1
        assert mp.update_window(p, Kd, Vd, n_total, state) == 1
        assert state.n_clustered == n_total and state.n_blocks == before.n_blocks + 1
        # earlier blocks are untouched by the update
        C0 = before.n_clusters
        assert torch.equal(state.key_centroids[:, :, :C0], before.key_centroids[:, :, :C0])
        assert torch.equal(state.assign[:, :, :n], before.assign[:, :, :n])
        check_last_round(p, K, V, n_total, 3 + 8 * phase, state.n_blocks - 1, prev, state)
        n = n_total
    q = workloads.make_queries(w, means, step)
    dbg = mp.DecodeDebug.allocate(p, state, DEV)
    out = mp.decode(p, q.to(DEV), Kd, Vd, n, state, T, debug=dbg).cpu().numpy()
    check_decode_units(p, state, q, K, V, n, T, out, dbg.selected.cpu().numpy(), range(p.units))


def test_concurrent_update_leaves_the_old_state_usable():
    """The window update on a second stream while decodes continue on the
    first with the state as it was: every decode during the update gives the
    bits of the decode on the old state, and after the update's event the
    decode gives the bits of a serial update."""
    mp = M()
    w = workloads.WORKLOADS["qwen3-8b-layer-b4-online"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(DEV), V.to(DEV)
    p = params_for(w)
    T = w.budgets[0]
    n_prompt, n_total = w.n_tokens, w.n_tokens + w.cluster_block
    q = workloads.make_queries(w, means, 0).to(DEV)
    # serial reference: before and after the update
    ref_state = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, n_prompt, ref_state)
    before = mp.decode(p, q, Kd, Vd, n_total, ref_state, T).clone()
    assert mp.update_window(p, Kd, Vd, n_total, ref_state) == 1
    after = mp.decode(p, q, Kd, Vd, n_total, ref_state, T).clone()
    assert not torch.equal(before, after)
    # concurrent: decodes on the current stream while the update runs
    state = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, n_prompt, state)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    view, done, added = mp.update_window_concurrent(p, Kd, Vd, n_total, state, side)
    assert added == 1 and view.n_clustered == n_prompt and state.n_clustered == n_total
    ws = mp.Workspace().get(p, view, DEV)
    dbg_view = mp.DecodeDebug.allocate(p, view, DEV)
    outs = [mp.decode(p, q, Kd, Vd, n_total, view, T, workspace=ws, debug=dbg_view if i == 0 else None).clone()
            for i in range(12)]
    overlapped = not done.query()  # the update was still running after the decodes were enqueued
    torch.cuda.current_stream().wait_event(done)
    dbg_new = mp.DecodeDebug.allocate(p, state, DEV)
    new = mp.decode(p, q, Kd, Vd, n_total, state, T, workspace=ws, debug=dbg_new)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, before)
    assert torch.equal(new, after)
    print("update still running while the decodes were enqueued:", overlapped)
    # the oracle on sampled units: during the update, the old clusters with
    # the new block as an unclustered tail attended exactly; after it, the
    # new block's clusters
    sample = [0, 9, 18, 31]
    qc = q.cpu()
    check_decode_units(p, view, qc, K, V, n_total, T, outs[0].cpu().numpy(), dbg_view.selected.cpu().numpy(), sample)
    assert view.n_clustered == n_prompt
    check_decode_units(p, state, qc, K, V, n_total, T, new.cpu().numpy(), dbg_new.selected.cpu().numpy(), sample)


def test_update_equals_build_on_gpu():
    """Clustering a prompt and then appending aligned blocks gives the state
    one build over the whole length gives, when the round counts agree."""
    mp = M()
    w = dataclasses.replace(workloads.WORKLOADS["qwen3-8b-layer-b4-online"], batch=1, n_kv_heads=2, n_q_heads=8)
    K, V, _ = workloads.make_cache(w)
    Kd, Vd = K.to(DEV), V.to(DEV)
    p = params_for(w, build_iters=5, update_iters=5)
    whole = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, w.capacity, whole)
    part = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, part)
    assert mp.update_window(p, Kd, Vd, w.capacity, part) == w.generated_blocks
    for name in ("key_centroids", "value_centroids", "sizes", "offsets", "token_ids", "assign", "sorted_keys"):
        assert torch.equal(getattr(whole, name), getattr(part, name)), name


def test_hierarchical_128k_sampled():
    """Two-level variant at 131072 tokens: the coarse level is checked against
    the oracle's coarse build on the GPU's fine state, and the decode
    (candidates, fine selection, output) on sampled units."""
    mp = M()
    w = workloads.WORKLOADS["qwen3-8b-layer-b4-128k-hier"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(DEV), V.to(DEV)
    p = params_for(w)
    state = mp.ClusterState(p, DEV)
    mp.build_clusters(p, Kd, Vd, w.n_tokens, state)
    torch.cuda.synchronize()
    assert state.n_clusters == 8192 and state.n_coarse == 1024
    G = p.group
    T, Tc = w.budgets[0], w.coarse_candidate_tokens
    rng = np.random.default_rng(1)
    sample = sorted(rng.choice(p.units, 4, replace=False).tolist())
    # coarse level, teacher forced: the last weighted round from the GPU's
    # state one round earlier, and the first round from the oracle's own
    # seeded init, on every block of two sampled units
    prev = mp.ClusterState(dataclasses.replace(p, coarse_iters=p.coarse_iters - 1), DEV, sorted_copy=False)
    mp.build_clusters(prev.params, Kd, Vd, w.n_tokens, prev)
    one = mp.ClusterState(dataclasses.replace(p, coarse_iters=1), DEV, sorted_copy=False)
    mp.build_clusters(one.params, Kd, Vd, w.n_tokens, one)
    torch.cuda.synchronize()
    nd = 0
    for u in sample[:2]:
        b, h = divmod(u, p.n_kv_heads)
        nd += check_coarse_round(p, prev, state, b, h)
        nd += check_coarse_round(p, None, one, b, h, from_init=True)
    print(f"coarse tie-window assignment differences: {nd}")
    del prev, one
    for step in range(2):
        q = workloads.make_queries(w, means, step)
        dbg = mp.DecodeDebug.allocate(p, state, DEV)
        out = mp.decode(p, q.to(DEV), Kd, Vd, w.n_tokens, state, T, debug=dbg).cpu().numpy()
        sel = dbg.selected.cpu().numpy()
        cand = dbg.candidates.cpu().numpy()
        for u in sample:
            b, h = divmod(u, p.n_kv_heads)
            st = oracle_state_from_gpu(state, b, h, p)
            qu = q[b, h * G:(h + 1) * G]
            q64 = O.f64(qu)
            ref = O.decode_unit_hier(qu, K[b, h], V[b, h], w.n_tokens, st, T, Tc)
            want = ref.out
            if not np.array_equal(cand[b, h], ref.candidates):
                D = st.n_coarse
                cr = (q64 @ st.ckbar[:D].T).mean(0) / np.sqrt(128)
                tol = rank_tolerance(q64, st.ckbar[:D])
                assert selection_is_valid(cr, tol, st.csizes[:D], Tc, cand[b, h]), f"unit {u}: candidates"
            if not (np.array_equal(cand[b, h], ref.candidates) and np.array_equal(sel[b, h], ref.selected)):
                forced = O.decode_unit_hier(qu, K[b, h], V[b, h], w.n_tokens, st, T, Tc, candidates=cand[b, h])
                inside = st.sizes[:st.n_clusters] * (cand[b, h][np.maximum(st.parent[:st.n_clusters], 0)] > 0) \
                    * (st.parent[:st.n_clusters] >= 0)
                tol = rank_tolerance(q64, st.kbar[:st.n_clusters])
                assert selection_is_valid(forced.r, tol, inside.astype(np.int32), T, sel[b, h]), f"unit {u}: fine"
                want = O.decode_unit_hier(qu, K[b, h], V[b, h], w.n_tokens, st, T, Tc, candidates=cand[b, h],
                                          selected=sel[b, h]).out
            ok, ea, er = close(out[b, h * G:(h + 1) * G], want)
            assert ok, f"unit {u}: max abs {ea:.3g}"
            assert st.sizes[:st.n_clusters][sel[b, h].astype(bool)].sum() <= T
