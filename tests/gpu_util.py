"""Helpers of the GPU parity tests: moving cluster state between the oracle's
per-unit numpy form and the library's device arrays, and the acceptance rules
for integer decisions taken from floating-point scores.

Tie windows.  The GPU takes nearest-centroid and ranking decisions from fp32
sums; the oracle from fp64.  A differing decision is accepted only when the
two candidates' fp64 scores are closer than the rigorous bound on the fp32
rounding of the GPU's sum (Higham: |fl(sum) - sum| <= gamma_n * sum |terms|,
gamma_n = n u / (1 - n u), u = 2^-24), or than 1e-6 relative.
"""
import math

import numpy as np
import torch

import oracle as O

U32 = 2.0 ** -24


def gamma(n):
    return n * U32 / (1 - n * U32)


def storage_of(dtype):
    return O.BF16 if dtype == torch.bfloat16 else O.F32


# ---------------------------------------------------------------------------
# state transfer
# ---------------------------------------------------------------------------

def oracle_state_from_gpu(state, b, h, params) -> O.UnitState:
    """Copies unit (b, h) of a device ClusterState into an oracle UnitState."""
    C, n = state.n_clusters, state.n_clustered
    st = O.empty_state(params.head_dim, params.capacity_tokens, state.capacity_clusters, storage_of(params.dtype))
    st.kbar[:C] = state.key_centroids[b, h, :C].double().cpu().numpy()
    st.vbar[:C] = state.value_centroids[b, h, :C].double().cpu().numpy()
    st.mu[:C] = state.key_centroids_f32[b, h, :C].double().cpu().numpy()
    st.sizes[:C] = state.sizes[b, h, :C].cpu().numpy()
    st.offsets[:C + 1] = state.offsets[b, h, :C + 1].cpu().numpy()
    st.token_ids[:n] = state.token_ids[b, h, :n].cpu().numpy()
    st.assign[:n] = state.assign[b, h, :n].cpu().numpy()
    st.n_clusters, st.n_clustered = C, n
    # block table implied by the build/update history (regular blocks)
    Bc, r = params.cluster_block, params.tokens_per_centroid
    p, c0, j = 0, 0, 0
    while p < n:
        L = min(Bc, n - p)
        Cj = -(-L // r)
        st.blocks.append(O.Block(p, L, c0, Cj, j))
        p, c0, j = p + L, c0 + Cj, j + 1
    if params.hierarchical:
        D = state.n_coarse
        st.ckbar = state.coarse_key_centroids[b, h, :D].double().cpu().numpy()
        st.cvbar = state.coarse_value_centroids[b, h, :D].double().cpu().numpy()
        st.cmu = state.coarse_key_centroids_f32[b, h, :D].double().cpu().numpy()
        st.csizes = state.coarse_sizes[b, h, :D].cpu().numpy().astype(np.int32)
        st.coffsets = state.coarse_offsets[b, h, :D + 1].cpu().numpy().astype(np.int32)
        st.cmembers = state.coarse_members[b, h].cpu().numpy().astype(np.int32)
        st.parent = state.parent[b, h].cpu().numpy().astype(np.int32)
        st.n_coarse = D
    return st


def load_oracle_states(state, params, units, K=None, V=None):
    """Writes oracle UnitStates (list indexed by unit = b * Hkv + h) into a
    device ClusterState; fills the sorted copy from K/V when it exists."""
    dev = state.key_centroids.device
    Hkv = params.n_kv_heads
    dt = params.dtype
    for u, st in enumerate(units):
        b, h = divmod(u, Hkv)
        C, n = st.n_clusters, st.n_clustered
        state.key_centroids[b, h, :C] = torch.from_numpy(st.kbar[:C]).to(dt).to(dev)
        state.value_centroids[b, h, :C] = torch.from_numpy(st.vbar[:C]).to(dt).to(dev)
        state.key_centroids_f32[b, h, :C] = torch.from_numpy(st.mu[:C]).float().to(dev)
        state.sizes[b, h, :C] = torch.from_numpy(st.sizes[:C]).to(dev)
        state.offsets[b, h, :C + 1] = torch.from_numpy(st.offsets[:C + 1]).to(dev)
        state.token_ids[b, h, :n] = torch.from_numpy(st.token_ids[:n]).to(dev)
        state.assign[b, h, :n] = torch.from_numpy(st.assign[:n]).to(dev)
        if state.sorted_keys is not None:
            ids = torch.from_numpy(st.token_ids[:n]).long()
            state.sorted_keys[b, h, :n] = K[b, h, ids].to(dev)
            state.sorted_values[b, h, :n] = V[b, h, ids].to(dev)
    state.n_clusters = units[0].n_clusters
    state.n_clustered = units[0].n_clustered
    state.n_blocks = len(units[0].blocks)


# ---------------------------------------------------------------------------
# acceptance rules
# ---------------------------------------------------------------------------

def assign_tie_violations(x, mu_s, a_gpu, a_ref):
    """Indices where the GPU's nearest centroid differs from the oracle's by
    more than the fp32 rounding window.  Returns (n_differing, violations)."""
    diff = np.nonzero(a_gpu != a_ref)[0]
    bad = []
    for i in diff:
        c1, c0 = int(a_gpu[i]), int(a_ref[i])
        D = lambda c: float(x[i] @ mu_s[c] - 0.5 * mu_s[c] @ mu_s[c])
        E = lambda c: gamma(130) * float(np.abs(x[i] * mu_s[c]).sum() + 0.5 * (mu_s[c] ** 2).sum())
        gap = D(c0) - D(c1)
        if gap > max(1e-6 * max(1.0, abs(D(c0))), E(c0) + E(c1)):
            bad.append(int(i))
    return len(diff), bad


def rank_tolerance(q, kbar):
    """Per-cluster bound on the fp32 rounding of the group-mean score."""
    d = q.shape[1]
    terms = np.abs(q)[:, None, :] * np.abs(kbar)[None, :, :]  # [G][C][d]
    s_abs = terms.sum(-1) / math.sqrt(d)
    r = (q @ kbar.T).mean(0) / math.sqrt(d)
    return gamma(d + 8) * s_abs.mean(0) + 8 * U32 * np.abs(r) + 1e-12


def selection_is_valid(r64, tol, sizes, budget, sel):
    """True when `sel` is the budget cut of some order that agrees with r64
    outside the tolerance windows."""
    sel = sel.astype(bool)
    live = sizes > 0
    if sizes[sel].sum() > budget or np.any(sel & ~live):
        return False
    inc, exc = np.nonzero(sel)[0], np.nonzero(~sel & live)[0]
    if len(inc) and len(exc):
        # no excluded cluster ranks clearly above an included one
        worst_in = inc[np.argmin(r64[inc] + tol[inc])]
        if np.any(r64[exc] - tol[exc] > r64[worst_in] + tol[worst_in]):
            return False
    if len(exc):
        # the selection stopped because a near-top excluded cluster did not fit
        top = r64[exc].max()
        near = exc[r64[exc] + tol[exc] >= top - tol[exc].max()]
        if not np.any(sizes[near] + sizes[sel].sum() > budget):
            return False
    return True


def close(gpu, ref, atol=2e-3, rtol=1e-2):
    """Elementwise |gpu - ref| <= atol + rtol * |ref|; returns (ok, max_abs, max_rel)."""
    err = np.abs(gpu - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref)))
    rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    return ok, float(err.max()) if err.size else 0.0, rel


# ---------------------------------------------------------------------------
# coarse level of the hierarchy (size-weighted Lloyd over each block's
# non-empty fine key centroids), teacher forced
# ---------------------------------------------------------------------------

def _rne_bracket(lo, hi, storage):
    """Storage values a correctly rounded result of any x in [lo, hi] can take."""
    return O.round_storage(lo, storage), O.round_storage(hi, storage)


def check_coarse_round(p, prev, cur, b, h, seed=0, from_init=False):
    """One teacher-forced weighted Lloyd round of the coarse level of unit
    (b, h), block by block.  `cur` holds the GPU state after k rounds; the
    round starts from `prev` (the GPU state after k - 1 rounds) or, with
    from_init, from the seeded init the oracle draws itself (cur after one
    round).  Checks, against the oracle's steps on the GPU's fine state:
    parents (nearest stored coarse centroid, ties to the lower id) outside
    the fp32 tie window; weighted means (fp32 master within the rounding
    bound of the fp64 size-weighted mean, stored copy = master rounded to
    nearest even); coarse sizes, member lists and offsets exactly; coarse
    value centroids within the bound of the size-weighted mean of the fine
    value centroids.  Returns the number of tie-window assignment
    differences."""
    storage = storage_of(p.dtype)
    unit = b * p.n_kv_heads + h
    c = oracle_state_from_gpu(cur, b, h, p)
    q = None if from_init else oracle_state_from_gpu(prev, b, h, p)
    C = c.n_clusters
    if q is not None:  # the fine level does not depend on the coarse rounds
        np.testing.assert_array_equal(q.kbar[:C], c.kbar[:C])
        np.testing.assert_array_equal(q.sizes[:C], c.sizes[:C])
    dfull = -(-p.cluster_block // p.coarse_tokens_per_centroid)
    n_diff, pos = 0, 0
    want_members = np.zeros(C, np.int32)
    for blk in c.blocks:
        g0 = blk.index * dfull
        ids = np.nonzero(c.sizes[blk.c0:blk.c0 + blk.C] > 0)[0].astype(np.int32) + blk.c0
        m = len(ids)
        D = min(-(-blk.L // p.coarse_tokens_per_centroid), m)
        x, wts = c.kbar[ids], c.sizes[ids].astype(np.float64)
        if from_init:
            idx = O.init_indices(O.block_stream(seed, unit, blk.index, 1), m, D)
            mu_prev = x[idx].copy()
            mus_prev = x[idx].copy()
        else:
            mu_prev, mus_prev = q.cmu[g0:g0 + D], q.ckbar[g0:g0 + D]
        a_ref, _, _ = O.assign_step(x, mus_prev)
        a_gpu = c.parent[ids] - g0
        assert np.all((a_gpu >= 0) & (a_gpu < D)), "parent outside the block's coarse clusters"
        nd, bad = assign_tie_violations(x, mus_prev, a_gpu, a_ref)
        assert not bad, f"unit {unit} block {blk.index}: {len(bad)} coarse assignments outside the tie window"
        n_diff += nd
        mu, _, counts = O.update_step(x, a_gpu, mu_prev, mus_prev, storage, w=wts)
        live = counts > 0
        gm = c.cmu[g0:g0 + D]
        absmean = np.zeros_like(mu)
        wsum = np.zeros(D)
        np.add.at(absmean, a_gpu, wts[:, None] * np.abs(x))
        np.add.at(wsum, a_gpu, wts)
        absmean[live] /= wsum[live, None]
        bound = gamma(counts[:, None] + 1) * absmean + U32 * np.abs(mu)
        assert np.all(np.abs(gm - mu)[live] <= bound[live] + 1e-30), f"unit {unit} block {blk.index}: coarse means"
        np.testing.assert_array_equal(c.ckbar[g0:g0 + D][live], O.round_storage(gm[live], storage))
        # empty coarse clusters keep their centroid
        np.testing.assert_array_equal(c.ckbar[g0:g0 + D][~live], mus_prev[~live])
        # sizes, member lists (non-empty fine ids by coarse id, then fine id) and offsets
        np.testing.assert_array_equal(c.csizes[g0:g0 + D], np.bincount(a_gpu, weights=wts, minlength=D).astype(np.int64))
        for g in range(D):
            mem = ids[a_gpu == g]
            assert c.coffsets[g0 + g] == pos, f"unit {unit} block {blk.index}: offset of coarse cluster {g}"
            want_members[pos:pos + len(mem)] = mem
            pos += len(mem)
        # value centroids: the size-weighted mean of the members' fine value
        # centroids, rounded once to storage (the fp32 sum's rounding bound)
        v = c.vbar[ids]
        v64 = np.zeros((D, v.shape[1]))
        vabs = np.zeros((D, v.shape[1]))
        np.add.at(v64, a_gpu, wts[:, None] * v)
        np.add.at(vabs, a_gpu, wts[:, None] * np.abs(v))
        v64[live] /= wsum[live, None]
        vabs[live] /= wsum[live, None]
        vb = gamma(counts[:, None] + 1) * vabs + U32 * np.abs(v64)
        lo, hi = _rne_bracket(v64 - vb, v64 + vb, storage)
        gv = c.cvbar[g0:g0 + D]
        assert np.all((gv[live] >= lo[live]) & (gv[live] <= hi[live])), f"unit {unit} block {blk.index}: coarse values"
        assert np.all(gv[~live] == 0)
    np.testing.assert_array_equal(c.cmembers[:pos], want_members[:pos])
    assert c.coffsets[c.n_coarse] == pos
    return n_diff
