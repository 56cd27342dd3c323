"""fp64 CPU oracle for the Multipole Attention decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It loads
``liboracle.so`` built from ``mpattn_oracle.c`` in this directory with gcc and
shares no code with the GPU library.  Inputs are widened exactly to float64
numpy arrays; every result is float64 (or int32 for ids).

Sources are the web pages on "Multipole Attention for Efficient Long Context
Reasoning" (arXiv 2506.13059); each function names the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mpattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

EXACT, F32, BF16 = 0, 1, 2

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_i32, _i64, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64


def build_library(out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load():
    path = os.environ.get("MPATTN_ORACLE_LIB")  # another build of the same source (a sanitizer build)
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_library()
    lib = ctypes.CDLL(path)
    sig = {
        "orc_round_storage": (ctypes.c_double, [ctypes.c_double, ctypes.c_int]),
        "orc_round_array": (None, [_D, _i64, ctypes.c_int, _D]),
        "orc_sm64_mix": (_u64, [_u64]),
        "orc_sm64_draw": (_u64, [_u64, _u64]),
        "orc_block_stream": (_u64, [_u64, _i64, _i64, ctypes.c_int]),
        "orc_init_indices": (ctypes.c_int, [_u64, _i32, _i32, _I]),
        "orc_assign": (ctypes.c_double, [_D, _i32, _i32, _D, _i32, _D, _I, _D]),
        "orc_update": (None, [_D, _i32, _i32, _I, _D, _i32, ctypes.c_int, _D, _D, _I]),
        "orc_kmeans": (None, [_D, _i32, _i32, _D, _i32, _i32, ctypes.c_int, _I, _D, _D, _I, _I, _D]),
        "orc_cluster_block": (ctypes.c_int, [_D, _D, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                             _u64, _D, _D, _D, _I, _I, _I, _I, _D]),
        "orc_coarse_block": (ctypes.c_int, [_D, _D, _I, _i32, _i32, _i32, _i32, _i32, _i32,
                                            ctypes.c_int, _u64, _i32, _D, _D, _D, _I, _I, _I, _I, _D]),
        "orc_select": (_i64, [_D, _I, _i32, _i64, _I]),
        "orc_scores": (None, [_D, _i32, _i32, _D, _i32, _D, _D]),
        "orc_combine": (None, [_D, _i32, _D, _D, _i32, _I, _D, _D, _I, _I, _i32, _D]),
        "orc_decode": (_i64, [_D, _i32, _i32, _D, _D, _i32, _i32, _D, _D, _I, _I, _i32, _i64,
                              ctypes.c_int, _D, _I, _D, _D]),
        "orc_decode_hier": (_i64, [_D, _i32, _i32, _D, _D, _i32, _i32, _D, _D, _I, _I, _I, _i32,
                                   _D, _D, _I, _i32, _i64, _i64, _I, _I, _D, _I, _I, _D, _D, _D]),
        "orc_dense": (None, [_D, _i32, _D, _D, _i32, _D]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _d(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _i(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_I)


def f64(x) -> np.ndarray:
    """Exact widening of any float array (numpy or torch, any float dtype)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------

def round_storage(x, storage: int) -> np.ndarray:
    x = f64(x)
    y = np.empty_like(x)
    _lib.orc_round_array(_d(x), x.size, storage, _d(y))
    return y


def sm64_mix(z: int) -> int:
    return int(_lib.orc_sm64_mix(z & (2**64 - 1)))


def sm64_draw(s0: int, t: int) -> int:
    return int(_lib.orc_sm64_draw(s0 & (2**64 - 1), t))


def block_stream(seed: int, unit: int, block: int, level: int = 0) -> int:
    return int(_lib.orc_block_stream(seed & (2**64 - 1), unit, block, level))


def init_indices(s0: int, n: int, count: int) -> np.ndarray:
    out = np.zeros(count, np.int32)
    rc = _lib.orc_init_indices(s0 & (2**64 - 1), n, count, _i(out))
    if rc != 0:
        raise ValueError("init_indices: count > n or n <= 0")
    return out


def assign_step(x, mu_s, w=None):
    """Nearest stored centroid for every point (ties -> lowest index).
    Returns (assign, best squared distance, objective)."""
    x, mu_s = f64(x), f64(mu_s)
    n, d = x.shape
    a = np.zeros(n, np.int32)
    bd = np.zeros(n)
    wp = _d(f64(w)) if w is not None else None
    J = _lib.orc_assign(_d(x), n, d, _d(mu_s), mu_s.shape[0], wp, _i(a), _d(bd))
    return a, bd, J


def update_step(x, assign, mu, mu_s, storage: int, w=None):
    """Lloyd update in place on copies; returns (mu, mu_s, counts)."""
    x = f64(x)
    mu, mu_s = f64(mu).copy(), f64(mu_s).copy()
    a = np.ascontiguousarray(assign, dtype=np.int32)
    counts = np.zeros(mu.shape[0], np.int32)
    wp = _d(f64(w)) if w is not None else None
    _lib.orc_update(_d(x), x.shape[0], x.shape[1], _i(a), wp, mu.shape[0], storage, _d(mu), _d(mu_s),
                    _i(counts))
    return mu, mu_s, counts


def kmeans(x, C: int, iters: int, storage: int, init_idx, w=None):
    """Returns (mu, mu_s, assign, counts, J[iters])."""
    x = f64(x)
    n, d = x.shape
    mu = np.zeros((C, d))
    mu_s = np.zeros((C, d))
    a = np.zeros(n, np.int32)
    counts = np.zeros(C, np.int32)
    J = np.zeros(max(iters, 1))
    idx = np.ascontiguousarray(init_idx, dtype=np.int32)
    wp = _d(f64(w)) if w is not None else None
    _lib.orc_kmeans(_d(x), n, d, wp, C, iters, storage, _i(idx), _d(mu), _d(mu_s), _i(a), _i(counts), _d(J))
    return mu, mu_s, a, counts, J[:iters]


def select(key, sizes, budget: int):
    key = f64(key)
    sizes = np.ascontiguousarray(sizes, dtype=np.int32)
    sel = np.zeros(key.shape[0], np.int32)
    taken = _lib.orc_select(_d(key), _i(sizes), key.shape[0], budget, _i(sel))
    return sel, int(taken)


def scores(q, kbar):
    q, kbar = f64(q), f64(kbar)
    G, d = q.shape
    C = kbar.shape[0]
    s = np.zeros((G, C))
    r = np.zeros(C)
    _lib.orc_scores(_d(q), G, d, _d(kbar), C, _d(s), _d(r))
    return s, r


def dense(q, K, V) -> np.ndarray:
    """Textbook softmax attention for each row of q over (K, V)."""
    q, K, V = f64(q), f64(K), f64(V)
    q2 = q.reshape(-1, q.shape[-1])
    out = np.zeros_like(q2)
    for g in range(q2.shape[0]):
        qg = np.ascontiguousarray(q2[g])
        og = np.zeros(q2.shape[1])
        _lib.orc_dense(_d(qg), q2.shape[1], _d(K), _d(V), K.shape[0], _d(og))
        out[g] = og
    return out.reshape(q.shape)


# ----------------------------------------------------------------------------
# per-unit state: one sequence, one KV head
# ----------------------------------------------------------------------------

@dataclass
class Block:
    p: int      # first token
    L: int      # tokens
    c0: int     # first global cluster id
    C: int      # clusters
    index: int  # block index used to seed it


@dataclass
class UnitState:
    d: int
    capacity_tokens: int
    capacity_clusters: int
    storage: int
    mu: np.ndarray
    kbar: np.ndarray
    vbar: np.ndarray
    sizes: np.ndarray
    offsets: np.ndarray
    token_ids: np.ndarray
    assign: np.ndarray
    n_clustered: int = 0
    n_clusters: int = 0
    blocks: List[Block] = field(default_factory=list)
    J: List[np.ndarray] = field(default_factory=list)
    # hierarchy (coarse level), filled by build_coarse
    cmu: Optional[np.ndarray] = None
    ckbar: Optional[np.ndarray] = None
    cvbar: Optional[np.ndarray] = None
    csizes: Optional[np.ndarray] = None
    parent: Optional[np.ndarray] = None
    coffsets: Optional[np.ndarray] = None
    cmembers: Optional[np.ndarray] = None
    n_coarse: int = 0
    cJ: List[np.ndarray] = field(default_factory=list)


def clusters_for(L: int, tokens_per_centroid: int) -> int:
    """Clusters of a block of L tokens: ceil(L / tokens_per_centroid)."""
    return -(-L // tokens_per_centroid)


def empty_state(d: int, capacity_tokens: int, capacity_clusters: int, storage: int) -> UnitState:
    return UnitState(
        d=d, capacity_tokens=capacity_tokens, capacity_clusters=capacity_clusters, storage=storage,
        mu=np.zeros((capacity_clusters, d)), kbar=np.zeros((capacity_clusters, d)),
        vbar=np.zeros((capacity_clusters, d)), sizes=np.zeros(capacity_clusters, np.int32),
        offsets=np.zeros(capacity_clusters + 1, np.int32), token_ids=np.zeros(capacity_tokens, np.int32),
        assign=np.zeros(capacity_tokens, np.int32))


def cluster_block(st: UnitState, K, V, p: int, L: int, iters: int, tokens_per_centroid: int,
                  seed: int, unit: int, block_index: int) -> None:
    """Cluster tokens [p, p+L) of one unit and append the block's clusters."""
    C = clusters_for(L, tokens_per_centroid)
    if st.n_clusters + C > st.capacity_clusters:
        raise ValueError("cluster capacity exceeded")
    c0 = st.n_clusters
    J = np.zeros(max(iters, 1))
    s0 = block_stream(seed, unit, block_index, 0)
    rc = _lib.orc_cluster_block(_d(K), _d(V), st.d, p, L, c0, C, iters, st.storage, s0, _d(st.mu),
                                _d(st.kbar), _d(st.vbar), _i(st.sizes), _i(st.offsets), _i(st.token_ids),
                                _i(st.assign), _d(J))
    if rc != 0:
        raise RuntimeError(f"orc_cluster_block failed ({rc})")
    st.blocks.append(Block(p, L, c0, C, block_index))
    st.J.append(J[:iters])
    st.n_clusters += C
    st.n_clustered = p + L


def build_unit(K, V, n_tokens: int, *, tokens_per_centroid: int = 16, cluster_block_size: int = 8192,
               iters: int = 10, storage: int = BF16, seed: int = 0, unit: int = 0,
               capacity_tokens: Optional[int] = None, capacity_clusters: Optional[int] = None) -> UnitState:
    """Blockwise clustering of tokens [0, n_tokens) ([APP] "blockwise"): blocks
    of cluster_block_size tokens, the last one possibly shorter."""
    K, V = f64(K), f64(V)
    d = K.shape[1]
    cap_t = capacity_tokens or K.shape[0]
    if capacity_clusters is None:
        capacity_clusters = sum(clusters_for(min(cluster_block_size, cap_t - p), tokens_per_centroid)
                                for p in range(0, cap_t, cluster_block_size))
    st = empty_state(d, cap_t, capacity_clusters, storage)
    p, j = 0, 0
    while p < n_tokens:
        L = min(cluster_block_size, n_tokens - p)
        cluster_block(st, K, V, p, L, iters, tokens_per_centroid, seed, unit, j)
        p += L
        j += 1
    return st


def update_unit(st: UnitState, K, V, n_total: int, *, tokens_per_centroid: int = 16,
                cluster_block_size: int = 8192, iters: int = 5, seed: int = 0, unit: int = 0) -> int:
    """Online update ([ABS] fast cluster update; [APP] blockwise sliding-window
    update).  Reading: tokens past n_clustered form an unclustered tail; each
    time it holds a full block, that block is clustered on its own and its
    clusters are appended.  Returns the number of blocks added."""
    K, V = f64(K), f64(V)
    added = 0
    while n_total - st.n_clustered >= cluster_block_size:
        cluster_block(st, K, V, st.n_clustered, cluster_block_size, iters, tokens_per_centroid, seed, unit,
                      len(st.blocks))
        added += 1
    return added


def build_coarse(st: UnitState, *, coarse_tokens_per_centroid: int = 128, iters: int = 10, seed: int = 0,
                 unit: int = 0, capacity_coarse: Optional[int] = None) -> None:
    """Coarse level of the hierarchy, block by block (reading: size-weighted
    k-means over each block's non-empty fine key centroids)."""
    cap = capacity_coarse or sum(clusters_for(b.L, coarse_tokens_per_centroid) for b in st.blocks)
    d = st.d
    st.cmu, st.ckbar, st.cvbar = np.zeros((cap, d)), np.zeros((cap, d)), np.zeros((cap, d))
    st.csizes = np.zeros(cap, np.int32)
    st.parent = np.full(st.capacity_clusters, -1, np.int32)
    st.coffsets = np.zeros(cap + 1, np.int32)
    st.cmembers = np.zeros(st.capacity_clusters, np.int32)
    st.cJ = []
    g0, pos = 0, 0
    for b in st.blocks:
        D = clusters_for(b.L, coarse_tokens_per_centroid)
        J = np.zeros(max(iters, 1))
        s0 = block_stream(seed, unit, b.index, 1)
        # the blocks' member lists follow each other (non-empty fine ids only)
        n = _lib.orc_coarse_block(_d(st.kbar), _d(st.vbar), _i(st.sizes), d, b.c0, b.C, g0, D, iters,
                                  st.storage, s0, pos, _d(st.cmu), _d(st.ckbar), _d(st.cvbar),
                                  _i(st.csizes), _i(st.parent), _i(st.coffsets), _i(st.cmembers), _d(J))
        if n < 0:
            raise RuntimeError("orc_coarse_block failed (fewer non-empty fine clusters than coarse ones?)")
        g0 += D
        pos += n
        st.cJ.append(J[:iters])
    st.n_coarse = g0


@dataclass
class DecodeResult:
    out: np.ndarray        # [G][d]
    selected: np.ndarray   # [C] 0/1
    s: np.ndarray          # [G][C]
    r: np.ndarray          # [C]
    taken: int             # tokens selected
    candidates: Optional[np.ndarray] = None  # [D] 0/1 (hierarchy)
    cs: Optional[np.ndarray] = None          # [G][D]


def decode_unit(q, K, V, n_total: int, st: UnitState, budget: int, mode: int = 0) -> DecodeResult:
    """One decode step for one unit (mode 0 multipole, mode 1 omit unselected)."""
    q, K, V = f64(q), f64(K), f64(V)
    G, d = q.shape
    C = st.n_clusters
    out = np.zeros((G, d))
    sel = np.zeros(max(C, 1), np.int32)
    s = np.zeros((G, max(C, 1)))
    r = np.zeros(max(C, 1))
    kbar = np.ascontiguousarray(st.kbar[:max(C, 1)])
    vbar = np.ascontiguousarray(st.vbar[:max(C, 1)])
    taken = _lib.orc_decode(_d(q), G, d, _d(K), _d(V), n_total, st.n_clustered, _d(kbar), _d(vbar),
                            _i(st.sizes), _i(st.assign), C, budget, mode, _d(out), _i(sel), _d(s), _d(r))
    return DecodeResult(out, sel[:C], s[:, :C], r[:C], int(taken))


def decode_unit_hier(q, K, V, n_total: int, st: UnitState, budget: int, cand_budget: int,
                     candidates=None, selected=None) -> DecodeResult:
    """Two-level decode step; `candidates` / `selected` (0/1 arrays) force the
    coarse candidate set and the fine selection instead of computing them."""
    q, K, V = f64(q), f64(K), f64(V)
    G, d = q.shape
    C, D = st.n_clusters, st.n_coarse
    out = np.zeros((G, d))
    sel = np.zeros(C, np.int32)
    csel = np.zeros(D, np.int32)
    s = np.zeros((G, C))
    cs = np.zeros((G, D))
    r = np.zeros(C)
    fc = _i(np.ascontiguousarray(candidates, dtype=np.int32)) if candidates is not None else None
    fs = _i(np.ascontiguousarray(selected, dtype=np.int32)) if selected is not None else None
    taken = _lib.orc_decode_hier(_d(q), G, d, _d(K), _d(V), n_total, st.n_clustered,
                                 _d(np.ascontiguousarray(st.kbar[:C])), _d(np.ascontiguousarray(st.vbar[:C])),
                                 _i(st.sizes), _i(st.assign), _i(st.parent), C,
                                 _d(np.ascontiguousarray(st.ckbar[:D])), _d(np.ascontiguousarray(st.cvbar[:D])),
                                 _i(st.csizes), D, cand_budget, budget, fc, fs, _d(out), _i(csel), _i(sel), _d(s),
                                 _d(cs), _d(r))
    return DecodeResult(out, sel, s, r, int(taken), csel, cs)


def decode_with_selection(q, K, V, n_total: int, st: UnitState, selected, mode: int = 0) -> np.ndarray:
    """The combine of one decode step for a given selection (1 = exact) of
    the flat clusters; used to compare outputs when two correct selections
    differ only among near-equal scores."""
    q, K, V = f64(q), f64(K), f64(V)
    G, d = q.shape
    C = st.n_clusters
    sel = np.ascontiguousarray(selected, dtype=np.int32)
    s = np.zeros((G, C))
    r = np.zeros(C)
    kbar = np.ascontiguousarray(st.kbar[:C])
    vbar = np.ascontiguousarray(st.vbar[:C])
    _lib.orc_scores(_d(q), G, d, _d(kbar), C, _d(s), _d(r))
    exact = np.array([1 if i >= st.n_clustered else sel[st.assign[i]] for i in range(n_total)], np.int32)
    sizes = np.ascontiguousarray(st.sizes[:C])
    pseudo = ((mode == 0) & (sizes > 0) & (sel == 0)).astype(np.int32)
    out = np.zeros((G, d))
    for g in range(G):
        og = np.zeros(d)
        sg = np.ascontiguousarray(s[g])
        _lib.orc_combine(_d(np.ascontiguousarray(q[g])), d, _d(K), _d(V), n_total, _i(exact), _d(sg), _d(vbar),
                         _i(sizes), _i(pseudo), C, _d(og))
        out[g] = og
    return out


def parallel_map(fn, items, threads: Optional[int] = None):
    """Runs independent per-unit oracle calls on host threads (ctypes drops
    the GIL inside the C calls).  Returns results in input order."""
    items = list(items)
    threads = threads or min(len(items), os.cpu_count() or 1) or 1
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
