"""Python binding of libmpattn.so (the C ABI in include/mpattn.h).

Argument marshalling only: every step of clustering and decoding runs in the
library's HIP kernels.  torch provides device memory (state arrays,
workspaces, outputs) and the current HIP stream.  Loading fails loudly when
the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import copy
import ctypes
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# another build of the same sources may be named (a host-sanitizer build)
LIB_PATH = os.environ.get("MPATTN_LIB") or os.path.join(_HERE, "libmpattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_CAPACITY, ERR_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
OP_BUILD, OP_UPDATE, OP_DECODE, OP_DENSE = 0, 1, 2, 3
MODE_MULTIPOLE, MODE_OMIT, MODE_PER_HEAD = 0, 1, 2
CENTROIDS_STORED, CENTROIDS_FP8 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class MpattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class CParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "dtype", "capacity_tokens", "tokens_per_centroid",
        "cluster_block", "build_iters", "update_iters", "coarse_tokens_per_centroid", "coarse_iters",
        "coarse_candidate_tokens", "splits", "centroid_format")] + [("seed", ctypes.c_uint64)]


_VP = ctypes.c_void_p


class CState(ctypes.Structure):
    _fields_ = [(n, _VP) for n in (
        "key_centroids", "value_centroids", "key_centroids_f32", "sizes", "offsets", "token_ids", "assign",
        "sorted_keys", "sorted_values", "coarse_key_centroids", "coarse_value_centroids",
        "coarse_key_centroids_f32", "coarse_sizes", "coarse_offsets", "coarse_members", "parent",
        "key_codes", "key_scales", "value_codes", "value_scales")] + [
        (n, ctypes.c_int32) for n in (
            "capacity_clusters", "capacity_coarse", "n_clustered", "n_clusters", "n_coarse", "n_blocks")]


class CDebug(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("scores", "selected", "candidates", "exact_tokens")] + [("rescore", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, D = ctypes.POINTER(CParams), ctypes.POINTER(CState), ctypes.POINTER(CDebug)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    lib.mpattn_status_string.restype = ctypes.c_char_p
    lib.mpattn_status_string.argtypes = [ctypes.c_int]
    lib.mpattn_max_clusters.restype = i32
    lib.mpattn_max_clusters.argtypes = [P]
    lib.mpattn_max_coarse.restype = i32
    lib.mpattn_max_coarse.argtypes = [P]
    lib.mpattn_workspace_bytes.restype = sz
    lib.mpattn_workspace_bytes.argtypes = [P, i32, i32, i32]
    lib.mpattn_build_clusters.restype = ctypes.c_int
    lib.mpattn_build_clusters.argtypes = [P, _VP, _VP, i32, S, _VP, sz, _VP]
    lib.mpattn_update_window.restype = ctypes.c_int
    lib.mpattn_update_window.argtypes = [P, _VP, _VP, i32, S, _VP, sz, _VP]
    lib.mpattn_decode.restype = ctypes.c_int
    lib.mpattn_decode.argtypes = [P, _VP, _VP, _VP, i32, S, i32, i32, _VP, _VP, sz, _VP]
    lib.mpattn_decode_ex.restype = ctypes.c_int
    lib.mpattn_decode_ex.argtypes = [P, _VP, _VP, _VP, i32, S, i32, i32, _VP, _VP, sz, _VP, D, i32, i32]
    lib.mpattn_decode_stage_count.restype = i32
    lib.mpattn_decode_stage_count.argtypes = [P]
    lib.mpattn_decode_stage_name.restype = ctypes.c_char_p
    lib.mpattn_decode_stage_name.argtypes = [P, i32]
    lib.mpattn_dense_decode.restype = ctypes.c_int
    lib.mpattn_dense_decode.argtypes = [P, _VP, _VP, _VP, i32, _VP, _VP, sz, _VP]
    lib.mpattn_read_probe.restype = ctypes.c_int
    lib.mpattn_read_probe.argtypes = [_VP, sz, _VP, _VP]
    lib.mpattn_decode_noalloc.restype = ctypes.c_int
    lib.mpattn_decode_noalloc.argtypes = [P, _VP, _VP, _VP, i32, S, i32, i32, _VP, _VP]
    lib.mpattn_decode_noalloc_max_bytes.restype = sz
    lib.mpattn_decode_noalloc_max_bytes.argtypes = []
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.mpattn_status_string(status).decode()


@dataclass
class Params:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    capacity_tokens: int
    head_dim: int = 128
    dtype: torch.dtype = torch.bfloat16
    tokens_per_centroid: int = 16
    cluster_block: int = 8192
    build_iters: int = 10
    update_iters: int = 5
    coarse_tokens_per_centroid: int = 0
    coarse_iters: int = 10
    coarse_candidate_tokens: int = 0
    splits: int = 0
    seed: int = 0
    centroid_format: int = CENTROIDS_STORED  # CENTROIDS_FP8: the decode reads fp8 copies

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def hierarchical(self) -> bool:
        return self.coarse_tokens_per_centroid > 0

    def c(self) -> CParams:
        return CParams(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, _DTYPES[self.dtype],
                       self.capacity_tokens, self.tokens_per_centroid, self.cluster_block, self.build_iters,
                       self.update_iters, self.coarse_tokens_per_centroid, self.coarse_iters,
                       self.coarse_candidate_tokens, self.splits, self.centroid_format, self.seed & (2**64 - 1))

    def max_clusters(self) -> int:
        return int(lib.mpattn_max_clusters(ctypes.byref(self.c())))

    def max_coarse(self) -> int:
        return int(lib.mpattn_max_coarse(ctypes.byref(self.c())))

    def decode_stages(self) -> list:
        cp = self.c()
        return [lib.mpattn_decode_stage_name(ctypes.byref(cp), i).decode()
                for i in range(lib.mpattn_decode_stage_count(ctypes.byref(cp)))]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class ClusterState:
    """Device arrays of the cluster state (allocated through torch) and the
    host counters the library maintains."""

    def __init__(self, params: Params, device="cuda", sorted_copy: bool = True,
                 capacity_clusters: Optional[int] = None, capacity_coarse: Optional[int] = None):
        p = params
        U, N, d = p.units, p.capacity_tokens, p.head_dim
        C = capacity_clusters or p.max_clusters()
        if C <= 0:
            raise ValueError("invalid parameters")
        self.params = p
        self.capacity_clusters = C
        dt = p.dtype
        kw = dict(device=device)
        self.key_centroids = torch.zeros(p.batch, p.n_kv_heads, C, d, dtype=dt, **kw)
        self.value_centroids = torch.zeros(p.batch, p.n_kv_heads, C, d, dtype=dt, **kw)
        self.key_centroids_f32 = torch.zeros(p.batch, p.n_kv_heads, C, d, dtype=torch.float32, **kw)
        self.sizes = torch.zeros(p.batch, p.n_kv_heads, C, dtype=torch.int32, **kw)
        self.offsets = torch.zeros(p.batch, p.n_kv_heads, C + 1, dtype=torch.int32, **kw)
        self.token_ids = torch.zeros(p.batch, p.n_kv_heads, N, dtype=torch.int32, **kw)
        self.assign = torch.zeros(p.batch, p.n_kv_heads, N, dtype=torch.int32, **kw)
        self.sorted_keys = torch.zeros(p.batch, p.n_kv_heads, N, d, dtype=dt, **kw) if sorted_copy else None
        self.sorted_values = torch.zeros(p.batch, p.n_kv_heads, N, d, dtype=dt, **kw) if sorted_copy else None
        self.key_codes = self.key_scales = self.value_codes = self.value_scales = None
        if p.centroid_format == CENTROIDS_FP8:
            self.key_codes = torch.zeros(p.batch, p.n_kv_heads, C, d, dtype=torch.uint8, **kw)
            self.value_codes = torch.zeros(p.batch, p.n_kv_heads, C, d, dtype=torch.uint8, **kw)
            self.key_scales = torch.zeros(p.batch, p.n_kv_heads, C, d // 32, dtype=torch.uint8, **kw)
            self.value_scales = torch.zeros(p.batch, p.n_kv_heads, C, d // 32, dtype=torch.uint8, **kw)
        self.capacity_coarse = 0
        self.coarse_key_centroids = self.coarse_value_centroids = self.coarse_key_centroids_f32 = None
        self.coarse_sizes = self.coarse_offsets = self.coarse_members = self.parent = None
        if p.hierarchical:
            Dc = capacity_coarse or p.max_coarse()
            self.capacity_coarse = Dc
            self.coarse_key_centroids = torch.zeros(p.batch, p.n_kv_heads, Dc, d, dtype=dt, **kw)
            self.coarse_value_centroids = torch.zeros(p.batch, p.n_kv_heads, Dc, d, dtype=dt, **kw)
            self.coarse_key_centroids_f32 = torch.zeros(p.batch, p.n_kv_heads, Dc, d, dtype=torch.float32, **kw)
            self.coarse_sizes = torch.zeros(p.batch, p.n_kv_heads, Dc, dtype=torch.int32, **kw)
            self.coarse_offsets = torch.zeros(p.batch, p.n_kv_heads, Dc + 1, dtype=torch.int32, **kw)
            self.coarse_members = torch.zeros(p.batch, p.n_kv_heads, C, dtype=torch.int32, **kw)
            self.parent = torch.full((p.batch, p.n_kv_heads, C), -1, dtype=torch.int32, **kw)
        self.n_clustered = 0
        self.n_clusters = 0
        self.n_coarse = 0
        self.n_blocks = 0

    def c(self) -> CState:
        return CState(_ptr(self.key_centroids), _ptr(self.value_centroids), _ptr(self.key_centroids_f32),
                      _ptr(self.sizes), _ptr(self.offsets), _ptr(self.token_ids), _ptr(self.assign),
                      _ptr(self.sorted_keys), _ptr(self.sorted_values), _ptr(self.coarse_key_centroids),
                      _ptr(self.coarse_value_centroids), _ptr(self.coarse_key_centroids_f32),
                      _ptr(self.coarse_sizes), _ptr(self.coarse_offsets), _ptr(self.coarse_members),
                      _ptr(self.parent), _ptr(self.key_codes), _ptr(self.key_scales), _ptr(self.value_codes),
                      _ptr(self.value_scales), self.capacity_clusters, self.capacity_coarse, self.n_clustered,
                      self.n_clusters, self.n_coarse, self.n_blocks)

    def _take(self, cs: CState) -> None:
        self.n_clustered, self.n_clusters = cs.n_clustered, cs.n_clusters
        self.n_coarse, self.n_blocks = cs.n_coarse, cs.n_blocks


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_cache(p: Params, k: torch.Tensor, v: torch.Tensor) -> None:
    shape = (p.batch, p.n_kv_heads, p.capacity_tokens, p.head_dim)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != shape or t.dtype != p.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {p.dtype} CUDA tensor of shape {shape}, got "
                             f"{tuple(t.shape)} {t.dtype}")


def _raise(status: int, what: str) -> None:
    if status != OK:
        raise MpattnError(status, what)


def build_clusters(p: Params, k: torch.Tensor, v: torch.Tensor, n_tokens: int, state: ClusterState) -> None:
    """Clusters tokens [0, n_tokens) of every (sequence, KV head)."""
    _check_cache(p, k, v)
    cp, cs = p.c(), state.c()
    st = lib.mpattn_build_clusters(ctypes.byref(cp), _ptr(k), _ptr(v), n_tokens, ctypes.byref(cs), None, 0,
                                   _stream(k.device))
    _raise(st, "mpattn_build_clusters")
    state._take(cs)


def update_window(p: Params, k: torch.Tensor, v: torch.Tensor, n_tokens_total: int, state: ClusterState) -> int:
    """Clusters every full block of the unclustered tail; returns blocks added."""
    _check_cache(p, k, v)
    cp, cs = p.c(), state.c()
    before = state.n_blocks
    st = lib.mpattn_update_window(ctypes.byref(cp), _ptr(k), _ptr(v), n_tokens_total, ctypes.byref(cs), None, 0,
                                  _stream(k.device))
    _raise(st, "mpattn_update_window")
    state._take(cs)
    return state.n_blocks - before


def update_window_concurrent(p: Params, k: torch.Tensor, v: torch.Tensor, n_tokens_total: int, state: ClusterState,
                             stream: torch.cuda.Stream) -> Tuple[ClusterState, torch.cuda.Event, int]:
    """Enqueues mpattn_update_window on `stream` and returns (view, event,
    blocks added).  `view` is the state as it was before the update: the same
    device arrays with the old host counters.  Decodes on other streams may go
    on using it while the update runs, because the update writes only past the
    old clusters (new centroids and their fp8 copies, sizes, member lists,
    sorted rows) and
    rewrites the old clusters' end offset with its own value.  Once `event`
    has completed (e.g. after stream.wait_event(event) on the decode stream),
    `state` holds the new clusters.  Flat method only."""
    if p.hierarchical:
        raise ValueError("concurrent window update: flat method only")
    view = copy.copy(state)
    with torch.cuda.stream(stream):
        added = update_window(p, k, v, n_tokens_total, state)
        event = torch.cuda.Event()
        event.record(stream)
    return view, event, added


class Workspace:
    """A reusable device workspace sized by mpattn_workspace_bytes, one per
    (device, stream, workspace layout): a decode workspace keeps per-unit
    call tags, so a buffer that served another layout is zeroed again."""

    def __init__(self):
        self._buf: Dict[tuple, torch.Tensor] = {}

    def get(self, p: Params, state: ClusterState, device, stream: Optional[int] = None) -> torch.Tensor:
        cp = p.c()
        n = lib.mpattn_workspace_bytes(ctypes.byref(cp), state.capacity_clusters, state.capacity_coarse, OP_DECODE)
        if n == ctypes.c_size_t(-1).value:
            raise MpattnError(ERR_INVALID_ARG, "mpattn_workspace_bytes")
        if stream is None:
            stream = torch.cuda.current_stream(device).cuda_stream
        layout = (p.batch, p.n_q_heads, p.n_kv_heads, p.capacity_tokens, p.tokens_per_centroid, p.cluster_block,
                  p.coarse_tokens_per_centroid, p.coarse_candidate_tokens, p.splits, _DTYPES[p.dtype],
                  state.capacity_clusters, state.capacity_coarse, n)
        key = (str(device), int(stream), layout)
        buf = self._buf.get(key)
        if buf is None:
            buf = torch.zeros(max(n, 1), dtype=torch.uint8, device=device)  # tags and counters start at zero
            self._buf[key] = buf
        return buf


def decode_status(workspace: torch.Tensor) -> Tuple[int, int]:
    """The two counters at the start of a decode workspace (see
    mpattn_workspace_bytes): (key-exchange fallbacks, output values poisoned
    because a partial sum did not arrive in time).  Synchronises."""
    v = workspace[:8].view(torch.int32).cpu()
    return int(v[0]), int(v[1])


_default_ws = Workspace()


@dataclass
class DecodeDebug:
    # per-head selection: Hq in place of Hkv and 1 in place of G
    scores: Optional[torch.Tensor] = None        # [B][Hkv][n_clusters][G] float32
    selected: Optional[torch.Tensor] = None      # [B][Hkv][n_clusters] int32
    candidates: Optional[torch.Tensor] = None    # [B][Hkv][n_coarse] int32
    exact_tokens: Optional[torch.Tensor] = None  # [B][Hkv] int32
    rescore: int = 0                             # 1: every workgroup scores all clusters; 2: late-partner path

    @staticmethod
    def allocate(p: Params, state: ClusterState, device="cuda", per_head: bool = False) -> "DecodeDebug":
        B, C = p.batch, state.n_clusters
        H, G = (p.n_q_heads, 1) if per_head else (p.n_kv_heads, p.group)
        return DecodeDebug(
            scores=torch.zeros(B, H, C, G, dtype=torch.float32, device=device),
            selected=torch.zeros(B, H, C, dtype=torch.int32, device=device),
            candidates=torch.zeros(B, H, max(state.n_coarse, 1), dtype=torch.int32, device=device)
            if p.hierarchical else None,
            exact_tokens=torch.zeros(B, H, dtype=torch.int32, device=device))

    def c(self) -> CDebug:
        return CDebug(_ptr(self.scores), _ptr(self.selected), _ptr(self.candidates), _ptr(self.exact_tokens),
                      int(self.rescore))


def decode(p: Params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_tokens_total: int,
           state: ClusterState, token_budget: int, mode: int = MODE_MULTIPOLE, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, debug: Optional[DecodeDebug] = None,
           stages: Optional[Sequence[int]] = None) -> torch.Tensor:
    """One decode step for every sequence; returns out [B][Hq][d] float32.
    `stages` = (first, last) enqueues only that stage range."""
    _check_cache(p, k, v)
    qshape = (p.batch, p.n_q_heads, p.head_dim)
    if tuple(q.shape) != qshape or q.dtype != p.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {p.dtype} CUDA tensor of shape {qshape}")
    if out is None:
        out = torch.empty(qshape, dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != qshape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of shape [B][Hq][d]")
    if workspace is None:
        workspace = _default_ws.get(p, state, q.device)
    cp, cs = p.c(), state.c()
    if debug is not None:
        units = p.batch * (p.n_q_heads if mode == MODE_PER_HEAD else p.n_kv_heads)
        per_unit = {"scores": state.n_clusters * p.n_q_heads * p.batch // units, "selected": state.n_clusters,
                    "candidates": state.n_coarse, "exact_tokens": 1}
        for name, n in per_unit.items():
            t = getattr(debug, name)
            if t is not None and (not t.is_contiguous() or t.numel() * t.element_size() < units * n * 4):
                raise ValueError(f"debug.{name} must be contiguous and hold {units} x {n} 32-bit values")
    dbg = debug.c() if debug is not None else None
    if stages is None:
        first, last = 0, lib.mpattn_decode_stage_count(ctypes.byref(cp)) - 1
    else:
        first, last = stages
    st = lib.mpattn_decode_ex(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), n_tokens_total, ctypes.byref(cs),
                              token_budget, mode, _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream(q.device), ctypes.byref(dbg) if dbg is not None else None, first, last)
    _raise(st, "mpattn_decode")
    return out


def decode_noalloc(p: Params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_tokens_total: int,
                   state: ClusterState, token_budget: int, out: torch.Tensor, mode: int = MODE_MULTIPOLE) -> torch.Tensor:
    """mpattn_decode_noalloc: the decode with the library's own device
    workspace; `out` [B][Hq][d] float32 must be given (nothing is allocated)."""
    _check_cache(p, k, v)
    qshape = (p.batch, p.n_q_heads, p.head_dim)
    if tuple(q.shape) != qshape or q.dtype != p.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {p.dtype} CUDA tensor of shape {qshape}")
    if tuple(out.shape) != qshape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of shape [B][Hq][d]")
    cp, cs = p.c(), state.c()
    st = lib.mpattn_decode_noalloc(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), n_tokens_total, ctypes.byref(cs),
                                   token_budget, mode, _ptr(out), _stream(q.device))
    _raise(st, "mpattn_decode_noalloc")
    return out


def dense_decode(p: Params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_tokens: int,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense decode over tokens [0, n_tokens) (see mpattn_dense_decode);
    returns out [B][Hq][d] float32."""
    _check_cache(p, k, v)
    qshape = (p.batch, p.n_q_heads, p.head_dim)
    if tuple(q.shape) != qshape or q.dtype != p.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {p.dtype} CUDA tensor of shape {qshape}")
    if out is None:
        out = torch.empty(qshape, dtype=torch.float32, device=q.device)
    cp = p.c()
    if workspace is None:
        n = int(lib.mpattn_workspace_bytes(ctypes.byref(cp), 1, 0, OP_DENSE))
        if n == (1 << 64) - 1:
            raise MpattnError(ERR_INVALID_ARG, "mpattn_workspace_bytes")
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    st = lib.mpattn_dense_decode(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), n_tokens, _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(q.device))
    _raise(st, "mpattn_dense_decode")
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Enqueues one streaming read of `buf` (see mpattn_read_probe)."""
    _raise(lib.mpattn_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(buf.device)), "mpattn_read_probe")


def workspace_bytes(p: Params, state: ClusterState) -> int:
    cp = p.c()
    return int(lib.mpattn_workspace_bytes(ctypes.byref(cp), state.capacity_clusters, state.capacity_coarse,
                                          OP_DECODE))
