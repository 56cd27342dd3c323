"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, its struct layouts match the header as a C compiler sees it, and
every validation error is returned before anything touches a GPU (all pointers
below are fake and never dereferenced)."""
import ctypes
import dataclasses
import os
import re
import subprocess
import tempfile

import pytest
import torch

from sparse_long_context_means_amd import mpattn as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpattn.h")


def test_exports_every_declared_function():
    text = open(HEADER).read()
    names = set(re.findall(r"\b(mpattn_[a-z_0-9]+)\s*\(", text))
    assert {"mpattn_build_clusters", "mpattn_update_window", "mpattn_decode"} <= names
    for n in sorted(names):
        assert hasattr(M.lib, n), n


def test_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "mpattn.h"
#define P(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("params %zu state %zu debug %zu\n", sizeof(mpattn_params), sizeof(mpattn_state), sizeof(mpattn_decode_debug));
  P(mpattn_params, seed) P(mpattn_params, splits) P(mpattn_state, parent) P(mpattn_state, capacity_clusters)
  P(mpattn_state, n_blocks) P(mpattn_decode_debug, exact_tokens) P(mpattn_params, centroid_format)
  P(mpattn_state, key_codes) P(mpattn_state, value_scales)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = dict(zip(out[0].split()[0::2], map(int, out[0].split()[1::2])))
    assert sizes["params"] == ctypes.sizeof(M.CParams)
    assert sizes["state"] == ctypes.sizeof(M.CState)
    assert sizes["debug"] == ctypes.sizeof(M.CDebug)
    offs = dict(line.split() for line in out[1:] if line)
    assert int(offs["mpattn_params.seed"]) == M.CParams.seed.offset
    assert int(offs["mpattn_params.splits"]) == M.CParams.splits.offset
    assert int(offs["mpattn_state.parent"]) == M.CState.parent.offset
    assert int(offs["mpattn_state.capacity_clusters"]) == M.CState.capacity_clusters.offset
    assert int(offs["mpattn_state.n_blocks"]) == M.CState.n_blocks.offset
    assert int(offs["mpattn_decode_debug.exact_tokens"]) == M.CDebug.exact_tokens.offset
    assert int(offs["mpattn_params.centroid_format"]) == M.CParams.centroid_format.offset
    assert int(offs["mpattn_state.key_codes"]) == M.CState.key_codes.offset
    assert int(offs["mpattn_state.value_scales"]) == M.CState.value_scales.offset


def test_status_strings():
    for s in (M.OK, M.ERR_INVALID_ARG, M.ERR_UNSUPPORTED, M.ERR_WORKSPACE, M.ERR_CAPACITY, M.ERR_HIP):
        assert M.status_string(s) and M.status_string(s) != "unknown status"
    assert M.status_string(42) == "unknown status"


def _params(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, capacity_tokens=32768)
    base.update(kw)
    return M.Params(**base)


def test_capacity_bounds():
    p = _params()
    assert p.max_clusters() == 2048 + 4 + 1
    assert p.max_coarse() == 0
    ph = _params(capacity_tokens=131072, coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096)
    assert ph.max_coarse() == 1024 + 16 + 1
    assert _params(head_dim=64).max_clusters() == 0


def _fake_state(p, C=None, **over):
    C = C or p.max_clusters()
    fake = ctypes.c_void_p(0x10000)
    s = M.CState(*([fake] * 7 + [None, None] + [None] * 7 + [None] * 4), C, 0, 0, 0, 0, 0)
    if p.hierarchical:
        for f in ("coarse_key_centroids", "coarse_value_centroids", "coarse_key_centroids_f32", "coarse_sizes",
                  "coarse_offsets", "coarse_members", "parent"):
            setattr(s, f, fake)
        s.capacity_coarse = p.max_coarse()
    for k, v in over.items():
        setattr(s, k, v)
    return s


FAKE = ctypes.c_void_p(0x20000)


def _build(p, n, st):
    cp = p.c()
    return M.lib.mpattn_build_clusters(ctypes.byref(cp), FAKE, FAKE, n, ctypes.byref(st), None, 0, None)


def _decode(p, st, n_total, budget=128, mode=0, ws=1 << 40, first=0, last=None, q=FAKE):
    cp = p.c()
    last = M.lib.mpattn_decode_stage_count(ctypes.byref(cp)) - 1 if last is None else last
    return M.lib.mpattn_decode_ex(ctypes.byref(cp), q, FAKE, FAKE, n_total, ctypes.byref(st), budget, mode, FAKE,
                                  FAKE, ws, None, None, first, last)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), M.ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=2), M.ERR_UNSUPPORTED),    # G = 3
    (dict(n_q_heads=32, n_kv_heads=2), M.ERR_UNSUPPORTED),   # G = 16
    (dict(n_q_heads=7, n_kv_heads=2), M.ERR_INVALID_ARG),
    (dict(batch=0), M.ERR_INVALID_ARG),
    (dict(cluster_block=32768), M.ERR_UNSUPPORTED),
    (dict(tokens_per_centroid=0), M.ERR_INVALID_ARG),
    (dict(build_iters=0), M.ERR_INVALID_ARG),
    (dict(splits=-1), M.ERR_INVALID_ARG),
    (dict(coarse_tokens_per_centroid=64, cluster_block=8192), M.ERR_UNSUPPORTED),  # 128 coarse per block
    (dict(centroid_format=2), M.ERR_INVALID_ARG),
    (dict(centroid_format=1, dtype=torch.float32), M.ERR_UNSUPPORTED),
    (dict(centroid_format=1, coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096), M.ERR_UNSUPPORTED),
])
def test_parameter_validation(kw, status):
    p = _params(**kw)
    st = _fake_state(_params())
    assert _build(p, 100, st) == status
    assert _decode(p, st, 100) == status or status == M.ERR_INVALID_ARG


def test_build_validation():
    p = _params()
    st = _fake_state(p)
    cp = p.c()
    assert M.lib.mpattn_build_clusters(None, FAKE, FAKE, 10, ctypes.byref(st), None, 0, None) == M.ERR_INVALID_ARG
    assert M.lib.mpattn_build_clusters(ctypes.byref(cp), None, FAKE, 10, ctypes.byref(st), None, 0, None) == \
        M.ERR_INVALID_ARG
    assert M.lib.mpattn_build_clusters(ctypes.byref(cp), FAKE, FAKE, 10, None, None, 0, None) == M.ERR_INVALID_ARG
    assert _build(p, 0, st) == M.ERR_INVALID_ARG
    assert _build(p, 32769, st) == M.ERR_CAPACITY
    assert _build(p, 32768, _fake_state(p, C=2047)) == M.ERR_CAPACITY
    assert _build(p, 100, _fake_state(p, sorted_keys=FAKE)) == M.ERR_INVALID_ARG  # sorted K without sorted V
    assert _build(p, 100, _fake_state(p, sizes=None)) == M.ERR_INVALID_ARG
    ph = _params(coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096)
    assert _build(ph, 100, _fake_state(p)) == M.ERR_INVALID_ARG  # coarse arrays missing


def test_fp8_centroid_validation():
    """fp8 centroid copies: the state must carry all four arrays, and the
    decode runs on the one-launch path only."""
    p = _params(centroid_format=M.CENTROIDS_FP8)
    assert _build(p, 100, _fake_state(p)) == M.ERR_INVALID_ARG  # no code arrays
    full = dict(key_codes=FAKE, key_scales=FAKE, value_codes=FAKE, value_scales=FAKE)
    for missing in full:
        st = _fake_state(p, **{k: v for k, v in full.items() if k != missing})
        assert _build(p, 100, st) == M.ERR_INVALID_ARG
    st = _fake_state(p, n_clustered=4096, n_clusters=256, n_blocks=1, **full)
    assert p.decode_stages() != ["unit"]                       # 2 units: the split launches
    assert _decode(p, st, 4096) == M.ERR_UNSUPPORTED
    assert _decode(p, _fake_state(p, n_clustered=4096, n_clusters=256, n_blocks=1), 4096) == M.ERR_INVALID_ARG
    many = M.Params(batch=16, n_q_heads=32, n_kv_heads=8, capacity_tokens=32768, centroid_format=M.CENTROIDS_FP8)
    assert many.decode_stages() == ["unit"]
    assert _decode(dataclasses.replace(many, splits=4), _fake_state(many, n_clustered=4096, n_clusters=256,
                                                                    n_blocks=1, **full), 4096) == M.ERR_UNSUPPORTED


def test_update_validation():
    p = _params()
    st = _fake_state(p, n_clustered=16384, n_clusters=1024, n_blocks=2)
    cp = p.c()
    upd = lambda n, s: M.lib.mpattn_update_window(ctypes.byref(cp), FAKE, FAKE, n, ctypes.byref(s), None, 0, None)
    assert upd(16000, st) == M.ERR_INVALID_ARG     # behind the clustered prefix
    assert upd(40000, st) == M.ERR_CAPACITY
    assert upd(16384 + 8191, st) == M.OK            # tail shorter than a block: nothing to do
    assert st.n_clustered == 16384 and st.n_clusters == 1024
    full = _fake_state(p, n_clustered=16384, n_clusters=2040, n_blocks=2)
    assert upd(16384 + 8192, full) == M.ERR_CAPACITY


def test_decode_validation():
    p = _params()
    st = _fake_state(p, n_clustered=4096, n_clusters=256, n_blocks=1)
    need = M.lib.mpattn_workspace_bytes(ctypes.byref(p.c()), st.capacity_clusters, 0, M.OP_DECODE)
    assert 0 < need < (1 << 32)
    assert _decode(p, st, 4096, ws=need - 1) == M.ERR_WORKSPACE
    assert _decode(p, st, 4096, budget=-1) == M.ERR_INVALID_ARG
    assert _decode(p, st, 4000) == M.ERR_INVALID_ARG              # fewer tokens than clustered
    assert _decode(p, st, 40000) == M.ERR_INVALID_ARG             # beyond capacity
    assert _decode(p, st, 4096, mode=7) == M.ERR_INVALID_ARG
    assert _decode(p, st, 4096, q=None) == M.ERR_INVALID_ARG
    assert _decode(p, st, 4096, first=2, last=1) == M.ERR_INVALID_ARG
    assert _decode(p, st, 4096, first=0, last=4) == M.ERR_INVALID_ARG
    assert _decode(p, _fake_state(p), 0) == M.ERR_INVALID_ARG     # nothing clustered
    ph = _params(capacity_tokens=131072, coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096)
    sh = _fake_state(ph, n_clustered=8192, n_clusters=512, n_coarse=64, n_blocks=1)
    assert _decode(ph, sh, 8192, mode=M.MODE_OMIT) == M.ERR_UNSUPPORTED
    assert _decode(ph, sh, 8192, mode=M.MODE_PER_HEAD) == M.ERR_UNSUPPORTED
    assert _decode(ph, sh, 8192, ws=10) == M.ERR_WORKSPACE
    # per-head selection runs on the one-launch path only
    assert p.decode_stages() != ["unit"]
    assert _decode(p, st, 4096, mode=M.MODE_PER_HEAD) == M.ERR_UNSUPPORTED


def test_noalloc_decode_validation():
    """The allocation-free decode checks every argument, and that the
    layout fits its device array, before anything is enqueued (every case
    below returns before the device is touched)."""
    assert M.lib.mpattn_decode_noalloc_max_bytes() == 64 << 20
    p = _params()
    st = _fake_state(p, n_clustered=4096, n_clusters=256, n_blocks=1)
    cp = p.c()
    na = lambda n, budget=128, mode=0, q=FAKE, par=ctypes.byref(cp), s=st: M.lib.mpattn_decode_noalloc(
        par, q, FAKE, FAKE, n, ctypes.byref(s), budget, mode, FAKE, None)
    assert na(4096, budget=-1) == M.ERR_INVALID_ARG
    assert na(4000) == M.ERR_INVALID_ARG
    assert na(40000) == M.ERR_INVALID_ARG
    assert na(4096, mode=7) == M.ERR_INVALID_ARG
    assert na(4096, q=None) == M.ERR_INVALID_ARG
    assert na(4096, par=None) == M.ERR_INVALID_ARG
    assert na(0, s=_fake_state(p)) == M.ERR_INVALID_ARG
    assert na(4096, mode=M.MODE_PER_HEAD) == M.ERR_UNSUPPORTED
    # 512 units of 2053 clusters need more than the library's array
    big = _params(batch=64, n_q_heads=32, n_kv_heads=8)
    need = M.lib.mpattn_workspace_bytes(ctypes.byref(big.c()), big.max_clusters(), 0, M.OP_DECODE)
    assert need > M.lib.mpattn_decode_noalloc_max_bytes()
    sb = _fake_state(big, n_clustered=4096, n_clusters=256, n_blocks=1)
    cb = big.c()
    assert M.lib.mpattn_decode_noalloc(ctypes.byref(cb), FAKE, FAKE, FAKE, 4096, ctypes.byref(sb), 128, 0, FAKE,
                                       None) == M.ERR_WORKSPACE


def test_workspace_and_stages():
    p = _params()
    cp = p.c()
    assert M.lib.mpattn_workspace_bytes(ctypes.byref(cp), 100, 0, M.OP_BUILD) == 0
    assert M.lib.mpattn_workspace_bytes(ctypes.byref(cp), 100, 0, 9) == ctypes.c_size_t(-1).value
    assert p.decode_stages() == ["score", "select", "attend", "merge"]
    ph = _params(coarse_tokens_per_centroid=128, coarse_candidate_tokens=4096)
    # the hierarchy in one launch (bf16, automatic splits, G <= 4, up to 2048
    # coarse clusters and 4096 candidate tokens), else six launches
    assert ph.decode_stages() == ["hier_unit"]
    six = ["coarse_score", "coarse_select", "fine_score", "fine_select", "attend", "merge"]
    assert dataclasses.replace(ph, splits=4).decode_stages() == six
    assert dataclasses.replace(ph, coarse_candidate_tokens=4097).decode_stages() == six
    assert dataclasses.replace(ph, n_q_heads=16).decode_stages() == six                   # G = 8
    assert dataclasses.replace(ph, capacity_tokens=1 << 18).decode_stages() == six        # 2048 + 33 coarse
    assert dataclasses.replace(ph, dtype=torch.float32).decode_stages() == six
    # many units, automatic splits, bf16: the whole step of a unit in one workgroup
    many = M.Params(batch=16, n_q_heads=32, n_kv_heads=8, capacity_tokens=32768)
    assert many.decode_stages() == ["unit"]
    assert dataclasses.replace(many, splits=8).decode_stages() == ["score", "select", "attend", "merge"]
    assert dataclasses.replace(many, dtype=torch.float32).decode_stages() == ["score", "select", "attend", "merge"]
    # the one-launch workspace also holds the exchange of the per-head units:
    # eight workgroups per unit at 16 units of 4 heads, four per query head
    # at 64 one-head units
    few = M.Params(batch=2, n_q_heads=32, n_kv_heads=8, capacity_tokens=32768)
    assert few.decode_stages() == ["unit"]
    shared_only = 16 * 8 * 2048 * 8 + 16 * 8 * 4 * 130 * 8 + 16 * 8
    per_head = 64 * 4 * 2048 * 8 + 64 * 4 * 130 * 8 + 64 * 8
    ws = M.lib.mpattn_workspace_bytes(ctypes.byref(few.c()), 2048, 0, M.OP_DECODE)
    assert ws >= per_head > shared_only
    small = M.lib.mpattn_workspace_bytes(ctypes.byref(_params(splits=1).c()), 2053, 0, M.OP_DECODE)
    big = M.lib.mpattn_workspace_bytes(ctypes.byref(_params(splits=64).c()), 2053, 0, M.OP_DECODE)
    assert big > small


def test_dense_decode_validation():
    p = _params()
    cp = p.c()
    need = M.lib.mpattn_workspace_bytes(ctypes.byref(cp), 1, 0, M.OP_DENSE)
    assert 0 < need < (1 << 40)
    dense = lambda n, ws=1 << 40, q=FAKE, par=ctypes.byref(cp): M.lib.mpattn_dense_decode(
        par, q, FAKE, FAKE, n, FAKE, FAKE, ws, None)
    assert dense(0) == M.ERR_INVALID_ARG
    assert dense(p.capacity_tokens + 1) == M.ERR_INVALID_ARG
    assert dense(16, q=None) == M.ERR_INVALID_ARG
    assert dense(16, ws=need - 1) == M.ERR_WORKSPACE
    assert dense(16, par=None) == M.ERR_INVALID_ARG
    pf = _params(dtype=torch.float32)
    cpf = pf.c()
    assert M.lib.mpattn_dense_decode(ctypes.byref(cpf), FAKE, FAKE, FAKE, 16, FAKE, FAKE, 1 << 40, None) == \
        M.ERR_UNSUPPORTED
