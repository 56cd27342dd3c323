#!/usr/bin/env python3
"""Decode-step benchmark of the Multipole Attention hot path on one MI355X.

Workload: a Qwen3-8B-shaped attention layer (32 query heads, 8 KV heads, head
dim 128, bf16), batch 16, 32768-token clustered-Gaussian KV cache per sequence
(synthetic: no dataset or weights are available), 1 centroid per 16 tokens in
8192-token blocks, 95% sparsity (1638 exactly attended tokens per KV head),
a fresh query per step.

One step = one decode of the whole batch through the C ABI: score and budget
cut (one launch), then split-K attention with the merge (one launch).  The clustering is built once before timing (prefill time)
and reported separately.  Headline timing is cold: before every step a 1 GiB
streaming read (the library's read probe) evicts the 256 MB Infinity Cache and
the L2s with clean lines, so the centroids and rows come from HBM.  The steps
run back to back, each behind its flush, inside one event pair; the same
number of flushes timed alone is subtracted (median of 9 alternating rounds).
Cold steps each bracketed by their own event pair are reported too: that
figure also holds the event records and the dispatch of a launch that waits
for its start event (an empty kernel reads about 6 us that way, reported as
the floor).  The same probe, timed alone, gives the achievable read rate.
Warm (back-to-back, no flush) timing is reported as well.  The dominant
kernel's average duration for the roofline object is the back-to-back figure
when the step is one launch, else per-stage HIP events on the launch stream.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import ctypes
import dataclasses
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
HBM_TARGET_FRAC = 0.60           # decode target: this fraction of peak on the bytes read
DEFAULT_WORKLOAD = "qwen3-8b-layer-b16-32k-s95"

# HBM bytes per launch of the one-launch decode kernels, from two rocprofv3
# --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, mean over the
# run's dispatches), each scaled by what the same counter reads for data of
# known size: a 256 MiB device copy and the library's 256 MiB streaming read
# both give FETCH_SIZE 131085 KiB (x2.0); the copy's WRITE_SIZE is 262144 KiB
# (x1.0).  Valid only for the kernel sources they were taken on (sha256 over
# the listed files, in that order); otherwise reported null.
UNIT_TRAFFIC = {  # per centroid format
    "stored": {
        "sources_sha256": "e16e2b42a822fec0a3ac0257b7f51845c7ea3aeefdd3784d3767deb7ae92b4b9",
        "fetch_bytes": int(122922.2 * 2.0 * 1024),
        "write_bytes": int(3476.0 * 1.0 * 1024),
        "profile": "profiles/decode_b16_32k_s95_unit_hbm_counters.md",
    },
    "fp8": {
        "sources_sha256": "e16e2b42a822fec0a3ac0257b7f51845c7ea3aeefdd3784d3767deb7ae92b4b9",
        "fetch_bytes": int(90231.6 * 2.0 * 1024),
        "write_bytes": int(3475.9 * 1.0 * 1024),
        "profile": "profiles/decode_b16_32k_s95_unit_hbm_counters.md",
    },
}
HIER_TRAFFIC = {  # the one-launch hierarchical decode, 131072 tokens, batch 4
    "sources_sha256": "43b09a4a57c30a4567bb7a0f2e94b1077204e769155c48d927a7bd9e4453cc6c",
    "files": ("hier.hip", "attn.hpp", "device.hpp", "kernels.hpp"),
    "fetch_bytes": int(18356.8 * 2.0 * 1024),
    "write_bytes": int(3054.0 * 1.0 * 1024),
    "profile": "profiles/decode_b4_128k_hier_kernel.md",
}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=8, help="oracle decode steps timed for the CPU baseline")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--gather", action="store_true", help="decode by token-id gather instead of the sorted copy")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the dense reference, the ablation, the fp8 step and the other rows")
    ap.add_argument("--centroids", choices=["stored", "fp8"], default="stored",
                    help="centroids the timed decode reads: the stored bf16 ones (the method as the pages "
                         "describe it) or their fp8 copies")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--read-probe-mb", type=int, default=0,
                    help="only run the library's streaming read of this many MiB (counter calibration) and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every (sequence, KV head) unit is independent; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from sparse_long_context_means_amd import mpattn as M

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"copy probe: 3 copies of {args.copy_probe_mb} MiB")
        return
    if args.read_probe_mb:
        x = torch.ones(args.read_probe_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            M.read_probe(x, sink)
        torch.cuda.synchronize()
        log(f"read probe: 3 reads of {args.read_probe_mb} MiB")
        return

    w = workloads.WORKLOADS[args.workload]
    B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.n_tokens, w.head_dim
    G = Hq // Hkv
    T = w.budgets[0]
    t0 = time.time()
    K, V, means = workloads.make_cache(w)
    log(f"[bench] synthetic cache {tuple(K.shape)} {K.dtype} in {time.time() - t0:.1f}s")
    Kd, Vd = K.to(dev), V.to(dev)
    p = _params_for(M, w, capacity_tokens=N, splits=args.splits,
                    centroid_format=M.CENTROIDS_FP8 if args.centroids == "fp8" else M.CENTROIDS_STORED)
    state = M.ClusterState(p, dev, sorted_copy=not args.gather)

    # ---- build (prefill time), reported separately -------------------------
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    M.build_clusters(p, Kd, Vd, N, state)  # warm-up build (also JIT/code-object load)
    torch.cuda.synchronize()
    e0.record()
    M.build_clusters(p, Kd, Vd, N, state)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    U = B * Hkv
    C = state.n_clusters
    nb = math.ceil(N / w.cluster_block)
    assign_flop = 2.0 * U * N * (w.cluster_block // w.tokens_per_centroid) * d * w.build_iters
    log(f"[bench] build {build_ms:.2f} ms ({C} clusters per unit, {nb} blocks)")

    # ---- queries and per-step selection sizes (untimed) ----------------------
    n_q = args.warmup + args.steps
    qs = [workloads.make_queries(w, means, s).to(dev) for s in range(n_q)]
    ws = M.Workspace().get(p, state, dev)  # zero-filled
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    dbg = M.DecodeDebug.allocate(p, state, dev)
    exact_rows = []
    for s in range(n_q):
        M.decode(p, qs[s], Kd, Vd, N, state, T, out=out, workspace=ws, debug=dbg)
        exact_rows.append(int(dbg.exact_tokens.sum()))
    torch.cuda.synchronize()

    def bytes_of(step):
        e = exact_rows[step]
        crow = d + d // 32 if args.centroids == "fp8" else d * 2  # bytes of a centroid row
        score = B * Hq * d * 2 + U * C * crow             # queries + key centroids
        # exact K/V rows + their ids + every value centroid (the attend launch
        # streams the approximate term of all clusters and removes the selected)
        attend = e * d * 2 * 2 + e * 4 + U * C * crow
        other = U * C * 4 + B * Hq * d * 4                 # sizes + output
        return score, attend, other

    # ---- timed decode --------------------------------------------------------
    cp, cs = p.c(), state.c()
    n_stages = M.lib.mpattn_decode_stage_count(ctypes.byref(cp))
    stage_names = p.decode_stages()
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read to evict caches
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def evict():
        M.read_probe(flush, sink)

    # achievable streaming-read rate of this GPU (the same 1 GiB read)
    pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evict()
    probe_ms = []
    for _ in range(5):
        pa.record(stream)
        evict()
        pb.record(stream)
        torch.cuda.synchronize()
        probe_ms.append(pa.elapsed_time(pb))
    probe_gbps = flush.numel() * 4 / (min(probe_ms) * 1e-3) / 1e9
    log(f"[bench] streaming-read probe {probe_gbps:.0f} GB/s")

    def enqueue(s, first=0, last=n_stages - 1):
        st = M.lib.mpattn_decode_ex(ctypes.byref(cp), ctypes.c_void_p(qs[s].data_ptr()),
                                    ctypes.c_void_p(Kd.data_ptr()), ctypes.c_void_p(Vd.data_ptr()), N,
                                    ctypes.byref(cs), T, 0, ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(ws.data_ptr()), ws.numel(), sptr, None, first, last)
        if st != 0:
            raise RuntimeError(M.status_string(st))

    for s in range(args.warmup):
        evict()
        enqueue(s)
    torch.cuda.synchronize()

    # cold, headline: one event pair per step, cache flushed before each step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        ev[i][0].record(stream)
        enqueue(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])

    # cold, per stage: events between the stage launches (same stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stages + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        s = args.warmup + i
        evict()
        evs[i][0].record(stream)
        for k in range(n_stages):
            enqueue(s, k, k)
            evs[i][k + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = np.array([[evs[i][k].elapsed_time(evs[i][k + 1]) for k in range(n_stages)]
                         for i in range(args.steps)])

    # cold, back to back (headline): K x (cache flush + step) inside one event
    # pair, less K flushes timed alone the same way, in 9 alternating rounds
    # (median).  The per-step pairs above also time the two event records and
    # a dispatch that cannot begin before its start event; an empty kernel
    # reads about 6 us there (floor below).  Here every launch is queued
    # behind its flush, as in a stream of decode steps, and the caches are
    # still evicted before every step.
    def loop_us(with_step):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record(stream)
        for i in range(args.steps):
            evict()
            if with_step:
                enqueue(args.warmup + i)
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) * 1e3

    b2b_rounds = []
    for _ in range(9):
        both = loop_us(True)
        b2b_rounds.append((both - loop_us(False)) / args.steps)
    b2b_us = float(np.median(b2b_rounds))
    # the event-pair floor: an empty kernel (torch's fill of one float) timed
    # like a cold step
    tiny = torch.zeros(1, device=dev)
    floor = []
    for _ in range(20):
        evict()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        tiny.zero_()
        b_.record(stream)
        torch.cuda.synchronize()
        floor.append(a_.elapsed_time(b_) * 1e3)
    pair_floor_us = float(np.median(floor[2:]))

    # warm: back-to-back full steps, one event pair around all of them
    wa, wb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wa.record(stream)
    for i in range(args.steps):
        enqueue(args.warmup + i)
    wb.record(stream)
    torch.cuda.synchronize()
    warm_us = wa.elapsed_time(wb) * 1e3 / args.steps

    steps_idx = range(args.warmup, args.warmup + args.steps)
    byts = np.array([sum(bytes_of(s)) for s in steps_idx], dtype=np.float64)
    # dominant kernel: the per-unit kernel (the whole step) or the split
    # attend kernel
    if len(stage_names) == 1:  # one launch: the whole step
        dom = stage_names[0]
        att_bytes = byts.copy()
    else:
        dom = "attend"
        att_bytes = np.array([bytes_of(s)[1] for s in steps_idx], dtype=np.float64)
    pair_us = float(step_ms.mean() * 1e3)
    cold_us = b2b_us
    eff_gbps = float(byts.mean() / (cold_us * 1e-6) / 1e9)
    att_k = stage_names.index(dom)
    # the dominant kernel's average launch: the back-to-back figure when the
    # step is that one launch, else the per-stage event pairs
    att_us = b2b_us if len(stage_names) == 1 else float(stage_ms[:, att_k].mean() * 1e3)
    att_gbps = float(att_bytes.mean() / (att_us * 1e-6) / 1e9)
    log(f"[bench] cold {cold_us:.1f} us/step back to back ({pair_us:.1f} with an event pair per step, "
        f"empty-kernel floor {pair_floor_us:.1f})  warm {warm_us:.1f} us/step  "
        f"stages(us) " + " ".join(f"{n}={stage_ms[:, k].mean() * 1e3:.1f}" for k, n in enumerate(stage_names)))

    # every timed step must have completed normally: the workspace counters of
    # the one-launch decode (key-exchange fallbacks, outputs poisoned because a
    # partial did not arrive) and a finite output
    fallbacks, poisoned = M.decode_status(ws)
    finite = bool(torch.isfinite(out).all())
    if poisoned or not finite:
        raise RuntimeError(f"decode failed: {poisoned} poisoned outputs, finite output {finite}")
    status = {"key_exchange_fallbacks": fallbacks, "poisoned_outputs": poisoned, "output_finite": finite}

    # ---- memory: what the method keeps beside the KV cache -------------------
    Cm = state.capacity_clusters
    kv_bytes = 2 * U * N * d * 2
    memory = {
        "kv_cache_bytes": kv_bytes,
        "centroids_read_by_decode_bytes": 2 * U * Cm * d * 2 + U * Cm * 4 * 2,   # Kbar, Vbar, sizes, offsets
        "cluster_state_bytes": U * Cm * d * (2 + 2 + 4) + U * (2 * Cm + 1) * 4 + 2 * U * N * 4,
        "sorted_copy_bytes": 0 if args.gather else kv_bytes,
    }
    for k in ("centroids_read_by_decode_bytes", "cluster_state_bytes", "sorted_copy_bytes"):
        memory[k.replace("_bytes", "_frac_of_kv")] = round(memory[k] / kv_bytes, 4)
    log(f"[bench] memory beside the KV cache: centroids {memory['centroids_read_by_decode_frac_of_kv']:.3f}, "
        f"whole cluster state {memory['cluster_state_frac_of_kv']:.3f}, sorted copy {memory['sorted_copy_frac_of_kv']:.3f}")

    # ---- dense split-K decode of the same step (the pages' comparison point) --
    dense = fp8 = gather = None
    if not args.no_rows and args.centroids == "stored":
        dws = torch.empty(int(M.lib.mpattn_workspace_bytes(ctypes.byref(cp), 1, 0, M.OP_DENSE)), dtype=torch.uint8,
                          device=dev)
        dts = []
        for i in range(min(10, args.steps)):
            evict()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            M.dense_decode(p, qs[args.warmup + i], Kd, Vd, N, out=out, workspace=dws)
            b_.record(stream)
            torch.cuda.synchronize()
            dts.append(a_.elapsed_time(b_) * 1e3)
        dense_us = float(np.median(dts))
        dense_bytes = U * N * d * 2 * 2 + B * Hq * d * (2 + 4)
        dense = {"us_per_step": round(dense_us, 2), "algorithmic_MB": round(dense_bytes / 1e6, 1),
                 "roofline": {"bound": "hbm", "achieved": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(dense_bytes / (dense_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
                 "sparse_speedup": round(dense_us / cold_us, 2)}
        log(f"[bench] dense split-K decode {dense_us:.1f} us/step ({dense_us / cold_us:.2f}x the sparse step)")
        # the same build with fp8 centroid copies (same seed: the same clusters)
        p8 = dataclasses.replace(p, centroid_format=M.CENTROIDS_FP8)
        state8 = M.ClusterState(p8, dev, sorted_copy=not args.gather)
        M.build_clusters(p8, Kd, Vd, N, state8)
        torch.cuda.synchronize()
        variants = {"multipole": (p, state, M.MODE_MULTIPOLE), "omit": (p, state, M.MODE_OMIT),
                    "per_head": (p, state, M.MODE_PER_HEAD), "fp8_centroids": (p8, state8, M.MODE_MULTIPOLE)}
        n_abl = min(8, args.steps)
        dense["ablation"] = {
            "independent_heads": measure_ablation(M, variants, [qs[args.warmup + i] for i in range(n_abl)],
                                                  Kd, Vd, N, T, ws, dws, evict),
            "group_shared_component": measure_ablation(
                M, variants, [workloads.make_queries(w, means, args.warmup + i, group_shared=True).to(dev)
                              for i in range(n_abl)], Kd, Vd, N, T, ws, dws, evict)}
        # fp8 centroid copies on the timed queries: bytes and roofline
        f8_us = _cold_decode_us(M, p8, [qs[args.warmup + i] for i in range(args.steps)], Kd, Vd, N, state8, T, ws,
                                evict)
        f8_bytes = float(byts.mean()) - 2 * U * C * d * 2 + 2 * U * C * (d + d // 32)
        fp8 = {"us_per_step": round(f8_us, 2), "algorithmic_MB": round(f8_bytes / 1e6, 2),
               "roofline": {"bound": "hbm", "achieved": round(f8_bytes / (f8_us * 1e-6) / 1e9, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(f8_bytes / (f8_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                            "traffic": _unit_traffic_bytes("fp8") if args.workload == DEFAULT_WORKLOAD and
                            not args.gather else None},
               "speedup_vs_stored_centroids": round(cold_us / f8_us, 3)}
        log(f"[bench] fp8 centroids {f8_us:.1f} us/step ({fp8['roofline']['achieved']:.0f} GB/s algorithmic)")
        del state8
        del dws
        if not args.gather:
            # the same clusters without the sorted copy: exact rows gathered
            # from K, V through the token ids (no duplicate of the cache)
            stg = M.ClusterState(p, dev, sorted_copy=False)
            M.build_clusters(p, Kd, Vd, N, stg)
            torch.cuda.synchronize()
            wsg = M.Workspace().get(p, stg, dev)
            g_us = _cold_decode_us(M, p, [qs[args.warmup + i] for i in range(min(40, args.steps))], Kd, Vd, N, stg, T,
                                   wsg, evict)
            g_bytes = float(byts.mean())
            gather = {"us_per_step": round(g_us, 2), "algorithmic_MB": round(g_bytes / 1e6, 2),
                      "roofline": {"bound": "hbm", "achieved": round(g_bytes / (g_us * 1e-6) / 1e9, 1),
                                   "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(g_bytes / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
                      "extra_memory_bytes": 0, "sorted_copy_speedup": round(g_us / cold_us, 3)}
            log(f"[bench] gathered exact rows (no sorted copy) {g_us:.1f} us/step")
            del stg, wsg

    rows = None if args.no_rows else measure_rows(M, workloads, dev, evict)

    # ---- CPU baseline: the oracle on the machine's host cores --------------------
    cpu = None
    if not args.no_cpu_baseline and not p.hierarchical:  # the oracle leg times the flat decode
        import oracle as O
        from concurrent.futures import ThreadPoolExecutor

        threads = min(16, os.cpu_count() or 1)
        ust = []
        for u in range(U):
            b, h = divmod(u, Hkv)
            st = O.empty_state(d, N, state.capacity_clusters, O.BF16)
            st.kbar[:C] = state.key_centroids[b, h, :C].double().cpu().numpy()
            st.vbar[:C] = state.value_centroids[b, h, :C].double().cpu().numpy()
            st.sizes[:C] = state.sizes[b, h, :C].cpu().numpy()
            st.assign[:N] = state.assign[b, h, :N].cpu().numpy()
            st.n_clusters, st.n_clustered = C, N
            ust.append((st, O.f64(K[b, h]), O.f64(V[b, h])))
        qcpu = [qs[args.warmup + i].cpu() for i in range(args.cpu_steps)]

        def one(args_):
            i, u = args_
            b, h = divmod(u, Hkv)
            st, Ku, Vu = ust[u]
            O.decode_unit(qcpu[i][b, h * G:(h + 1) * G], Ku, Vu, N, st, T)

        jobs = [(i, u) for i in range(args.cpu_steps) for u in range(U)]
        c0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
        cpu_s = time.perf_counter() - c0
        # one host thread: the median of single full steps
        one_thread = []
        for i in range(min(3, args.cpu_steps)):
            c1 = time.perf_counter()
            for u in range(U):
                one((i, u))
            one_thread.append(time.perf_counter() - c1)
        # clustering: one (unit, block) of the workload, every Lloyd round,
        # on one thread; the build covers U units x nb blocks
        Kb, Vb = O.f64(K[0, 0]), O.f64(V[0, 0])
        st1 = O.empty_state(d, N, state.capacity_clusters, O.BF16)
        c2 = time.perf_counter()
        O.cluster_block(st1, Kb, Vb, 0, w.cluster_block, w.build_iters, w.tokens_per_centroid, 0, 0, 0)
        blk_s = time.perf_counter() - c2
        cpu = {"value": cpu_s / args.cpu_steps * 1e6, "unit": "us/step", "cores": threads,
               "host_cpu_count": os.cpu_count(), "kind": "oracle",
               "sample": f"{args.cpu_steps} full decode steps ({U} units each) of the same workload, fp64 oracle, "
                         f"units spread over {threads} host threads",
               "one_thread_us_per_step_median": round(float(np.median(one_thread)) * 1e6, 1),
               "one_thread_sample": f"{len(one_thread)} full decode steps, one host thread",
               "build_one_unit_block_s": round(blk_s, 3),
               "build_extrapolated_s": {"one_thread": round(blk_s * U * nb, 1),
                                        f"{threads}_threads": round(blk_s * U * nb / threads, 2),
                                        "basis": f"one (unit, block) of {w.cluster_block} tokens, {w.build_iters} "
                                                 f"rounds, timed; x {U * nb} (unit, block) pairs"},
               "cpu_model": _cpu_model()}
        log(f"[bench] oracle {cpu['value'] / 1e3:.1f} ms/step on {threads} threads, "
            f"{cpu['one_thread_us_per_step_median'] / 1e3:.1f} ms/step on one; one (unit, block) build {blk_s:.2f} s")

    res = {
        "metric": "decode attn µs/step + effective HBM GB/s, 32K ctx, bs16, 95% sparsity",
        "value": round(cold_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic clustered-Gaussian KV cache (no dataset/weights)",
        "config": {"workload": w.name, "batch": B, "seq_len": N, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d,
                   "centroids": "bf16" if args.centroids == "stored" else "fp8 e4m3, scale per 32",
                   "token_budget": T, "tokens_per_centroid": w.tokens_per_centroid,
                   "cluster_block": w.cluster_block, "exact_rows": "sorted copy" if not args.gather else "gather",
                   "splits": args.splits or "auto"},
        "effective_GBps": round(eff_gbps, 1),
        "effective_frac_of_hbm_peak": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "hbm_read_probe_GBps": round(probe_gbps, 1),
        "effective_frac_of_read_probe": round(eff_gbps / probe_gbps, 4),
        # the target: 60% of HBM peak on the bytes the step reads
        "hbm_target": {"frac": HBM_TARGET_FRAC,
                       "us_per_step": round(float(byts.mean()) / (HBM_TARGET_FRAC * HBM_PEAK_GBPS * 1e3), 2),
                       "met": bool(eff_gbps >= HBM_TARGET_FRAC * HBM_PEAK_GBPS)},
        "algorithmic_MB_per_step": round(float(byts.mean()) / 1e6, 2),
        "warm_us_per_step": round(warm_us, 2),
        "cold_back_to_back_rounds_us": [round(x, 2) for x in b2b_rounds],
        "cold_event_pair_us_per_step": round(pair_us, 2),
        "cold_event_pair_us_p10_p50_p90": [round(float(np.percentile(step_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
        "event_pair_floor_us": round(pair_floor_us, 2),
        "stage_sum_us": round(float(stage_ms.sum(1).mean()) * 1e3, 2),
        "stage_us": {n: round(float(stage_ms[:, k].mean()) * 1e3, 2) for k, n in enumerate(stage_names)},
        "timed_wall_ms_incl_cache_flush": round(wall_ms, 2),
        "build_ms": round(build_ms, 2),
        "build_assign_TFLOPs_lower_bound": round(assign_flop / (build_ms * 1e-3) / 1e12, 1),
        "roofline": None if p.hierarchical else {"bound": "hbm", "kernel": dom, "achieved": round(att_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": _unit_traffic_bytes(args.centroids)
                     if dom == "unit" and args.workload == DEFAULT_WORKLOAD and not args.gather else None,
                     "algorithmic_MB_per_launch": round(float(att_bytes.mean()) / 1e6, 2),
                     "avg_launch_us": round(att_us, 2)},
        "cpu_baseline": cpu,
        "decode_status": status,
        "memory": memory,
        "gather_exact_rows": gather,
        "dense_reference": dense,
        "fp8_centroids": fp8,
        "rows": rows,
    }
    print(json.dumps(res), flush=True)


def _params_for(M, w, **kw):
    base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, capacity_tokens=w.capacity,
                dtype=w.dtype, tokens_per_centroid=w.tokens_per_centroid, cluster_block=w.cluster_block,
                build_iters=w.build_iters, update_iters=w.update_iters,
                coarse_tokens_per_centroid=w.coarse_tokens_per_centroid,
                coarse_candidate_tokens=w.coarse_candidate_tokens, seed=0)
    base.update(kw)
    return M.Params(**base)


def _cold_decode_pair_us(M, p, qs, Kd, Vd, n_total, state, T, ws, evict, mode=0):
    """Median cold decode time (µs) over the given queries, caches evicted
    before each step, one event pair per step on the launch stream."""
    import numpy as np
    import torch
    ts = []
    for q in qs:
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        M.decode(p, q, Kd, Vd, n_total, state, T, mode=mode, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return float(np.median(ts))


def _cold_decode_us(M, p, qs, Kd, Vd, n_total, state, T, ws, evict, mode=0, rounds=3):
    """Cold decode time (µs per step) back to back: the queries' steps, each
    behind a cache flush, in one event pair, less the flushes alone; median
    over alternating rounds."""
    import numpy as np
    import torch

    def loop(with_step):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for q in qs:
            evict()
            if with_step:
                M.decode(p, q, Kd, Vd, n_total, state, T, mode=mode, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    loop(True)  # warm-up (output allocations)
    res = []
    for _ in range(rounds):
        both = loop(True)
        res.append((both - loop(False)) / len(qs))
    return float(np.median(res))


def measure_ablation(M, variants, qs, Kd, Vd, n_total, T, ws, dws, evict):
    """Output error against exact dense attention, and cold time, of decode
    variants (name -> (params, state, mode)): the shared selection with
    centroid terms (the method), the same selection with the unselected
    clusters dropped, per-query-head selection with centroid terms, and the
    method reading fp8 centroid copies.  Error per query head:
    ||o - o_dense|| / ||o_dense||."""
    import numpy as np
    import torch
    p0 = next(iter(variants.values()))[0]
    errs = {k: [] for k in variants}
    exact = {k: 0 for k in variants}
    for q in qs:
        ref = M.dense_decode(p0, q, Kd, Vd, n_total, workspace=dws).double()
        for name, (p, state, md) in variants.items():
            dbg = M.DecodeDebug.allocate(p, state, q.device, per_head=md == M.MODE_PER_HEAD)
            o = M.decode(p, q, Kd, Vd, n_total, state, T, mode=md, workspace=ws, debug=dbg).double()
            e = (o - ref).norm(dim=-1) / ref.norm(dim=-1)
            errs[name].append(e.flatten().cpu())
            rows = int(dbg.exact_tokens.sum())
            exact[name] += rows * (1 if md == M.MODE_PER_HEAD else p.group)
    torch.cuda.synchronize()
    res = {}
    for name, (p, state, md) in variants.items():
        e = torch.cat(errs[name]).numpy()
        res[name] = {"rel_l2_err_mean": float(f"{e.mean():.4g}"), "rel_l2_err_p99": float(f"{np.percentile(e, 99):.4g}"),
                     "rel_l2_err_max": float(f"{e.max():.4g}"),
                     "exact_rows_per_query_head": round(exact[name] / (len(qs) * p.batch * p.n_q_heads), 1),
                     "cold_us_per_step": round(_cold_decode_us(M, p, qs, Kd, Vd, n_total, state, T, ws, evict,
                                                               mode=md), 2)}
        log(f"[bench] ablation {name}: rel err mean {e.mean():.4f} max {e.max():.4f}  "
            f"{res[name]['cold_us_per_step']:.1f} us/step")
    res["queries"] = f"{len(qs)} decode steps x {p0.batch * p0.n_q_heads} query heads, budget {T} tokens"
    return res


def measure_rows(M, workloads, dev, evict):
    """The other rows of the path on their own workloads: the online window
    update (a new 8192-token block clustered, 5 rounds, batch 4) with a decode
    over the unclustered tail, and the hierarchical decode at 131072 tokens.
    Rooflines: the update's assign contraction against the bf16 matrix-core
    peak, the decodes against HBM."""
    import numpy as np
    import torch
    rows = {}
    d = 128
    # ---- the small workloads: the tiny fp32 case and the batch-1 layer -------
    for name in ("tiny-fp32", "qwen3-8b-layer-b1-32k"):
        w = workloads.WORKLOADS[name]
        K, V, means = workloads.make_cache(w)
        Kd, Vd = K.to(dev), V.to(dev)
        p = _params_for(M, w)
        st = M.ClusterState(p, dev)
        M.build_clusters(p, Kd, Vd, w.n_tokens, st)
        ws = M.Workspace().get(p, st, dev)
        qs = [workloads.make_queries(w, means, s).to(dev) for s in range(12)]
        C, U = st.n_clusters, p.units
        esz = 2 if w.dtype == torch.bfloat16 else 4
        for T in w.budgets:
            dbg = M.DecodeDebug.allocate(p, st, dev)
            M.decode(p, qs[0], Kd, Vd, w.n_tokens, st, T, workspace=ws, debug=dbg)
            E = int(dbg.exact_tokens.sum())
            byts = p.batch * p.n_q_heads * d * (esz + 4) + U * C * (2 * d * esz + 4) + E * (2 * d * esz + 4)
            us = _cold_decode_us(M, p, qs[2:], Kd, Vd, w.n_tokens, st, T, ws, evict)
            rows[f"{name}_T{T}"] = {
                "workload": name, "token_budget": T, "dtype": "f32" if esz == 4 else "bf16",
                "decode_stages": p.decode_stages(), "us_per_step": round(us, 2), "algorithmic_MB": round(byts / 1e6, 3),
                "roofline": {"bound": "hbm", "achieved": round(byts / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}}
            log(f"[bench] {name} T={T}: {us:.1f} us/step ({byts / 1e6:.2f} MB)")
        del K, V, Kd, Vd, st, ws
    torch.cuda.empty_cache()
    # ---- online update (H3) and decode with a tail ----------------------------
    w = workloads.WORKLOADS["qwen3-8b-layer-b4-online"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(dev), V.to(dev)
    p = _params_for(M, w)
    st = M.ClusterState(p, dev)
    M.build_clusters(p, Kd, Vd, w.n_tokens, st)
    n = w.n_tokens
    U = p.units
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    M.update_window(p, Kd, Vd, n + w.cluster_block, st)
    b.record()
    torch.cuda.synchronize()
    upd_ms = a.elapsed_time(b)
    n += w.cluster_block
    flop = 2.0 * U * w.cluster_block * (w.cluster_block // w.tokens_per_centroid) * d * w.update_iters
    tail = 4096
    M.update_window(p, Kd, Vd, n + tail, st)  # tail only: no block completes
    T = w.budgets[0]
    ws = M.Workspace().get(p, st, dev)
    qs = [workloads.make_queries(w, means, s).to(dev) for s in range(12)]
    dbg = M.DecodeDebug.allocate(p, st, dev)
    M.decode(p, qs[0], Kd, Vd, n + tail, st, T, workspace=ws, debug=dbg)
    E = int(dbg.exact_tokens.sum())
    C = st.n_clusters
    byts = p.batch * p.n_q_heads * d * (2 + 4) + U * C * (2 * d * 2 + 4) + E * 2 * d * 2 + U * tail * 2 * d * 2
    us = _cold_decode_us(M, p, qs[2:], Kd, Vd, n + tail, st, T, ws, evict)
    rows["H3_online_update"] = {
        "workload": w.name, "block_tokens": w.cluster_block, "rounds": w.update_iters, "ms": round(upd_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(flop / (upd_ms * 1e-3) / 1e12, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(flop / (upd_ms * 1e-3) / 1e12 / 2500.0, 4)}}
    rows["H3_decode_with_tail"] = {
        "workload": w.name, "n_clustered": n, "tail_tokens": tail, "token_budget": T, "us_per_step": round(us, 2),
        "algorithmic_MB": round(byts / 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(byts / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}}
    log(f"[bench] H3 update {upd_ms:.3f} ms, decode with {tail}-token tail {us:.1f} us")
    # ---- the update on a second stream while decodes continue on the first ---
    main, side = torch.cuda.current_stream(dev), torch.cuda.Stream(dev)
    n_total = w.n_tokens + w.cluster_block  # the new block is the tail until clustered
    dq = qs[:8] * 4
    dout = torch.empty(p.batch, p.n_q_heads, d, dtype=torch.float32, device=dev)
    dev_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in dq]

    def decodes(view):  # nothing allocated inside: the loop only enqueues
        for q, (e_a, e_b) in zip(dq, dev_evs):
            e_a.record(main)
            M.decode(p, q, Kd, Vd, n_total, view, T, out=dout, workspace=ws)
            e_b.record(main)
        return dev_evs

    alone_st = M.ClusterState(p, dev)
    M.build_clusters(p, Kd, Vd, w.n_tokens, alone_st)
    evs = decodes(alone_st)
    torch.cuda.synchronize()
    dec_alone = float(np.median([x.elapsed_time(y) * 1e3 for x, y in evs]))
    torch.cuda.empty_cache()
    import gc

    def concurrent_trial():
        conc_st = M.ClusterState(p, dev)
        M.build_clusters(p, Kd, Vd, w.n_tokens, conc_st)
        torch.cuda.synchronize()
        # both streams start at `origin`, which follows ~4 ms of streaming
        # reads on the main stream: by then the host has enqueued the update
        # and all the decodes, so the two really overlap
        for _ in range(20):
            evict()
        origin = torch.cuda.Event(enable_timing=True)
        origin.record(main)
        side.wait_event(origin)
        h0 = time.perf_counter()
        view, done, _ = M.update_window_concurrent(p, Kd, Vd, n_total, conc_st, side)
        end = torch.cuda.Event(enable_timing=True)
        end.record(side)  # right behind the update's launches
        evs = decodes(view)
        enq_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        upd = origin.elapsed_time(end)
        dur = [x.elapsed_time(y) * 1e3 for x, y in evs if origin.elapsed_time(x) < upd]
        last = max(origin.elapsed_time(y) for _, y in evs)
        return upd, dur, last, enq_ms

    # the second of two trials (the first one runs the machinery once), with
    # the garbage collector held off while the host enqueues
    gc.disable()
    try:
        concurrent_trial()
        upd_conc, during, last_dec, enq_ms = concurrent_trial()
    finally:
        gc.enable()
    rows["H3_concurrent_update"] = {
        "workload": w.name, "decodes_enqueued": len(dq),
        "decodes_end_ms": round(last_dec, 3), "host_enqueue_ms": round(enq_ms, 3),
        "decode_us_alone": round(dec_alone, 2),
        "decode_us_during_update": round(float(np.median(during)), 2) if during else None,
        "decodes_during_update": len(during),
        "update_ms_alone": round(upd_ms, 3), "update_ms_beside_decodes": round(upd_conc, 3)}
    log(f"[bench] H3 concurrent: decode {dec_alone:.1f} us alone, "
        f"{(np.median(during) if during else float('nan')):.1f} us during the update ({len(during)} decodes); "
        f"update {upd_ms:.3f} ms alone, {upd_conc:.3f} ms beside decodes")
    del K, V, Kd, Vd, st, ws
    torch.cuda.empty_cache()
    # ---- hierarchical decode (H8) ---------------------------------------------
    w = workloads.WORKLOADS["qwen3-8b-layer-b4-128k-hier"]
    K, V, means = workloads.make_cache(w)
    Kd, Vd = K.to(dev), V.to(dev)
    p = _params_for(M, w)
    st = M.ClusterState(p, dev)
    M.build_clusters(p, Kd, Vd, w.n_tokens, st)
    torch.cuda.synchronize()
    a.record()
    M.build_clusters(p, Kd, Vd, w.n_tokens, st)
    b.record()
    torch.cuda.synchronize()
    build_ms = a.elapsed_time(b)
    U, N, T = p.units, w.n_tokens, w.budgets[0]
    ws = M.Workspace().get(p, st, dev)
    qs = [workloads.make_queries(w, means, s).to(dev) for s in range(12)]
    dbg = M.DecodeDebug.allocate(p, st, dev)
    M.decode(p, qs[0], Kd, Vd, N, st, T, workspace=ws, debug=dbg)
    E = int(dbg.exact_tokens.sum())
    cand = dbg.candidates.cpu().numpy().astype(bool)           # [B][Hkv][D]
    coff = st.coarse_offsets.cpu().numpy()                      # [B][Hkv][D+1]
    D = st.n_coarse
    fine_in_cand = int(((coff[..., 1:D + 1] - coff[..., :D]) * cand[..., :D]).sum())
    # coarse K̄ and V̄ and sizes of every coarse cluster; fine K̄, V̄ and sizes of
    # the fine clusters inside the candidates; the exact rows; queries, output
    byts = U * D * (2 * d * 2 + 4) + fine_in_cand * (2 * d * 2 + 4 + 4) + E * 2 * d * 2 \
        + p.batch * p.n_q_heads * d * (2 + 4)
    us = _cold_decode_us(M, p, qs[2:], Kd, Vd, N, st, T, ws, evict)
    us_pair = _cold_decode_pair_us(M, p, qs[2:], Kd, Vd, N, st, T, ws, evict)
    rows["H8_hierarchical_decode"] = {
        "workload": w.name, "token_budget": T, "coarse_candidate_tokens": w.coarse_candidate_tokens,
        "build_ms": round(build_ms, 2), "us_per_step": round(us, 2), "us_per_step_event_pair": round(us_pair, 2),
        "algorithmic_MB": round(byts / 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(byts / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": _counter_traffic(HIER_TRAFFIC) if p.decode_stages() == ["hier_unit"] else None}}
    log(f"[bench] H8 build {build_ms:.1f} ms, hierarchical decode {us:.1f} us ({byts / 1e6:.1f} MB)")
    del K, V, Kd, Vd, st, ws
    torch.cuda.empty_cache()
    return rows


def _counter_traffic(t, files=("unit.hip", "attn.hpp", "device.hpp", "kernels.hpp")):
    """Counter-derived HBM bytes per launch recorded in t, or None when the
    kernel sources differ from the ones the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_long_context_means_amd", "csrc")
    for fn in t.get("files", files):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != t["sources_sha256"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def _unit_traffic_bytes(fmt):
    """Counter-derived HBM bytes per launch of the per-unit kernel for a
    centroid format, or None (no record, or the sources changed)."""
    t = UNIT_TRAFFIC.get(fmt)
    return None if t is None else _counter_traffic(t)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


if __name__ == "__main__":
    main()
