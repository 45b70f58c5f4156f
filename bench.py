#!/usr/bin/env python3
"""Benchmark of one sparse top-k decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM, all through the C ABI of libsparsekv.so.

Headline workload (the largest single-GPU configuration, token-level
eviction pool): B = 32 sequences, 8 KV heads, G = 1, d = 128, L = 65536
logical tokens of which exactly half are dead (holes scattered inside the
16-token blocks), bf16 keys and values in a pool with permuted blocks reached
through a per-token table, top-k = 2048 over the live tokens plus the first 4
and last 128 live tokens.  Step: score scan (with the first top-k digit) ->
exact top-k -> gather + split attention -> merge.

With the headline, the same JSON line carries `other_configs`, each timed the
same way in the same process (a shorter oracle sample each):
  1   single_head     B=1, L=4096 fp32 contiguous, planted query, top-64
  2   gqa_paged       B=4, 8 KV heads x 4 query heads, L=32768 bf16 paged
                      (seeded block permutation), 4 outlier channels x8,
                      top-2048 + 4 sink + 64 local
  2L  gqa_paged_long  the same at L = 131072
  4   indexer_mla     B=1, indexer keys d=128 + shared latent 576 (value 512),
                      128 query heads, L=131072 paged, top-2048 by the indexer
  5   paris           compressed-code retrieval over 8 x 1,048,060 encoded keys
                      (query LUT, collision vote, top-C, rerank, top-100) + the
                      attention over retrieved + sink 4 + local 512
Other --workload values time one configuration alone (paris_encode: the
off-step encode; paris_decode: the decode loop with the Update Buffer;
compact: token-table compaction; --path prefilter / blocks: the
threshold-prefiltered and block-summary variants).

Successive steps use distinct device copies of the inputs they stream (four
by default, like four layers), so that a step never finds its data in the
256 MB last-level cache left by the step before.  The K timed steps are
captured into one HIP graph and replayed once, as a serving loop would
(--eager launches every kernel from the host instead).  Per-call durations
come from HIP events: with --eager inside the timed region; otherwise from a
second graph of the same K steps with event-record nodes around each call,
replayed right after the timed one (event nodes cost about 14 us per step on
this runtime, so the timed graph carries none).

Prints ONE JSON line (rank 0, N = 1) with the throughput in keys per second,
the per-step time, the roofline entry of the dominant kernel (its HBM traffic
from the committed rocprofv3 counter record when that was taken on the
kernel's current source) and the CPU oracle timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kv-copies C]
                  [--path fused|separate|prefilter|blocks] [--eager]
                  [--no-cpu-baseline] [--no-other-configs]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
DENSE = ("gqa_paged", "gqa_paged_long", "token_pool", "single_head", "indexer_mla")
WORKLOADS = DENSE + ("paris", "paris_encode", "paris_decode", "compact")
PARIS_UPDATE = 512      # Update Buffer tokens (the page's experiments use 256 or 512)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; paris_decode: 4 x 512, one Update Buffer "
                         "cycle of each of the four layers)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10; paris_decode 16)")
    ap.add_argument("--workload", default="token_pool", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="with the headline workload: skip the other configurations")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle sample length of the headline (other configurations: a "
                         "third of it)")
    ap.add_argument("--kv-copies", type=int, default=4,
                    help="distinct device copies of the streamed inputs, used in turn by "
                         "successive steps (like successive layers), so that no step finds "
                         "its data in the 256 MB last-level cache")
    ap.add_argument("--path", default="fused", choices=("fused", "separate", "prefilter", "blocks"),
                    help="dense workloads: fused = sparsekv_score_hist + "
                         "sparsekv_select_attend_resume (top-k fused with the attention); "
                         "separate = sparsekv_score_hist + sparsekv_topk_resume + "
                         "sparsekv_gather_attend (always used where the fused call does not "
                         "support the shape); prefilter = sparsekv_score_prefilter + "
                         "sparsekv_topk_prefiltered (threshold predicted by the EMA of the "
                         "previous steps' k-th scores) + sparsekv_gather_attend")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host instead of replaying one HIP graph "
                         "that holds the K timed steps")
    ap.add_argument("--no-stream-reference", action="store_true",
                    help="skip the streaming-read reference measured after the timed steps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    decode = args.workload == "paris_decode"
    if args.steps is None:
        args.steps = 4 * PARIS_UPDATE if decode else 50
    if args.warmup is None:
        args.warmup = 16 if decode else 10
    return args


class HipEvents:
    """HIP events through the runtime torch already loaded.  graph_record()
    inserts an event-record node into the graph being captured on the
    current stream (torch does not offer external events on ROCm)."""

    def __init__(self):
        import ctypes
        import torch
        self.ct = ctypes
        self.torch = torch
        self.lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, rc))

    def _stream(self):
        return self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def create(self):
        e = self.ct.c_void_p()
        self._ok(self.lib.hipEventCreate(self.ct.byref(e)), "hipEventCreate")
        return e

    def record(self, e):
        self._ok(self.lib.hipEventRecord(e, self._stream()), "hipEventRecord")

    def graph_record(self, e):
        ct, s = self.ct, self._stream()
        status, cid, graph = ct.c_int(), ct.c_ulonglong(), ct.c_void_p()
        deps, nd = ct.POINTER(ct.c_void_p)(), ct.c_size_t()
        self._ok(self.lib.hipStreamGetCaptureInfo_v2(s, ct.byref(status), ct.byref(cid), ct.byref(graph),
                                                     ct.byref(deps), ct.byref(nd)),
                 "hipStreamGetCaptureInfo_v2")
        if status.value != 1:
            raise RuntimeError("graph_record outside a stream capture")
        node = ct.c_void_p()
        self._ok(self.lib.hipGraphAddEventRecordNode(ct.byref(node), graph, deps, nd, e),
                 "hipGraphAddEventRecordNode")
        # the new node becomes the only dependency of what is captured next
        self._ok(self.lib.hipStreamUpdateCaptureDependencies(s, ct.byref(node), ct.c_size_t(1), 1),
                 "hipStreamUpdateCaptureDependencies")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        self._ok(self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value


def timed_steps(step, n_calls, args, hip):
    """Warm up, then time exactly args.steps calls of step(i, mark).  step
    calls mark(j) after its j-th ABI call (j = 0 .. n_calls - 1).  Returns wall seconds of the timed region, GPU ms per step
    between events bracketing it, and per-call ms [steps][n_calls]."""
    import torch
    K = args.steps
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    evs = [[hip.create() for _ in range(n_calls + 1)] for _ in range(K)]
    bracket = [hip.create(), hip.create()]

    def marker(i, in_graph):
        rec = hip.graph_record if in_graph else hip.record
        return lambda j: rec(evs[i][j + 1])

    def run(i, in_graph):
        # evs[i][0] opens the step; step() marks the end of each of its calls
        (hip.graph_record if in_graph else hip.record)(evs[i][0])
        step(i, marker(i, in_graph))

    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.record(bracket[0])
        for i in range(K):
            run(i, False)
        hip.record(bracket[1])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        note = "per-call events recorded inside the timed region"
    else:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0, None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph, graph_ev = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i, None)
        with torch.cuda.graph(graph_ev):
            for i in range(K):
                run(i, True)
        graph.replay()
        torch.cuda.synchronize()
        # timed region: exactly K steps (one replay), synchronised on both sides
        t0 = time.perf_counter()
        hip.record(bracket[0])
        graph.replay()
        hip.record(bracket[1])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ev.replay()
        torch.cuda.synchronize()
        note = ("per-call events from a replay of the same K steps with event-record graph "
                "nodes, right after the timed replay")
    calls = [[hip.elapsed_ms(evs[i][j], evs[i][j + 1]) for j in range(n_calls)] for i in range(K)]
    return wall, hip.elapsed_ms(bracket[0], bracket[1]) / K, calls, note


# Source files that define each timed kernel: a counter record counts only
# while these files are byte-identical to the ones it was taken on.
CSRC = "sparse_top_kv_indexer_amd/csrc/"
_COMMON = [CSRC + "skv_device.h", CSRC + "skv_internal.h"]
_SEL = [CSRC + "skv_rowsel.h", CSRC + "skv_topk.h"]
_SCAN = [CSRC + "score.hip", CSRC + "skv_topk.h"] + _COMMON
_TOPK = [CSRC + "topk.hip", CSRC + "skv_listsel.h"] + _SEL + _COMMON
_ATT = [CSRC + "attend.hip", CSRC + "skv_topk.h"] + _COMMON
_MLA = [CSRC + "mla.hip", CSRC + "skv_listsel.h"] + _SEL + _COMMON
_PARIS = [CSRC + "paris.hip", "include/sparsekv.h"] + _SEL + _COMMON
KERNEL_SOURCES = {
    "score_stream_kernel": _SCAN, "score_valu_kernel": _SCAN,
    "topk_alone_kernel": _TOPK, "topk_compact_kernel": _TOPK, "topk_finish_kernel": _TOPK,
    "topk_hist_kernel": _TOPK, "topk_survivor_kernel": _TOPK,
    "attend_mfma_kernel": _ATT, "attend_split_kernel": _ATT, "attend_reduce_kernel": _ATT,
    "select_attend_kernel": [CSRC + "select_attend.hip", CSRC + "skv_listsel.h"] + _SEL + _COMMON,
    "finish_attend_kernel": [CSRC + "select_attend.hip", CSRC + "skv_listsel.h"] + _SEL + _COMMON,
    "mla_split_kernel": _MLA, "mla_list_kernel": _MLA,
    "query_lut_kernel": _PARIS, "vote_kernel": _PARIS, "cand_write_kernel": _PARIS,
    "rerank_kernel": _PARIS, "encode_kernel": _PARIS,
}


def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(HERE, f), "rb").read())
    return h.hexdigest()


def time_isolated(call, args, hip):
    """Mean duration of one launch of a call (its kernels only), ms: the
    call(i) of args.steps steps captured back to back in one HIP graph
    (rotating over the same input copies as the step), replayed once to
    warm up, then once between two events.  No event node sits between the
    launches, so the figure carries the kernels and the boundaries between
    them, not the event overhead of the per-call timing."""
    import torch
    K = args.steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = hip.create(), hip.create()
    hip.record(e0)
    g.replay()
    hip.record(e1)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1) / K
    del g
    return ms


def traffic_entry(workload, kernels):
    """HBM bytes per launch of the named kernels (summed), from the committed
    rocprofv3 counter record of the workload (profiles/pmc_<workload>.json),
    if every one was taken on the kernel's current source files; else None."""
    path = os.path.join(HERE, "profiles", "pmc_%s.json" % workload)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))["kernels"]
        total = 0.0
        for k in kernels:
            e = rec[k]
            if e["source_sha256"] != sources_sha256(KERNEL_SOURCES[k]):
                return None
            total += e["hbm_bytes_per_launch"]
        return total
    except (KeyError, ValueError, OSError):
        return None


def base_record(metric, value, unit, args, ms_per_step, dtype, config):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded, shaped like the pages' workloads)", "config": config}


def roofline(kernel, bound, alg, seconds, traffic, extra=None):
    if bound == "hbm":
        achieved, peak, unit = alg / seconds / 1e9, PEAK_HBM_GBPS, "GB/s"
    else:
        achieved, peak, unit = alg / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    r = {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
         "frac": achieved / peak, "traffic": traffic}
    if extra:
        r.update(extra)
    return r


def stream_reference():
    """Streaming rates measured on this GPU, a second yardstick beside the
    8 TB/s peak: the library's read probe over 2 GiB in grid-stride order
    (reads only; plain and non-temporal loads, best over a few grid sizes),
    the same 2 GiB as 4 KB pieces in a seeded random order (the access
    pattern of a scan over a pool of 4 KB runs in permuted block order), and
    torch's 1 GiB device copy (reads + writes), best of 10 runs each."""
    import torch
    n = (2 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(12345)
    order = torch.randperm((2 << 30) // 4096, generator=g).to(torch.int32).cuda()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(10):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return nbytes / min(t) / 1e9

    from sparse_top_kv_indexer_amd import yardstick as Y
    grids = (1024, 2048, 4096, 8192)
    plain = max(best(lambda: Y.read_probe(x, gr, sink), 4 * n) for gr in grids)
    nt = max(best(lambda: Y.read_probe(x, gr, sink, nontemporal=True), 4 * n) for gr in grids)
    pieces = max(best(lambda: Y.read_pieces(x, order, gr, sink), 4 * n) for gr in grids)
    copy = best(lambda: y.copy_(x[: n // 2]), 2 * 4 * (n // 2))
    del x, y, sink, order
    torch.cuda.empty_cache()
    return {"stream_read_GBps": max(plain, nt), "stream_read_plain_GBps": plain,
            "stream_read_nontemporal_GBps": nt, "read_4k_pieces_random_GBps": pieces,
            "stream_copy_GBps": copy,
            "stream_note": "skv_read_probe_ex (libskv_yardstick) over 2 GiB in grid-stride order "
                           "(reads only, plain and non-temporal loads, best grid of 1024..8192 "
                           "workgroups); skv_read_pieces over the same 2 GiB as 4 KB pieces in a "
                           "seeded random order; a torch 1 GiB device copy (read + write); best of 10"}


def host_cpu():
    """The host the oracle ran on: CPU model and the cores this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def step_percentiles(calls):
    """p10 / p50 / p90 of the per-step GPU time (sum of a step's call events), us."""
    import numpy as np
    t = np.asarray(calls).sum(axis=1) * 1e3
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)),
            "p90": float(np.percentile(t, 90))}


# ------------------------------------------------------------------ dense
def make_dense(name):
    import workloads as W
    return {"gqa_paged": W.make_gqa_paged, "token_pool": W.make_token_pool,
            "gqa_paged_long": lambda: W.make_gqa_paged(L=131072),
            "single_head": W.make_single_head, "indexer_mla": W.make_indexer_mla}[name]()


def dense_cpu_baseline(st, min_seconds=10.0):
    """The oracle as it stands on (sequence, KV head) rows of the same
    workload, taken in order and repeated until at least min_seconds of CPU
    work: float64 scores, full sort, dense masked softmax."""
    import workloads as W
    from oracle import dense as D
    from threadpoolctl import threadpool_info
    kv = st.score_kv
    live = [W.live_tokens(kv, b) for b in range(kv.B)]
    rows = [(b, h) for b in range(kv.B) for h in range(kv.H)]
    keys = 0
    n_rows = 0
    t0 = time.perf_counter()
    while True:
        b, h = rows[n_rows % len(rows)]
        D.step(st, rows=[(b, h)])
        keys += int(live[b].size)
        n_rows += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max([1] + blas)
    return {"value": keys / dt, "unit": "keys/s", "cores": cores, "kind": "oracle", **host_cpu(),
            "sample": "%d (sequence, KV head) rows of the same workload in order (%d keys), %.1f s; "
                      "numpy float64, BLAS threads=%d, other ops single-threaded"
                      % (n_rows, keys, dt, cores)}


def bench_dense(args, hip):
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    dev = torch.device("cuda:0")
    st = make_dense(args.workload)
    mla = st.kv.v is None
    kv = S.kv_to_device(st.kv, dev)
    skv = kv if st.score_kv is st.kv else S.kv_to_device(st.score_kv, dev)
    bf = st.kv.dtype == "bf16"
    q = S.to_device(st.q, dev, bf)
    sq = q if st.score_q is st.q else S.to_device(st.score_q, dev, st.score_kv.dtype == "bf16")
    lo = S.to_device(st.lo.astype(np.int32), dev)
    hi = S.to_device(st.hi.astype(np.int32), dev)
    B, H, L, k = skv.B, skv.H, skv.L_max, st.k
    G, sG = st.G, st.score_G
    scores = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    out = torch.empty((kv.B, kv.H * G, kv.d_v), dtype=torch.float32, device=dev)
    # fused: sparsekv_score_hist + sparsekv_select_attend_resume -- the top-k
    # finished inside the attention kernel (GQA rows of any length, k <= 4096
    # beyond one 32768-slot sweep; the latent attention)
    fused = args.path == "fused" and (mla or (skv is kv and sG == G and bf and kv.d_k == 128
                                              and G <= 8 and (L <= 32768 or k <= 4096)))
    prefilter = args.path == "prefilter"
    blocks = args.path == "blocks"
    if blocks:
        return bench_blocks(args, hip, st, kv, q, lo, hi)
    # long rows with k <= 2048: the scan lists segment candidates and the
    # selecting kernel takes them (sparsekv_score_segments +
    # sparsekv_select_attend_segments); else the histogram scan + resume
    seg = fused and S.sparsekv_segments(kv, G, k) > 0
    thr = torch.full((B, H), float("-inf"), dtype=torch.float32, device=dev)
    used = torch.zeros((B, H), dtype=torch.int32, device=dev)
    if fused:
        ws_sel = S.workspace(max(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, kv, G, k),
                                 S.sparsekv_workspace_size(S.SKV_OP_SELECT, skv, sG, k)), dev)
        ws_att = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, G, k), dev)
    else:
        ws_sel = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT, skv, sG, k), dev)
        ws_att = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, G, k), dev)

    def copy_kv(t):
        return dataclasses.replace(t, k=t.k.clone(), v=None if t.v is None else t.v.clone())

    pairs = [(skv, kv)]
    for _ in range(max(1, args.kv_copies) - 1):
        c = copy_kv(kv)
        pairs.append((c if skv is kv else copy_kv(skv), c))

    def step(i, mark):
        s_kv, a_kv = pairs[i % len(pairs)]
        if prefilter:
            S.sparsekv_score_prefilter(s_kv, sq, sG, lo, hi, thr, scores, ws_sel)
        elif seg:
            S.sparsekv_score_segments(s_kv, sq, sG, lo, hi, k, scores, ws_sel)
        else:
            S.sparsekv_score_hist(s_kv, sq, sG, lo, hi, scores, ws_sel)
        if mark:
            mark(0)
        if prefilter:
            S.sparsekv_topk_prefiltered(scores, lo, hi, k, thr, idx, cnt, ws_sel, used=used)
            if mark:
                mark(1)
            S.sparsekv_gather_attend(a_kv, q, G, idx, k, lo, hi, st.scale, out, ws_att)
        elif seg:
            S.sparsekv_select_attend_segments(a_kv, q, G, lo, hi, k, st.scale, scores, idx, cnt,
                                              out, ws_sel)
        elif fused:
            S.sparsekv_select_attend_resume(a_kv, q, G, lo, hi, k, st.scale, scores, idx, cnt, out,
                                            ws_sel)
        else:
            S.sparsekv_topk_resume(scores, lo, hi, k, idx, cnt, ws_sel)
            if mark:
                mark(1)
            S.sparsekv_gather_attend(a_kv, q, G, idx, k, lo, hi, st.scale, out, ws_att)
        if mark:
            mark(1 if fused else 2)

    wall, gpu_ms, calls, note = timed_steps(step, 2 if fused else 3, args, hip)
    calls = np.array(calls)
    ms_per_step = wall * 1e3 / args.steps
    # the dominant kernel alone: the scan with its histogram, on a workspace
    # of its own (the histograms accumulate over the repeated launches)
    ws_iso = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT, skv, sG, k), dev)
    if prefilter:
        thr_iso = thr.clone()
        scan_iso_ms = time_isolated(
            lambda i: S.sparsekv_score_prefilter(pairs[i % len(pairs)][0], sq, sG, lo, hi, thr_iso,
                                                 scores, ws_iso), args, hip)
    elif seg:
        scan_iso_ms = time_isolated(
            lambda i: S.sparsekv_score_segments(pairs[i % len(pairs)][0], sq, sG, lo, hi, k, scores,
                                                ws_iso), args, hip)
    else:
        scan_iso_ms = time_isolated(
            lambda i: S.sparsekv_score_hist(pairs[i % len(pairs)][0], sq, sG, lo, hi, scores,
                                            ws_iso), args, hip)
    del ws_iso
    att_iso_ms = None
    if mla:
        att_iso_ms = time_isolated(
            lambda i: S.sparsekv_gather_attend(pairs[i % len(pairs)][1], q, G, idx, k, lo, hi,
                                               st.scale, out, ws_att), args, hip)
    # live keys and algorithmic bytes of the scan and the gather, counted
    # from the workload's own tables
    import workloads as W
    live = [W.live_tokens(st.score_kv, b) for b in range(B)]
    n_keys = sum(int(t.size) for t in live) * H
    es = 2 if st.score_kv.dtype == "bf16" else 4
    per_key = st.score_kv.d_k * es + 4 + (4 if st.score_kv.token_table is not None else 0)
    scan_bytes = n_keys * per_key + sq.numel() * sq.element_size()
    cnt_np = cnt.cpu().numpy()
    n_att = int(cnt_np.sum())
    for b in range(B):
        t_live = W.live_tokens(st.kv, b)
        n_att += int(((t_live < st.lo[b]) | (t_live >= st.hi[b])).sum()) * kv.H
    # per attended token: its K and V rows (the latent row once); the fused
    # call with one query head takes the logit from the scan's score instead
    # of the K row
    if mla:
        row_bytes = kv.d_k * (2 if bf else 4)
    elif fused and G == 1:
        row_bytes = kv.d_v * (2 if bf else 4) + 4
    else:
        row_bytes = 2 * kv.d_k * (2 if bf else 4)
    gather_bytes = n_att * row_bytes
    step_bytes = scan_bytes + gather_bytes
    scan_s = scan_iso_ms * 1e-3
    kname = ("score_stream_kernel" if (bf and skv.d_k % 32 == 0 and skv.d_k <= 256) else
             "score_valu_kernel")
    # the counter record holds the histogram scan; the survivor scan has none
    tr = None if prefilter else traffic_entry(args.workload, [kname])
    cfg = {"workload": args.workload, "B": B, "H_kv": kv.H, "G": G, "d": kv.d_k,
           "L": L, "k": k, "layout": st.kv.mode, "kv_dtype": st.kv.dtype,
           "kv_copies": len(pairs), "launch": "eager" if args.eager else "hip_graph",
           "path": "fused" if fused else ("prefilter" if prefilter else "separate"),
           "candidates": ("scan segments (%d per row)" % S.sparsekv_segments(kv, G, k) if seg else
                          "key histogram" if not prefilter else "predicted threshold")}
    if args.workload != "indexer_mla":
        cfg.update(sink=int(st.lo[0]), local=int(st.kv.seq_len[0] - st.hi[0]))
    else:
        cfg.update(d_latent=kv.d_k, d_value=kv.d_v, d_indexer=skv.d_k)
    rec = base_record("history keys scanned/s (one sparse top-k decode step of one layer)",
                      n_keys / (ms_per_step * 1e-3), "keys/s", args, ms_per_step,
                      "bf16" if bf else "f32", cfg)
    rec.update({
        "us_per_step": ms_per_step * 1e3,
        "us_per_step_gpu": gpu_ms * 1e3,
        "timing": note,
        "us_per_step_events": step_percentiles(calls),
        "us_per_call": ({"score_scan": float(np.mean(calls[:, 0])) * 1e3,
                         "select_attend_merge": float(np.mean(calls[:, 1])) * 1e3} if fused else
                        {"score_scan": float(np.mean(calls[:, 0])) * 1e3,
                         "topk": float(np.mean(calls[:, 1])) * 1e3,
                         "gather_attend": float(np.mean(calls[:, 2])) * 1e3}),
        "keys_scanned_per_step": n_keys,
        **({"prefilter_rows_from_survivors": float(used.float().mean().item()),
            "prefilter_note": "the same query every step, so after the first step the "
                              "predicted threshold is the exact k-th score"}
           if prefilter else {}),
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": roofline(("score scan (sparsekv_score_prefilter: %s listing the keys above "
                              "the predicted threshold)" if prefilter else
                              "score scan (sparsekv_score_segments: %s listing segment candidates)"
                              if seg else
                              "score scan (sparsekv_score_hist: %s with the fused top-k histogram)")
                             % kname, "hbm", scan_bytes, scan_s, tr,
                             {"algorithmic_bytes_per_launch": scan_bytes, "bytes_per_key": per_key,
                              "us_per_launch": scan_iso_ms * 1e3,
                              "timing": "isolated replay of %d back-to-back launches" % args.steps}),
    })
    if mla:
        # the latent attention is a dense contraction on matrix cores:
        # per selected token and head, 576 + 512 multiply-adds (the isolated
        # timing is of sparsekv_gather_attend over the step's selection)
        att_s = att_iso_ms * 1e-3
        flops = 2.0 * n_att * G * (kv.d_k + kv.d_v)
        rec["roofline_attention"] = roofline("latent attention (sparsekv_gather_attend: "
                                             "mla_split_kernel + merge)", "mfma", flops, att_s,
                                             traffic_entry(args.workload, ["mla_split_kernel",
                                                                           "attend_reduce_kernel"]),
                                             {"algorithmic_flops_per_launch": flops,
                                              "gathered_bytes": gather_bytes,
                                              "us_per_launch": att_iso_ms * 1e3,
                                              "timing": "isolated replay of %d back-to-back "
                                                        "launches" % args.steps})
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = dense_cpu_baseline(st, args.cpu_seconds)
    return rec


def bench_blocks(args, hip, st, kv, q, lo, hi):
    """Block-summary step: re-summarise the block of each sequence's last
    token, scan the summaries (Quest's bound per 16-token block), exact top-K
    blocks (K = k / 16) and their tokens (one call), then gather + attention
    with sink and local.  The summary pools of the KV copies are built before
    timing."""
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    dev = q.device
    B, H, G, L, k = kv.B, kv.H, st.G, kv.L_max, st.k
    K = k // 16
    bsc = torch.empty((B, H, L // 16), dtype=torch.float32, device=dev)
    bidx = torch.empty((B, H, K), dtype=torch.int32, device=dev)
    bcnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    tok = torch.empty((B, H, 16 * K), dtype=torch.int32, device=dev)
    out = torch.empty((B, H * G, kv.d_v), dtype=torch.float32, device=dev)
    ws_blk = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_BLOCK_SELECT, kv, G, K), dev)
    ws_att = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, G, 16 * K), dev)
    copies = [kv] + [dataclasses.replace(kv, k=kv.k.clone(), v=kv.v.clone())
                     for _ in range(max(1, args.kv_copies) - 1)]
    pools = []
    for c in copies:
        summ = S.block_summary_pool(c)
        for b in range(B):
            S.sparsekv_block_summarize(c, b, 0, L // 16, summ)
        pools.append(summ)
    torch.cuda.synchronize()

    def step(i, mark):
        c, summ = copies[i % len(copies)], pools[i % len(copies)]
        # re-summarises each sequence's last block, then scans, selects, expands
        S.sparsekv_block_select(c, summ, q, G, lo, hi, K, bsc, bidx, bcnt, tok, ws_blk)
        if mark:
            mark(0)
        S.sparsekv_gather_attend(c, q, G, tok, 16 * K, lo, hi, st.scale, out, ws_att)
        if mark:
            mark(1)

    wall, gpu_ms, calls, note = timed_steps(step, 2, args, hip)
    calls = np.array(calls)
    ms_per_step = wall * 1e3 / args.steps
    import workloads as W
    live = [W.live_tokens(st.kv, b) for b in range(B)]
    n_keys = sum(int(t.size) for t in live) * H
    n_blocks = sum(int(np.unique(t // 16).size) for t in live) * H
    # per live block row: the [mx, mn] summary, its score and its table entry
    per_block = 2 * kv.d_k * 2 + 4 + 4
    scan_bytes = n_blocks * per_block + B * H * G * 2 * kv.d_k * 2
    tok_np = tok.cpu().numpy()
    n_att = int((tok_np >= 0).sum())
    for b in range(B):
        n_att += int(((live[b] < st.lo[b]) | (live[b] >= st.hi[b])).sum()) * H
    gather_bytes = n_att * kv.d_k * 2 * 2
    sel_s = float(np.mean(calls[:, 0])) * 1e-3
    cfg = {"workload": args.workload, "B": B, "H_kv": H, "G": G, "d": kv.d_k, "L": L,
           "k": k, "K_blocks": K, "layout": st.kv.mode, "kv_dtype": st.kv.dtype,
           "kv_copies": len(copies), "launch": "eager" if args.eager else "hip_graph",
           "path": "blocks", "sink": int(st.lo[0]), "local": int(st.kv.seq_len[0] - st.hi[0])}
    rec = base_record("history keys ranked/s (block-summary sparse decode step of one layer)",
                      n_keys / (ms_per_step * 1e-3), "keys/s", args, ms_per_step, "bf16", cfg)
    rec.update({
        "us_per_step": ms_per_step * 1e3,
        "us_per_step_gpu": gpu_ms * 1e3,
        "timing": note,
        "us_per_step_events": step_percentiles(calls),
        "us_per_call": {"block_select": float(np.mean(calls[:, 0])) * 1e3,
                        "gather_attend": float(np.mean(calls[:, 1])) * 1e3},
        "keys_covered_per_step": n_keys,
        "live_block_rows_per_step": n_blocks,
        "tokens_attended_per_step": n_att,
        "step_algorithmic_bytes": scan_bytes + gather_bytes,
        "roofline": roofline("block selection (sparsekv_block_select: summary scan, top-K "
                             "blocks, expansion)", "hbm", scan_bytes, sel_s, None,
                             {"algorithmic_bytes_per_launch": scan_bytes,
                              "bytes_per_block_row": per_block}),
    })
    return rec


# ------------------------------------------------------------------ paris
RETRIEVE_KERNELS = ("query_lut_kernel", "vote_kernel", "cand_write_kernel", "rerank_kernel",
                    "topk_alone_kernel")


def paris_cpu_baseline(min_seconds):
    """The oracle's encode + retrieval on a bounded sample of the same
    workload: one KV head (4 query heads) of a 65,536-token history drawn the
    same way, repeated until at least min_seconds of CPU work."""
    import workloads as W
    from oracle import lloyd
    from oracle import paris as P
    p = W.make_paris(tag=55, H=1, L=65536 + 516)
    lv, th = lloyd.codebook_f32(8)
    n_runs = 0
    t0 = time.perf_counter()
    while True:
        P.retrieve(p, P.build_index(p, lv, th), lv)
        n_runs += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    from threadpoolctl import threadpool_info
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max([1] + blas)
    return {"value": n_runs * p.H * p.n / dt, "unit": "keys/s", "cores": cores, "kind": "oracle",
            **host_cpu(),
            "sample": "%d x (encode + retrieve) of 1 KV head x %d keys of the same distribution, "
                      "%.1f s; numpy fp32 in the prescribed operation order, BLAS threads=%d"
                      % (n_runs, p.n, dt, cores)}


PARIS_RHOS = (0.02, 0.05, 0.10)   # tier budgets rho reported (beta = 0.02)


def paris_recall(p, cb, index, kv, q, dev):
    """recall@100 of the retrieval at each rho of PARIS_RHOS, against the
    exact top-100 of max_g q_g . k over the index region computed by the
    library's own exact path (sparsekv_score + sparsekv_topk), mean over the
    KV heads."""
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    qa = q.view(1, p.H * p.G, p.d)
    sc = S.sparsekv_score(kv, qa, p.G)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=dev)
    hi = torch.tensor([p.L - p.local], dtype=torch.int32, device=dev)
    true_idx, _ = S.sparsekv_topk(sc, lo, hi, p.k_final)
    true_idx = true_idx.cpu().numpy()[0]
    out = {}
    for rho in PARIS_RHOS:
        idx, n_cand, _ = S.sparsekv_retrieve(cb, index, q, p.G, rho, p.beta, p.k_final)
        got = idx.cpu().numpy()
        r = [len(set(got[h].tolist()) & set(true_idx[h].tolist())) / p.k_final for h in range(p.H)]
        out[repr(rho)] = float(np.mean(r))
    del sc
    return out


def bench_paris(args, hip):
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    import workloads as W
    dev = torch.device("cuda:0")
    p = W.make_paris()
    cb = S.new_codebook(torch.from_numpy(p.signs).to(dev))
    kv = S.kv_to_device(p.kv(), dev)
    encode_only = args.workload == "paris_encode"
    indexes = [S.new_index(p.H, p.n, device=dev) for _ in range(max(1, args.kv_copies)
                                                              if encode_only else 1)]
    for ix in indexes:
        S.sparsekv_encode(cb, kv, 0, p.sink, p.L - p.local, ix)
    torch.cuda.synchronize()
    if encode_only:
        kvs = [kv] + [dataclasses.replace(kv, k=kv.k.clone(), v=None)
                      for _ in range(max(1, args.kv_copies) - 1)]

        def step(i, mark):
            ix = indexes[i % len(indexes)]
            ix.n = 0
            S.sparsekv_encode(cb, kvs[i % len(kvs)], 0, p.sink, p.L - p.local, ix)
            if mark:
                mark(0)

        wall, gpu_ms, calls, note = timed_steps(step, 1, args, hip)
        ms = wall * 1e3 / args.steps
        n = p.H * p.n
        # per key: 256 B row in; 16 B ids + 64 B codes + 64 B w out
        alg = n * (256 + 16 + 64 + 64)
        t_s = float(np.mean(np.array(calls)[:, 0])) * 1e-3
        rec = base_record("keys encoded/s (compressed-code index build, off the decode step)",
                          n / (ms * 1e-3), "keys/s", args, ms, "f32",
                          {"workload": "paris_encode", "H_kv": p.H, "d": p.d, "L": p.L, "n": p.n,
                           "n_sub": p.n_sub, "m": p.m, "copies": len(kvs),
                           "launch": "eager" if args.eager else "hip_graph"})
        rec.update({"us_per_step": ms * 1e3, "us_per_step_gpu": gpu_ms * 1e3, "timing": note,
                    "roofline": roofline("encode (sparsekv_encode: encode_kernel)", "hbm", alg, t_s,
                                         None, {"algorithmic_bytes_per_launch": alg,
                                                "bytes_per_key": 400})})
        return rec

    # retrieval step: index copies (the id arrays, 134 MB, would otherwise sit
    # in the last-level cache) and the attention over the result
    base = indexes[0]
    ixs = [base]
    for _ in range(max(1, args.kv_copies) - 1):
        ixs.append(dataclasses.replace(base, ids=base.ids.clone(), cw=base.cw.clone(),
                                       hist=base.hist.clone(), pos=base.pos.clone()))
    kvs = [kv] + [dataclasses.replace(kv, k=kv.k.clone(), v=kv.v.clone())
                  for _ in range(max(1, args.kv_copies) - 1)]
    q = S.to_device(p.q, dev, bf16=True)
    qa = q.view(1, p.H * p.G, p.d)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=dev)
    hi = torch.tensor([p.L - p.local], dtype=torch.int32, device=dev)
    ridx = torch.empty((p.H, p.k_final), dtype=torch.int32, device=dev)
    ncand = torch.empty((p.H,), dtype=torch.int32, device=dev)
    out = torch.empty((1, p.H * p.G, p.d), dtype=torch.float32, device=dev)
    ws_r = S.workspace(S.retrieve_workspace_size(base, p.G, p.beta, p.k_final), dev)
    ws_a = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, p.G, p.k_final), dev)

    def step(i, mark):
        S.sparsekv_retrieve(cb, ixs[i % len(ixs)], q, p.G, p.rho, p.beta, p.k_final, idx=ridx,
                            n_cand=ncand, ws=ws_r)
        if mark:
            mark(0)
        S.sparsekv_gather_attend(kvs[i % len(kvs)], qa, p.G, ridx.view(1, p.H, -1), p.k_final, lo, hi,
                                 p.scale, out, ws_a)
        if mark:
            mark(1)

    wall, gpu_ms, calls, note = timed_steps(step, 2, args, hip)
    calls = np.array(calls)
    ms = wall * 1e3 / args.steps
    ret_iso_ms = time_isolated(
        lambda i: S.sparsekv_retrieve(cb, ixs[i % len(ixs)], q, p.G, p.rho, p.beta, p.k_final,
                                      idx=ridx, n_cand=ncand, ws=ws_r), args, hip)
    recall = paris_recall(p, cb, base, kv, q, dev)
    n_keys = p.H * p.n
    C = int(math.ceil(p.beta * p.n))
    ret_bytes = n_keys * 16 + p.H * C * 128      # ids scanned + codes and w of the candidates
    gather = p.H * (p.k_final + p.sink + p.local) * 512
    t_ret = ret_iso_ms * 1e-3
    rec = base_record("history keys voted/s (one compressed-code retrieval decode step)",
                      n_keys / (ms * 1e-3), "keys/s", args, ms, "u8/f32",
                      {"workload": "paris", "B": 1, "H_kv": p.H, "G": p.G, "d": p.d, "L": p.L,
                       "n": p.n, "beta": p.beta, "rho": p.rho, "C": C, "k_final": p.k_final,
                       "sink": p.sink, "local": p.local, "copies": len(ixs),
                       "launch": "eager" if args.eager else "hip_graph"})
    rec.update({
        "us_per_step": ms * 1e3, "us_per_step_gpu": gpu_ms * 1e3, "timing": note,
        "us_per_step_events": step_percentiles(calls),
        "us_per_call": {"retrieve": float(np.mean(calls[:, 0])) * 1e3,
                        "gather_attend": float(np.mean(calls[:, 1])) * 1e3},
        "keys_voted_per_step": n_keys,
        "recall_at_100": recall,
        "step_algorithmic_bytes": ret_bytes + gather,
        "step_GBps": (ret_bytes + gather) / (ms * 1e-3) / 1e9,
        "roofline": roofline("retrieval (sparsekv_retrieve: query LUT, collision vote, top-C, "
                             "rerank, top-100; the vote kernel moves 94 % of the bytes)", "hbm",
                             ret_bytes, t_ret, traffic_entry("paris", RETRIEVE_KERNELS),
                             {"algorithmic_bytes_per_launch": ret_bytes,
                              "traffic_kernels": list(RETRIEVE_KERNELS),
                              "us_per_launch": ret_iso_ms * 1e3,
                              "timing": "isolated replay of %d back-to-back launches"
                                        % args.steps}),
    })
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = paris_cpu_baseline(args.cpu_seconds)
    return rec


def bench_paris_decode(args, hip):
    """Multi-step decode over the compressed path with the Update Buffer.
    Four layers (index and KV copies) append the same token each decode
    step; a timed step is one layer's work: sparsekv_update_buffer (encodes
    512 tokens into that layer's index when its buffer is full, else nothing),
    sparsekv_retrieve over the index as it stands, sparsekv_gather_attend
    over retrieved + sink + Local + buffer.  The prefill leaves the buffers
    so that every layer flushes once inside the timed steps; launched eagerly
    (the flush is a host decision and the index grows between steps)."""
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    import workloads as W
    dev = torch.device("cuda:0")
    p = W.make_paris()
    U = PARIS_UPDATE
    n_layers = max(1, args.kv_copies)
    total = args.warmup + args.steps
    n_tok = (total + n_layers - 1) // n_layers          # tokens appended per layer
    cap = p.L - p.sink - p.local
    # the decode starts from an earlier step's state: the buffer already
    # holds b0 tokens, chosen so that the token appended in the middle of the
    # timed steps fills it
    t_flush = (args.warmup + args.steps // 2) // n_layers + 1
    b0 = max(0, U - t_flush) % U
    L0 = p.L - n_tok
    n0 = L0 - p.sink - p.local - b0
    assert n0 > 0 and n0 + U * ((n_tok + b0) // U) <= cap, "decode does not fit"
    cb = S.new_codebook(torch.from_numpy(p.signs).to(dev))
    kv0 = S.kv_to_device(p.kv(), dev)
    seqs = torch.arange(L0 + 1, L0 + 1 + n_tok, dtype=torch.int32, device=dev)
    kvs = [kv0] + [dataclasses.replace(kv0, k=kv0.k.clone(), v=kv0.v.clone())
                   for _ in range(n_layers - 1)]
    idxs = []
    for c in kvs:
        ix = S.new_index(p.H, cap, device=dev)
        c.seq_len.fill_(L0)
        S.sparsekv_encode(cb, c, 0, p.sink, p.sink + n0, ix)
        idxs.append(ix)
    # per-token retrieval end (host rule, the same for every layer) and its device copy
    n_of = []
    n = n0
    for j in range(n_tok):
        seq = L0 + 1 + j
        if seq - (p.sink + n) >= p.local + U:
            n += U * ((seq - p.sink - n - p.local) // U)
        n_of.append(n)
    his = torch.tensor([p.sink + x for x in n_of], dtype=torch.int32, device=dev)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=dev)
    q = S.to_device(p.q, dev, bf16=True)
    qa = q.view(1, p.H * p.G, p.d)
    ridx = torch.empty((p.H, p.k_final), dtype=torch.int32, device=dev)
    ncand = torch.empty((p.H,), dtype=torch.int32, device=dev)
    out = torch.empty((1, p.H * p.G, p.d), dtype=torch.float32, device=dev)
    ws_r = S.workspace(S.retrieve_workspace_size(dataclasses.replace(idxs[0], n=cap), p.G, p.beta,
                                                 p.k_final), dev)
    ws_a = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv0, p.G, p.k_final), dev)
    torch.cuda.synchronize()
    state = {"call": 0, "flushes": 0, "flush_calls": []}

    def step(i, mark):
        c = state["call"]
        state["call"] += 1
        layer, j = c % n_layers, c // n_layers
        kv = dataclasses.replace(kvs[layer], seq_len=seqs[j:j + 1])
        f = S.sparsekv_update_buffer(cb, kv, 0, L0 + 1 + j, p.sink, p.local, U, idxs[layer])
        assert idxs[layer].n == n_of[j]
        if f:
            state["flushes"] += f
            state["flush_calls"].append((c, i))
        if mark:
            mark(0)
        S.sparsekv_retrieve(cb, idxs[layer], q, p.G, p.rho, p.beta, p.k_final, idx=ridx,
                            n_cand=ncand, ws=ws_r)
        if mark:
            mark(1)
        S.sparsekv_gather_attend(kv, qa, p.G, ridx.view(1, p.H, -1), p.k_final, lo,
                                 his[j:j + 1], p.scale, out, ws_a)
        if mark:
            mark(2)

    args.eager = True
    wall, gpu_ms, calls, note = timed_steps(step, 3, args, hip)
    calls = np.array(calls)
    ms = wall * 1e3 / args.steps
    timed = [i for (c, i) in state["flush_calls"] if c >= args.warmup]
    t_flush_us = float(np.mean(calls[timed, 0])) * 1e3 if timed else None
    keys = p.H * float(np.mean([n_of[(args.warmup + i) // n_layers] for i in range(args.steps)]))
    t_ret = float(np.mean(calls[:, 1])) * 1e-3
    C = int(math.ceil(p.beta * keys / p.H))
    ret_bytes = keys * 16 + p.H * C * 128
    no_flush = [i for i in range(args.steps) if i not in set(timed)]
    step_no_flush_us = float(np.mean(calls[no_flush].sum(axis=1))) * 1e3
    rec = base_record("history keys voted/s (compressed-code decode loop with the Update Buffer)",
                      keys / (ms * 1e-3), "keys/s", args, ms, "u8/f32",
                      {"workload": "paris_decode", "B": 1, "H_kv": p.H, "G": p.G, "d": p.d,
                       "L": p.L, "start_len": L0, "n_start": n0, "buffer_start": b0,
                       "update": U, "beta": p.beta,
                       "rho": p.rho, "k_final": p.k_final, "sink": p.sink, "local": p.local,
                       "layers": n_layers, "tokens_appended": n_tok, "launch": "eager"})
    rec.update({
        "us_per_step": ms * 1e3, "us_per_step_gpu": gpu_ms * 1e3, "timing": note,
        "us_per_step_events": step_percentiles(calls),
        "us_per_call": {"update_buffer_flush": t_flush_us,
                        "retrieve": t_ret * 1e6,
                        "gather_attend": float(np.mean(calls[:, 2])) * 1e3},
        "flushes_in_timed_steps": len(timed),
        "us_per_step_without_flush": step_no_flush_us,
        "us_per_layer_token_amortised": (step_no_flush_us + (t_flush_us or 0.0) / U),
        "roofline": roofline("retrieval (sparsekv_retrieve over the growing index)", "hbm",
                             ret_bytes, t_ret, None, {"algorithmic_bytes_per_launch": ret_bytes}),
    })
    if t_flush_us:
        enc_bytes = p.H * U * (256 + 16 + 64 + 64)
        rec["roofline_flush"] = roofline("flush (sparsekv_update_buffer: encode_kernel over 512 "
                                         "tokens x 8 heads)", "hbm", enc_bytes, t_flush_us * 1e-6,
                                         None, {"algorithmic_bytes_per_launch": enc_bytes})
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = paris_cpu_baseline(args.cpu_seconds)
    return rec


def bench_compact(args, hip):
    """Token-table compaction of the token-pool workload (32 sequences x
    65,536 logical tokens, half of them dead, 8 heads, d = 128) with 2,048
    spare blocks as headroom: the host planner makes one plan per sequence
    (at most 64 source blocks each, theta_F = 0.25), and a timed step applies
    all of them in one sparsekv_compact_apply launch, then the reverse moves
    in a second one (so that every step moves the same tokens); the I1 hash
    and I2 check over the whole pool are timed once each."""
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S
    import workloads as W
    dev = torch.device("cuda:0")
    st = W.make_token_pool(spare_blocks=2048)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    kv_d = S.kv_to_device(kv, dev)
    counts = W.block_occupancy(kv.token_table, kv.seq_len, n_blocks)
    free = [int(x) for x in st.meta["free_blocks"]]
    F_before = S.sparsekv_waste_ratio(counts[counts > 0])
    t0 = time.perf_counter()
    plans = []
    n_freed = n_used = 0
    for b in range(kv.B):
        moves, src, n_dst = S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, b, free,
                                                    len(free), 0.25, 64, counts=counts)
        for p_ in src:
            counts[p_] = 0
        for j, p_ in enumerate(free[:n_dst]):
            counts[p_] = min(16, len(moves) - 16 * j)
        free = free[n_dst:]
        plans.append(moves)
        n_freed += len(src)
        n_used += n_dst
    plan_s = time.perf_counter() - t0
    fwd = np.concatenate(plans)
    rev = fwd[:, [0, 1, 3, 2]].copy()
    n_mv = int(fwd.shape[0])
    fwd_d, rev_d = torch.from_numpy(fwd).to(dev), torch.from_numpy(rev).to(dev)
    h0, c0 = S.sparsekv_live_hash(kv_d)
    torch.cuda.synchronize()
    h0 = h0.clone()

    def step(i, mark):
        S.sparsekv_compact_apply(kv_d, fwd_d)
        if mark:
            mark(0)
        S.sparsekv_compact_apply(kv_d, rev_d)
        if mark:
            mark(1)

    args.eager = True
    wall, gpu_ms, calls, note = timed_steps(step, 2, args, hip)
    calls = np.array(calls)
    ms = wall * 1e3 / args.steps
    # the checks, once each, with events around them
    e = [hip.create() for _ in range(3)]
    hip.record(e[0])
    h1, c1 = S.sparsekv_live_hash(kv_d)
    hip.record(e[1])
    dup = S.sparsekv_check_unique(kv_d, n_blocks)
    hip.record(e[2])
    torch.cuda.synchronize()
    hash_us, uniq_us = hip.elapsed_ms(e[0], e[1]) * 1e3, hip.elapsed_ms(e[1], e[2]) * 1e3
    assert torch.equal(h0, h1) and dup.cpu().tolist() == [0, 0], "compaction broke an invariant"
    row = kv.d_k * 2
    per_move = kv.H * 2 * row * 2 + 16 + 4       # K and V rows read + written, move, table entry
    t_apply = float(np.mean(calls[:, 0])) * 1e-3
    live = int(c1.sum().item())
    hash_bytes = live * kv.H * 2 * row
    F_after = S.sparsekv_waste_ratio(counts[counts > 0])
    rec = base_record("tokens relocated/s (token-table compaction, sparsekv_compact_apply)",
                      2 * n_mv / (ms * 1e-3), "tokens/s", args, ms, "bf16",
                      {"workload": "compact", "B": kv.B, "H_kv": kv.H, "d": kv.d_k, "L": kv.L_max,
                       "dead_frac": 0.5, "spare_blocks": 2048, "max_src": 64, "theta_F": 0.25,
                       "launch": "eager"})
    rec.update({
        "us_per_step": ms * 1e3, "us_per_step_gpu": gpu_ms * 1e3, "timing": note,
        "moves_per_launch": n_mv, "source_blocks_freed": n_freed, "target_blocks_used": n_used,
        "us_per_step_events": step_percentiles(calls),
        "us_per_call": {"apply_forward": t_apply * 1e6,
                        "apply_reverse": float(np.mean(calls[:, 1])) * 1e3,
                        "live_hash_all": hash_us, "check_unique_all": uniq_us},
        "plan_host_ms": plan_s * 1e3,
        "waste_ratio_before": F_before, "waste_ratio_after_one_round": F_after,
        "roofline": roofline("compaction copy (sparsekv_compact_apply)", "hbm", n_mv * per_move,
                             t_apply, None, {"algorithmic_bytes_per_launch": n_mv * per_move,
                                             "bytes_per_move": per_move}),
        "roofline_hash": roofline("I1 hash (sparsekv_live_hash over all live tokens)", "hbm",
                                  hash_bytes, hash_us * 1e-6, None,
                                  {"algorithmic_bytes_per_launch": hash_bytes}),
    })
    return rec


# configurations carried in the headline's line, by the ids the workloads
# are known by (2L: workload 2 at L = 131072)
CONFIG_ID = {"single_head": "1", "gqa_paged": "2", "gqa_paged_long": "2L", "token_pool": "3",
             "indexer_mla": "4", "paris": "5"}
OTHER_CONFIGS = ("single_head", "gqa_paged", "gqa_paged_long", "indexer_mla", "paris")


def run_workload(args, hip):
    if args.workload in DENSE:
        return bench_dense(args, hip)
    if args.workload == "paris_decode":
        return bench_paris_decode(args, hip)
    if args.workload == "compact":
        return bench_compact(args, hip)
    return bench_paris(args, hip)


def add_stream_reference(rec, ref):
    for key in ("roofline", "roofline_attention"):
        ro = rec.get(key)
        if ro and ro.get("bound") == "hbm" and ref:
            ro.update(ref)
            ro["frac_of_stream_read"] = ro["achieved"] / ref["stream_read_GBps"]
            ro["frac_of_4k_pieces_read"] = ro["achieved"] / ref["read_4k_pieces_random_GBps"]


def summary(rec):
    """The entry of one configuration in other_configs: time per step, step
    and dominant-kernel rates against the peaks, and the oracle baseline."""
    keep = ("metric", "value", "unit", "dtype", "config", "us_per_step", "us_per_step_gpu",
            "us_per_step_events", "us_per_call", "step_algorithmic_bytes", "step_GBps",
            "step_frac_of_hbm_peak", "roofline", "roofline_attention", "cpu_baseline")
    out = {k: rec[k] for k in keep if k in rec}
    if "step_GBps" in out and "step_frac_of_hbm_peak" not in out:
        out["step_frac_of_hbm_peak"] = out["step_GBps"] / PEAK_HBM_GBPS
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the single-GPU hot path only; run it with --gpus 1 "
              "(multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    import gc
    import torch
    import sparse_top_kv_indexer_amd as S  # noqa: F401  (fails loudly without the library)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return
    hip = HipEvents()
    rec = run_workload(args, hip)
    rec["config"]["config_id"] = CONFIG_ID.get(args.workload)
    gc.collect()
    torch.cuda.empty_cache()
    ref = None if args.no_stream_reference else stream_reference()
    add_stream_reference(rec, ref)
    if args.workload == "token_pool" and args.path == "fused" and not args.no_other_configs:
        others = {}
        for w in OTHER_CONFIGS:
            a = argparse.Namespace(**vars(args))
            a.workload = w
            a.cpu_seconds = args.cpu_seconds / 3.0
            print("other config %s (%s)" % (CONFIG_ID[w], w), file=sys.stderr, flush=True)
            r = run_workload(a, hip)
            r["config"]["config_id"] = CONFIG_ID[w]
            add_stream_reference(r, ref)
            others[CONFIG_ID[w]] = summary(r)
            del r
            gc.collect()
            torch.cuda.empty_cache()
        rec["other_configs"] = others
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
