#!/usr/bin/env python3
"""Benchmark of one sparse top-k decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: score scan -> exact top-k -> gather + split-k
attention (+ split merge), all through the C ABI of libsparsekv.so.

Default workload (the GQA paged decode the metric is quoted on):
  B = 4 sequences, 8 KV heads x 4 query heads, d = 128, L = 32768 bf16 keys
  and values in a 16-token paged pool whose block order is a seeded
  permutation, 4 outlier channels per KV head scaled x8, top-k = 2048 per KV
  head plus 4 sink and 64 local tokens.

Successive steps use distinct device copies of the KV pool in turn (four by
default, like four layers), so that a step never finds its keys in the 256 MB
last-level cache left by the step before.  The K timed steps are captured
into one HIP graph and replayed once, as a serving loop would (--eager
launches every kernel from the host instead).  Per-kernel durations come from
HIP events: with --eager inside the timed region; otherwise from a second
graph of the same K steps with event-record nodes around each call, replayed
right after the timed one (event nodes cost about 14 us per step on this
runtime, so the timed graph carries none).

Prints ONE JSON line (rank 0, N = 1) with the throughput in history keys
scanned per second, the per-step time, the roofline entry of the dominant
kernel (the score scan) and the CPU oracle timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kv-copies C] [--eager]
                  [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBPS = 8000.0
WORKLOADS = ("gqa_paged", "token_pool", "single_head")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_paged", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-copies", type=int, default=4,
                    help="distinct device copies of the KV pool, used in turn by successive "
                         "steps (like successive layers), so that no step finds its keys in "
                         "the 256 MB last-level cache")
    ap.add_argument("--path", default="fused", choices=("fused", "separate"),
                    help="fused: sparsekv_score_hist + sparsekv_select_attend_resume (top-k "
                         "fused with the attention); separate: sparsekv_score_hist + "
                         "sparsekv_topk_resume + sparsekv_gather_attend")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host instead of replaying one HIP graph "
                         "that holds the K timed steps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def make(name):
    import workloads as W
    if name == "gqa_paged":
        return W.make_gqa_paged()
    if name == "token_pool":
        return W.make_token_pool()
    return W.make_single_head()


def workload_config(st):
    kv = st.kv
    return {"workload": {"gqa_paged": "gqa_paged_decode", "token_pool": "token_table_decode",
                         "single_head": "single_head_fp32"}[st.meta.get("bench_name", "gqa_paged")],
            "B": kv.B, "H_kv": kv.H, "G": st.G, "d": kv.d_k, "L": kv.L_max, "k": st.k,
            "sink": int(st.lo[0]), "local": int(kv.seq_len[0] - st.hi[0]),
            "layout": kv.mode, "kv_dtype": kv.dtype}


def scan_bytes_per_key(st):
    """Algorithmic bytes the score scan must move per live key: the key row,
    the fp32 score written, and the 4-byte table entry of token-level pools."""
    es = 2 if st.kv.dtype == "bf16" else 4
    b = st.kv.d_k * es + 4
    if st.kv.token_table is not None:
        b += 4
    return b


def live_keys(st):
    kv = st.kv
    if kv.token_table is not None:
        return int((kv.token_table >= 0).sum()) * kv.H
    return int(kv.seq_len.sum()) * kv.H


def traffic_entry(kernel_src, n_launch_bytes_alg):
    """HBM bytes per score-scan launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", "score_scan_gqa_paged_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
        if rec.get("source_sha256") != h:
            return None
        return rec["hbm_bytes_per_launch"]
    except Exception:
        return None


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
        self.events = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, rc))

    def _stream(self):
        return self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def create(self):
        e = self.ct.c_void_p()
        self._ok(self.lib.hipEventCreate(self.ct.byref(e)), "hipEventCreate")
        self.events.append(e)
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


def cpu_baseline(st, n_keys_step, min_seconds=10.0):
    """The oracle as it stands, on whole steps of the same workload (every
    (sequence, KV head) row: float64 scores, full sort, dense masked
    softmax), repeated until at least min_seconds of CPU work."""
    from oracle import dense as D
    from threadpoolctl import threadpool_info
    rows = [(b, h) for b in range(st.kv.B) for h in range(st.kv.H)]
    n_steps = 0
    t0 = time.perf_counter()
    while True:
        for r in rows:
            D.step(st, rows=[r])
        n_steps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max([1] + blas)
    return {"value": n_steps * n_keys_step / dt, "unit": "keys/s", "cores": cores, "kind": "oracle",
            "sample": "%d whole steps of the same workload (%d rows, %d keys each), %.1f s; "
                      "numpy float64, BLAS threads=%d, other ops single-threaded"
                      % (n_steps, len(rows), n_keys_step, dt, cores),
            "seconds_per_step": dt / n_steps}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the single-GPU hot path only; run it with --gpus 1 "
              "(multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import sparse_top_kv_indexer_amd as S

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

    st = make(args.workload)
    st.meta["bench_name"] = args.workload
    kv = S.kv_to_device(st.kv, dev)
    bf = st.kv.dtype == "bf16"
    q = S.to_device(st.q, dev, bf)
    lo = S.to_device(st.lo.astype(np.int32), dev)
    hi = S.to_device(st.hi.astype(np.int32), dev)
    B, H, L, G, k = kv.B, kv.H, kv.L_max, st.G, st.k
    scores = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    out = torch.empty((B, H * G, kv.d_v), dtype=torch.float32, device=dev)
    fused = args.path == "fused"
    if fused:
        ws_sel = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, kv, G, k), dev)
    else:
        ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, G, k), dev)
        ws_sel = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT, kv, G, k), dev)
    copies = [kv] + [dataclasses.replace(kv, k=kv.k.clone(), v=None if kv.v is None else kv.v.clone())
                     for _ in range(max(1, args.kv_copies) - 1)]
    hip = HipEvents()

    def step(i, ev=None, in_graph=False):
        # sparsekv_select in its two halves (score scan with the first top-k
        # digit fused, then the rest of the exact top-k), so that the events
        # time the scan alone
        c = copies[i % len(copies)]
        mark = (lambda e: hip.graph_record(e)) if in_graph else (lambda e: hip.record(e))
        if ev is not None:
            mark(ev[0])
        S.sparsekv_score_hist(c, q, G, lo, hi, scores, ws_sel)
        if ev is not None:
            mark(ev[1])
        if fused:
            S.sparsekv_select_attend_resume(c, q, G, lo, hi, k, st.scale, scores, idx, cnt, out,
                                            ws_sel)
            if ev is not None:
                mark(ev[2])
        else:
            S.sparsekv_topk_resume(scores, lo, hi, k, idx, cnt, ws_sel)
            if ev is not None:
                mark(ev[2])
            S.sparsekv_gather_attend(c, q, G, idx, k, lo, hi, st.scale, out, ws)
        if ev is not None:
            mark(ev[3])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[hip.create() for _ in range(4)] for _ in range(args.steps)]
    bracket = [hip.create(), hip.create()]
    if args.eager:
        # timed region: exactly K steps launched from the host, with events
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.record(bracket[0])
        for i in range(args.steps):
            step(i, evs[i])
        hip.record(bracket[1])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        timing_note = "per-kernel events recorded inside the timed region"
    else:
        # The K steps are captured into one HIP graph and replayed (as a
        # serving loop would).  Event-record nodes inside a graph cost about
        # 14 us per step on this runtime, so the timed replay carries none;
        # the per-kernel durations come from a second graph of the same K
        # steps, identical except for event-record nodes around each call,
        # replayed right after.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph, graph_ev = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        with torch.cuda.graph(graph_ev):
            for i in range(args.steps):
                step(i, evs[i], in_graph=True)
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
        timing_note = ("per-kernel events from a replay of the same K steps with "
                       "event-record graph nodes, right after the timed replay")

    score_ms = [hip.elapsed_ms(e[0], e[1]) for e in evs]
    topk_ms = [hip.elapsed_ms(e[1], e[2]) for e in evs]
    attn_ms = [hip.elapsed_ms(e[2], e[3]) for e in evs]
    step_ms = [hip.elapsed_ms(e[0], e[3]) for e in evs]
    gpu_ms_per_step = hip.elapsed_ms(bracket[0], bracket[1]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    n_keys = live_keys(st)
    per_key = scan_bytes_per_key(st)
    score_bytes = n_keys * per_key + q.numel() * q.element_size()
    score_avg_s = float(np.mean(score_ms)) * 1e-3
    achieved = score_bytes / score_avg_s / 1e9
    gather_bytes = 0
    if True:
        cnt_np = cnt.cpu().numpy()
        n_att = cnt_np.sum() + (st.lo.astype(np.int64).sum() + (st.kv.seq_len - st.hi).astype(np.int64).sum()) * H
        gather_bytes = int(n_att) * kv.d_k * (2 if bf else 4) * 2
    step_bytes = score_bytes + gather_bytes
    tr = traffic_entry(os.path.join(HERE, "sparse_top_kv_indexer_amd", "csrc", "score.hip"),
                       score_bytes)
    rec = {
        "metric": "history keys scanned/s (one sparse top-k decode step of one layer)",
        "value": n_keys / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": dict(workload_config(st), kv_copies=len(copies),
                       launch="eager" if args.eager else "hip_graph", path=args.path),
        "us_per_step": ms_per_step * 1e3,
        "us_per_step_gpu": gpu_ms_per_step * 1e3,
        "timing": timing_note,
        "us_per_step_events": {"median": float(np.median(step_ms)) * 1e3,
                               "p10": float(np.percentile(step_ms, 10)) * 1e3,
                               "p90": float(np.percentile(step_ms, 90)) * 1e3},
        "kernels_us": ({"score": float(np.mean(score_ms)) * 1e3,
                        "topk_attend_merge": float(np.mean(topk_ms)) * 1e3} if fused else
                       {"score": float(np.mean(score_ms)) * 1e3,
                        "topk": float(np.mean(topk_ms)) * 1e3,
                        "gather_attend": float(np.mean(attn_ms)) * 1e3}),
        "keys_scanned_per_step": n_keys,
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"kernel": "score scan (sparsekv_score_hist: score_stream_kernel with the "
                               "fused top-k histogram)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": tr,
                     "algorithmic_bytes_per_launch": score_bytes,
                     "bytes_per_key": per_key},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(st, n_keys)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
