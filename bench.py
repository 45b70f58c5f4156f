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

Prints ONE JSON line (rank 0, N = 1) with the throughput in history keys
scanned per second, the per-step time, the roofline entry of the dominant
kernel (the score scan) and the CPU oracle timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
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


def cpu_baseline(st, n_keys_step):
    """The oracle as it stands, on the whole step of the default workload
    (every (sequence, KV head) row: float64 scores, full sort, dense masked
    softmax)."""
    import numpy as np
    from oracle import dense as D
    from threadpoolctl import threadpool_info
    rows = [(b, h) for b in range(st.kv.B) for h in range(st.kv.H)]
    t0 = time.perf_counter()
    for r in rows:
        D.step(st, rows=[r])
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max([1] + blas)
    return {"value": n_keys_step / dt, "unit": "keys/s", "cores": cores, "kind": "oracle",
            "sample": "one whole step of the same workload (%d rows, %d keys), %.1f s; "
                      "numpy float64, BLAS threads=%d, other ops single-threaded"
                      % (len(rows), n_keys_step, dt, cores),
            "seconds_per_step": dt}


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
    ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, kv, G, k), dev)
    ws_sel = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT, kv, G, k), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # sparsekv_select in its two halves (score scan with the first top-k
        # digit fused, then the rest of the exact top-k), so that the events
        # time the scan alone
        if ev is not None:
            ev[0].record(stream)
        S.sparsekv_score_hist(kv, q, G, lo, hi, scores, ws_sel)
        if ev is not None:
            ev[1].record(stream)
        S.sparsekv_topk_resume(scores, lo, hi, k, idx, cnt, ws_sel)
        if ev is not None:
            ev[2].record(stream)
        S.sparsekv_gather_attend(kv, q, G, idx, k, lo, hi, st.scale, out, ws)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    score_ms = [e[0].elapsed_time(e[1]) for e in evs]
    topk_ms = [e[1].elapsed_time(e[2]) for e in evs]
    attn_ms = [e[2].elapsed_time(e[3]) for e in evs]
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
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
        "config": workload_config(st),
        "us_per_step": ms_per_step * 1e3,
        "us_per_step_events": {"median": float(np.median(step_ms)) * 1e3,
                               "p10": float(np.percentile(step_ms, 10)) * 1e3,
                               "p90": float(np.percentile(step_ms, 90)) * 1e3},
        "kernels_us": {"score": float(np.mean(score_ms)) * 1e3,
                       "topk": float(np.mean(topk_ms)) * 1e3,
                       "gather_attend": float(np.mean(attn_ms)) * 1e3},
        "keys_scanned_per_step": n_keys,
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"kernel": "score scan (sparsekv_score_hist: score_mfma_kernel with the "
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
