#!/usr/bin/env python3
"""Write the oracle's results for the full-size compressed-code retrieval
workload (8 KV heads x 4 query heads, L = 1,048,576 keys, beta = rho = 0.02,
top-100, sink 4, local 512) to paris_full_expected.json, and the same
retrieval at the larger tier budgets rho = 0.05 and 0.10 (beta unchanged)
under "by_rho".

Calls only the seeded input generator and oracle/ (no GPU, no HIP library).
The oracle's fp32 encode of 8.4 M keys takes several minutes on one core, so
the KV heads are encoded in parallel processes; each head runs the unchanged
oracle code.  Usage: python tests/golden/make_paris_full.py
"""
import dataclasses
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import dense as D  # noqa: E402
from oracle import lloyd  # noqa: E402
from oracle import paris as P  # noqa: E402

OUT = os.path.join(HERE, "paris_full_expected.json")
SAMPLE_ENTRIES = [0, 1, 4095, 65536, 524287, 1048059]
RHOS = (0.05, 0.10)      # tier budgets besides the workload's rho = beta = 0.02
_P = None


def _head(h):
    p = _P
    lv, th = lloyd.codebook_f32(8)
    n = p.n
    ids = np.empty((n, 16), np.uint8)
    codes = np.empty((n, 64), np.uint8)
    w = np.empty((n, 16), np.float32)
    ch = 1 << 16
    for s0 in range(0, n, ch):
        s1 = min(n, s0 + ch)
        i_, c_, w_, _ = P.encode_keys(p.keys[h, p.sink + s0:p.sink + s1], p.signs, 16, lv, th)
        ids[s0:s1], codes[s0:s1], w[s0:s1] = i_, c_, w_
    return h, ids, codes, w


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    global _P
    t0 = time.time()
    _P = p = W.make_paris()
    print("generated", time.time() - t0, flush=True)
    lv, th = lloyd.codebook_f32(8)
    with mp.get_context("fork").Pool(min(8, os.cpu_count() or 1)) as pool:
        parts = sorted(pool.map(_head, range(p.H)))
    print("encoded", time.time() - t0, flush=True)
    index = {"ids": np.stack([x[1] for x in parts]), "codes": np.stack([x[2] for x in parts]),
             "w": np.stack([x[3] for x in parts])}
    index["hist"] = np.stack([P.histogram(index["ids"][h], 256) for h in range(p.H)])
    index["pos"] = np.arange(p.sink, p.sink + p.n, dtype=np.int64)
    res = P.retrieve(p, index, lv)
    print("retrieved", time.time() - t0, flush=True)
    true = P.exact_top(p, 100)
    kvn = p.kv()
    qn = p.q.reshape(1, p.H * p.G, p.d)
    heads = []
    for h in range(p.H):
        o = D.attend_row(kvn, qn, p.G, 0, h, res["idx"][h], p.sink, p.L - p.local, p.scale)
        heads.append({
            "idx": sorted(int(x) for x in res["idx"][h]),
            "n_cand": int(len(res["idx"][h])),
            "C": int(res["cand"][h].size),
            "vote_hist": np.bincount(res["S"][h], minlength=97).tolist(),
            "votes_sha256": sha(res["S"][h].astype(np.uint8)),
            "cand_sha256": sha(res["cand"][h].astype(np.int32)),
            "est_sha256": sha(res["est"][h].astype(np.float32)),
            "index_hist_sha256": sha(index["hist"][h].astype(np.int32)),
            "samples": {str(e): {"ids": index["ids"][h, e].tolist(),
                                 "codes": index["codes"][h, e].tolist(),
                                 "w_bits": index["w"][h, e].view(np.uint32).tolist()}
                        for e in SAMPLE_ENTRIES},
            "recall_at_100": P.recall_at(res["idx"][h], true[h]),
            "out": o.tolist(),
        })
        print("head", h, "recall", heads[-1]["recall_at_100"], flush=True)
    by_rho = {}
    for rho in RHOS:
        pr = dataclasses.replace(p, rho=rho)
        rr = P.retrieve(pr, index, lv)
        by_rho[repr(rho)] = [{
            "idx": sorted(int(x) for x in rr["idx"][h]),
            "votes_sha256": sha(rr["S"][h].astype(np.uint8)),
            "cand_sha256": sha(rr["cand"][h].astype(np.int32)),
            "est_sha256": sha(rr["est"][h].astype(np.float32)),
            "recall_at_100": P.recall_at(rr["idx"][h], true[h]),
        } for h in range(p.H)]
        print("rho", rho, "mean recall",
              sum(x["recall_at_100"] for x in by_rho[repr(rho)]) / p.H, flush=True)
    rec = {"about": "oracle results for the full-size compressed-code retrieval workload "
                    "(workloads.make_paris() defaults), written by tests/golden/make_paris_full.py",
           "L": p.L, "H": p.H, "G": p.G, "n": p.n, "beta": p.beta, "rho": p.rho,
           "k_final": p.k_final, "sink": p.sink, "local": p.local,
           "levels_bits": lv.view(np.uint32).tolist(), "heads": heads, "by_rho": by_rho}
    json.dump(rec, open(OUT, "w"))
    print("wrote", OUT, time.time() - t0, flush=True)


if __name__ == "__main__":
    main()
