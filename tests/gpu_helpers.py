"""Helpers for the GPU parity tests: upload a workload, run the HIP step through
the binding, compare against the oracle with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_top_kv_indexer_amd as S
from oracle import dense as D

DEV = "cuda:0"

# attention outputs: bf16 / fp32 inputs with fp32 accumulation
ATTN_TOL = 2e-3
# selection: a swapped pair must be a near tie in the float64 scores
TIE_REL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)


class Run:
    """One upload of a Step, reusable for several calls."""

    def __init__(self, st):
        self.st = st
        bf = st.kv.dtype == "bf16"
        self.kv = S.kv_to_device(st.kv, DEV)
        self.skv = self.kv if st.score_kv is st.kv else S.kv_to_device(st.score_kv, DEV)
        self.q = S.to_device(st.q, DEV, bf)
        self.sq = self.q if st.score_q is st.q else S.to_device(st.score_q, DEV, st.score_kv.dtype == "bf16")
        self.lo = S.to_device(st.lo.astype(np.int32), DEV)
        self.hi = S.to_device(st.hi.astype(np.int32), DEV)

    def score(self):
        return S.sparsekv_score(self.skv, self.sq, self.st.score_G)

    def topk(self, scores):
        return S.sparsekv_topk(scores, self.lo, self.hi, self.st.k)

    def select(self):
        """score + top-k in one call (histogram fused into the scan)."""
        return S.sparsekv_select(self.skv, self.sq, self.st.score_G, self.lo, self.hi, self.st.k)

    def attend(self, idx):
        return S.sparsekv_gather_attend(self.kv, self.q, self.st.G, idx, self.st.k, self.lo, self.hi,
                                        self.st.scale)

    def select_attend(self, ws=None):
        """the fused decode step: scan, top-k and attention in one call"""
        r = S.sparsekv_select_attend(self.kv, self.q, self.st.G, self.lo, self.hi, self.st.k,
                                     self.st.scale, ws=ws)
        torch.cuda.synchronize()
        return r

    def step(self, fused=True):
        if fused == "all":
            return self.select_attend()
        if fused:
            sc, idx, cnt = self.select()
        else:
            sc = self.score()
            idx, cnt = self.topk(sc)
        out = self.attend(idx)
        torch.cuda.synchronize()
        return sc, idx, cnt, out


def check_scores(st, gpu_scores: np.ndarray, rows):
    """|s_gpu - s_ref| <= gamma_{d(+1)} * max_g sum_j |q_gj k_j| per key."""
    kv, G = st.score_kv, st.score_G
    n = kv.d_k + (1 if kv.dtype == "f32" else 0)
    worst = 0.0
    for b, h in rows:
        ref = D.scores_row(kv, st.score_q, G, b, h)
        got = gpu_scores[b, h].astype(np.float64)
        dead = ~np.isfinite(ref)
        assert np.array_equal(np.isneginf(got), dead), (b, h)
        t, K, _ = D.logical_kv(kv, b, h)
        qg = D.to_f64(st.score_q[b, h * G:(h + 1) * G], kv.dtype)
        bound = np.zeros(kv.L_max)
        bound[t] = gamma(n) * (np.abs(K) @ np.abs(qg).T).max(axis=1)
        err = np.abs(got[~dead] - ref[~dead])
        assert np.all(err <= bound[~dead] + 1e-30), (b, h, float((err - bound[~dead]).max()))
        if err.size:
            worst = max(worst, float((err / np.maximum(bound[~dead], 1e-30)).max()))
    return worst


def check_selection(ref_scores_row, ref_sel, got_idx_row, got_count):
    """Set parity with the near-tie rule; returns the number of swaps."""
    got = got_idx_row[:got_count]
    assert np.all(got_idx_row[got_count:] == -1)
    assert len(np.unique(got)) == got.size
    assert np.all(np.diff(got) > 0)                      # ascending
    assert got.size == ref_sel.size
    a, r = set(got.tolist()), set(ref_sel.tolist())
    extra, missing = sorted(a - r), sorted(r - a)
    assert len(extra) == len(missing)
    for i, j in zip(sorted(extra, key=lambda x: -ref_scores_row[x]),
                    sorted(missing, key=lambda x: -ref_scores_row[x])):
        si, sj = ref_scores_row[i], ref_scores_row[j]
        assert abs(si - sj) <= TIE_REL * max(abs(si), abs(sj)), (i, j, si, sj)
    return len(extra)
