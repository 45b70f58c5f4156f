"""GPU parity of the threshold-prefiltered exact top-k (sparsekv_score_prefilter
+ sparsekv_topk_prefiltered): over several decode steps with the EMA-predicted
threshold, the selection must be exactly sparsekv_topk's on the same scores
(and the oracle's up to near ties), whether the survivors sufficed or the row
fell back; the threshold update follows alpha kth + (1 - alpha) thr."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D

from gpu_helpers import DEV, Run, check_selection, say

pytestmark = pytest.mark.gpu


def _kth(scores_row, lo, hi, k):
    """k-th largest finite score of the window (fp32), -inf with fewer than k."""
    w = scores_row[lo:hi]
    w = w[np.isfinite(w)]
    return np.float32(np.sort(w)[::-1][k - 1]) if w.size >= k else np.float32(-np.inf)


def _steps(st, qs, alpha=0.5, thr0=None):
    """Run the prefiltered top-k once per query in qs (same KV); check every
    step against sparsekv_topk on the same scores and against the oracle.
    Returns the per-step 'used' flags."""
    r = Run(st)
    kv, G, k = r.skv, st.score_G, st.k
    B, H, L = kv.B, kv.H, kv.L_max
    ws = S.workspace(S.topk_workspace_size(B, H, L, k), DEV)
    thr = torch.full((B, H), -np.inf if thr0 is None else thr0, dtype=torch.float32, device=DEV)
    scores = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, H, k), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B, H), dtype=torch.int32, device=DEV)
    used = torch.empty((B, H), dtype=torch.int32, device=DEV)
    flags = []
    for step, qn in enumerate(qs):
        q = S.to_device(qn, DEV, kv.dtype == "bf16")
        thr_old = thr.cpu().numpy().copy()
        S.sparsekv_score_prefilter(kv, q, G, r.lo, r.hi, thr, scores, ws)
        S.sparsekv_topk_prefiltered(scores, r.lo, r.hi, k, thr, idx, cnt, ws, alpha=alpha,
                                    used=used)
        ref_idx, ref_cnt = S.sparsekv_topk(scores, r.lo, r.hi, k)
        torch.cuda.synchronize()
        sc = scores.cpu().numpy()
        gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
        assert np.array_equal(gc, ref_cnt.cpu().numpy())
        assert np.array_equal(gi, ref_idx.cpu().numpy())
        u = used.cpu().numpy()
        th = thr.cpu().numpy()
        for b in range(B):
            lo, hi = int(st.lo[b]), int(st.hi[b])
            for h in range(H):
                kth = _kth(sc[b, h], lo, hi, k)
                want = kth if (thr_old[b, h] == -np.inf or kth == -np.inf) else \
                    np.float32(alpha) * kth + np.float32(1 - alpha) * thr_old[b, h]
                if np.isinf(want):
                    assert th[b, h] == want, (step, b, h)
                else:
                    assert abs(th[b, h] - want) <= 4e-7 * max(abs(want), 1e-30), (step, b, h, th[b, h], want)
        # independent check of the selection against the float64 oracle
        for b in range(B):
            for h in range(H):
                s_ref = D.scores_row(st.score_kv, qn, G, b, h)
                sel = D.select_topk(s_ref, int(st.lo[b]), int(st.hi[b]), k)
                assert gc[b, h] == sel.size
                check_selection(s_ref, sel, gi[b, h], gc[b, h])
        say("  step", step, "rows from survivors", int(u.sum()), "of", u.size)
        flags.append(u)
    return flags


def _queries(st, n, tag, eps=0.05):
    """n decode steps: the workload's query twice (the second step's threshold
    is then the exact k-th score), then small seeded perturbations of it (the
    k-th score moves a little from step to step; rows whose prediction
    overshoots fall back)."""
    q0 = D.to_f64(st.score_q, st.score_kv.dtype).astype(np.float32)
    rng = np.random.default_rng(tag)
    out = []
    for i in range(n):
        q = q0 if i < 2 else q0 + eps * rng.standard_normal(q0.shape).astype(np.float32)
        out.append(W.f32_to_bf16_bits(q) if st.score_kv.dtype == "bf16" else q)
    return out


@pytest.mark.parametrize("G,L,layout", [(4, 3000, "paged"), (1, 5000, "token"), (2, 2500, "contiguous"),
                                        (1, 40000, "paged")])
def test_prefilter_steps_equal_exact_topk(G, L, layout):
    st = W.make_gqa_paged(tag=500 + G, B=2, H=3, G=G, L=L - L % 16, k=min(300, L // 8), sink=4,
                          local=32, seq_len=[L - L % 16, (L - L % 16) * 2 // 3])
    if layout == "token":
        bt = st.kv.block_table
        t = np.arange(st.kv.L_max)
        tt = (bt[:, t // 16] * 16 + t % 16).astype(np.int32)
        tt[np.random.default_rng(G).random(tt.shape) < 0.3] = -1
        tt[:, :4] = bt[:, :1] * 16 + np.arange(4)
        st.kv.token_table, st.kv.block_table = tt, None
    elif layout == "contiguous":
        pool = st.kv.k
        logical = pool[st.kv.block_table]
        st.kv.k = np.ascontiguousarray(logical.transpose(0, 2, 1, 3, 4).reshape(
            st.kv.B, st.kv.H, st.kv.L_max, st.kv.d_k))
        pool = st.kv.v
        st.kv.v = np.ascontiguousarray(pool[st.kv.block_table].transpose(0, 2, 1, 3, 4).reshape(
            st.kv.B, st.kv.H, st.kv.L_max, st.kv.d_v))
        st.kv.block, st.kv.block_table = 0, None
    say("prefilter", st.name, "G", G, "L", st.kv.L_max, layout)
    flags = _steps(st, _queries(st, 4, 600 + G))
    if L <= 16384:
        assert flags[0].all()        # thr = -inf: every candidate survives, still fits the list
    assert flags[1].all()            # thr = the exact k-th score of the same query


def test_prefilter_fallbacks():
    """A threshold above every score (too few survivors) and a threshold of
    -inf over rows of more than 16384 candidates (list overflow) both fall
    back to the full row, with the same exact result."""
    st = W.make_gqa_paged(tag=520, B=1, H=2, G=4, L=24000 - 24000 % 16, k=500, sink=4, local=16)
    qs = _queries(st, 2, 521)
    f = _steps(st, qs[:1], thr0=1e30)
    assert not f[0].any()
    f = _steps(st, qs[:1])
    assert not f[0].any()


def test_prefilter_ties_ranked_by_position():
    """Rows where many keys are identical copies (equal scores at the
    threshold): equal keys are taken lowest position first."""
    st = W.make_gqa_paged(tag=530, B=1, H=2, G=2, L=4096, k=200, sink=4, local=16)
    pool = st.kv.k
    bt = st.kv.block_table
    rng = np.random.default_rng(531)
    for h in range(2):
        src = pool[bt[0, 5], h, 3].copy()
        for t in rng.choice(np.arange(16, 4000), size=600, replace=False):
            pool[bt[0, t // 16], h, t % 16] = src
    flags = _steps(st, _queries(st, 3, 532))
    assert flags[1].all()


@pytest.mark.slow
def test_prefilter_indexer_full_size():
    """One 131072-key indexer row (the long-context configuration), 3 steps."""
    st = W.make_indexer_mla()
    flags = _steps(st, _queries(st, 3, 540, eps=0.02))
    assert flags[1].all()
