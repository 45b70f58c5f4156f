"""GPU parity of the fused decode-step calls for rows longer than one
32768-slot sweep.  The latent attention (sparsekv_select_attend_resume after
the indexer's sparsekv_score_hist) finishes the exact top-k inside the
attention kernel: the slice listing, then every attending workgroup resolves
the row's selection from the list itself.  GQA rows (sparsekv_select_attend
and its resume) take the slice-listing top-k and the split attention inside
the same call: with 128 rows or more one workgroup per row lists its row
itself (no listing kernel), selects and attends over all of the selection
(no split merge), with fewer 8
workgroups per row each finish it and attend an eighth, then the merge.  Checked against the float64 oracle (selection set, attention
within 2e-3) and against the separate calls, including rows whose candidate
list overflows (many tied scores) so that the selection falls back to reading
the row per digit."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D

from gpu_helpers import ATTN_TOL, DEV, Run, check_selection, say

pytestmark = pytest.mark.gpu


def _resume(r, ws=None):
    st = r.st
    skv, kv = r.skv, r.kv
    B, H, L = skv.B, skv.H, skv.L_max
    scores = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    idx = torch.full((B, H, st.k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    out = torch.full((kv.B, kv.H * st.G, kv.d_v), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = S.workspace(max(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, kv, st.G, st.k),
                             S.sparsekv_workspace_size(S.SKV_OP_SELECT, skv, st.score_G, st.k)), DEV)
    S.sparsekv_score_hist(skv, r.sq, st.score_G, r.lo, r.hi, scores, ws)
    S.sparsekv_select_attend_resume(kv, r.q, st.G, r.lo, r.hi, st.k, st.scale, scores, idx, cnt,
                                    out, ws)
    torch.cuda.synchronize()
    return scores, idx, cnt, out, ws


def _indexer(r, ws=None):
    """sparsekv_indexer_attend: the indexer scan, top-k and latent attention
    in one call (segment candidates for rows longer than one sweep, k <= 2048)."""
    st = r.st
    skv, kv = r.skv, r.kv
    B, H, L = skv.B, skv.H, skv.L_max
    scores = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    idx = torch.full((B, H, st.k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    out = torch.full((kv.B, kv.H * st.G, kv.d_v), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, kv, st.G, st.k), DEV)
    S.sparsekv_indexer_attend(skv, r.sq, st.score_G, kv, r.q, st.G, r.lo, r.hi, st.k, st.scale,
                              scores, idx, cnt, out, ws)
    torch.cuda.synchronize()
    return scores, idx, cnt, out, ws


def _check(st, rows=None):
    say("fused long case", st.name, "G", st.G, "L", st.kv.L_max, "k", st.k)
    r = Run(st)
    # the one-call indexer step against the oracle and the two-call path
    _, iidx, icnt, iout, _ = _indexer(r)
    iidx, icnt, iout = iidx.cpu().numpy(), icnt.cpu().numpy(), iout.cpu().numpy()
    sc, idx, cnt, out, ws = _resume(r)
    idx, cnt, out = idx.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(iidx, idx) and np.array_equal(icnt, cnt)
    assert np.abs(iout - out).max() <= ATTN_TOL
    B, H = st.score_kv.B, st.score_kv.H
    rows = [(b, h) for b in range(B) for h in range(H)] if rows is None else rows
    ref = D.step(st, rows=rows)
    swaps = 0
    for b, h in rows:
        sel = ref["idx"][b, h][: ref["count"][b, h]]
        assert cnt[b, h] == ref["count"][b, h], (b, h)
        sw = check_selection(ref["scores"][b, h], sel, idx[b, h], cnt[b, h])
        swaps += sw
        if sw == 0:
            hs = list(range(h * st.G, (h + 1) * st.G))
            err = np.abs(out[b, hs] - ref["out"][b, hs]).max()
            assert err <= ATTN_TOL, (b, h, err)
    # the separate calls select the same set
    _, idx2, cnt2, out2 = r.step(fused=True)
    assert np.array_equal(idx, idx2.cpu().numpy()) and np.array_equal(cnt, cnt2.cpu().numpy())
    assert np.abs(out - out2.cpu().numpy()).max() <= ATTN_TOL
    # the workspace regions that must start the next call at zero are zero
    rws = B * H
    # (two histogram copies per row when at most 4 rows are longer than one
    # 32,768-slot sweep, else one)
    copies = 2 if (rws <= 4 and st.score_kv.L_max > 32768) else 1
    assert torch.count_nonzero(ws[: rws * copies * 4096 * 4]).item() == 0
    return swaps


@pytest.mark.parametrize("L,k,heads", [(65536, 2048, 128), (40000, 77, 16), (50016, 4096, 32),
                                       (33024, 300, 64)])
def test_fused_latent_long_rows(L, k, heads):
    st = W.make_indexer_mla(tag=700 + heads, L=L, k=k, n_heads=heads)
    assert _check(st) == 0


def test_fused_latent_with_sink_local_and_short_sequence():
    st = W.make_indexer_mla(tag=710, L=65536, k=1000, n_heads=128)
    st.lo = np.array([7], np.int32)
    st.hi = np.array([65536 - 300], np.int32)
    assert _check(st) == 0
    st = W.make_indexer_mla(tag=711, L=65536, k=512, n_heads=64)
    st.kv.seq_len[:] = 40001
    st.score_kv.seq_len[:] = 40001
    st.hi = np.array([40001 - 100], np.int32)
    assert _check(st) == 0


def test_fused_latent_list_overflow_takes_the_row_fallback():
    """All indexer keys equal: every score ties, the candidate list (and
    every scan segment's candidates) overflows and each attending workgroup
    selects from the row itself (lowest positions win the ties)."""
    st = W.make_indexer_mla(tag=712, L=40960, k=1024, n_heads=16)
    st.score_kv.k[:] = st.score_kv.k[0, 0, 0]
    r = Run(st)
    ref = D.step(st)
    for call in (_resume, _indexer):
        sc, idx, cnt, out, _ = call(r)
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        assert cnt[0, 0] == 1024
        assert idx[0, 0].tolist() == list(range(1024))
        assert np.abs(out.cpu().numpy() - ref["out"]).max() <= ATTN_TOL


def test_indexer_segments_crowded_by_a_run_of_top_keys():
    """1,500 consecutive tokens carry the highest indexer scores, so the scan
    segments holding them cannot list all of their keys that rank in the
    top-k: their cuts lie above the k-th candidate and the row is selected
    from its scores; the result is still the exact top-k."""
    st = W.make_indexer_mla(tag=713, L=65536, k=2048, n_heads=32)
    qf = (st.score_q[0, 0].astype(np.uint32) << 16).view(np.float32)
    kb = (((qf * 4).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # bf16 of 4 q
    blocks = st.score_kv.block_table[0]
    for t in range(3000, 4500):
        st.score_kv.k[blocks[t // 16], 0, t % 16] = kb
    assert _check(st) == 0
    r = Run(st)
    _, idx, cnt, _, _ = _indexer(r)
    sel = set(idx[0, 0].cpu().numpy().tolist())
    assert int(cnt[0, 0]) == 2048 and set(range(3000, 4500)) <= sel


def test_indexer_attend_repeated_calls_and_short_k():
    """Two calls in a row on one workspace (the segment lists are rewritten
    whole by every scan), then k = 1 and a window that leaves fewer
    candidates than k."""
    st = W.make_indexer_mla(tag=714, L=49152, k=700, n_heads=16)
    r = Run(st)
    ref = D.step(st)
    ws = None
    for _ in range(2):
        _, idx, cnt, out, ws = _indexer(r, ws)
        sel = ref["idx"][0, 0][: ref["count"][0, 0]]
        assert check_selection(ref["scores"][0, 0], sel, idx[0, 0].cpu().numpy(),
                               int(cnt[0, 0])) == 0
        assert np.abs(out.cpu().numpy() - ref["out"]).max() <= ATTN_TOL
    st.k = 1
    assert _check(st) == 0
    st.k = 2000
    st.lo = np.array([30000], np.int32)
    st.hi = np.array([31500], np.int32)   # 1,500 candidates < k
    assert _check(st) == 0


@pytest.mark.slow
def test_fused_latent_full_size():
    """The indexer + shared-latent workload at L = 131072, top-2048, 128 heads."""
    st = W.make_indexer_mla()
    assert _check(st) == 0


# ------------------------------------------------------- GQA rows, long
def _check_gqa(st, rows=None):
    """The fused call on long GQA rows against the oracle and against
    resume-after-scan."""
    say("fused long GQA", st.name, "G", st.G, "L", st.kv.L_max, "k", st.k, st.kv.mode)
    r = Run(st)
    sc, idx, cnt, out = [t.cpu().numpy() for t in r.select_attend()]
    B, H = st.kv.B, st.kv.H
    rows = [(b, h) for b in range(B) for h in range(H)] if rows is None else rows
    ref = D.step(st, rows=rows)
    swaps = 0
    for b, h in rows:
        sel = ref["idx"][b, h][: ref["count"][b, h]]
        assert cnt[b, h] == ref["count"][b, h], (b, h)
        sw = check_selection(ref["scores"][b, h], sel, idx[b, h], cnt[b, h])
        swaps += sw
        if sw == 0:
            hs = list(range(h * st.G, (h + 1) * st.G))
            err = np.abs(out[b, hs] - ref["out"][b, hs]).max()
            assert err <= ATTN_TOL, (b, h, err)
    _, idx2, cnt2, out2, _ = _resume(r)
    assert np.array_equal(idx, idx2.cpu().numpy()) and np.array_equal(cnt, cnt2.cpu().numpy())
    assert np.abs(out - out2.cpu().numpy()).max() <= ATTN_TOL
    return swaps


@pytest.mark.parametrize("G,L,k", [(4, 40000, 2048), (1, 65536, 100), (8, 33024, 4096)])
def test_fused_gqa_long_paged(G, L, k):
    st = W.make_gqa_paged(tag=720 + G, B=2, H=2, G=G, L=L, k=k, sink=4, local=64,
                          seq_len=[L, L - 777])
    assert _check_gqa(st) == 0


def test_fused_gqa_long_token_table():
    st = W.make_token_pool(tag=730, B=3, H=2, L=65536, k=2048, sink=4, local=128)
    assert _check_gqa(st) == 0


def test_fused_gqa_long_segments_crowded_by_a_run_of_top_keys():
    """Few long GQA rows take the scan's segment candidates: a run of 3,000
    top-scoring tokens in one row overflows its segments, so that row is
    selected from its scores; the other rows keep the candidates."""
    st = W.make_gqa_paged(tag=732, B=2, H=2, G=1, L=65536, k=2048, sink=4, local=64)
    qf = (st.q[1, 1].astype(np.uint32) << 16).view(np.float32)
    kb = (((qf * 4).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # bf16 of 4 q
    blocks = st.kv.block_table[1]
    for t in range(10000, 13000):
        st.kv.k[blocks[t // 16], 1, t % 16] = kb
    assert _check_gqa(st) == 0
    r = Run(st)
    _, idx, cnt, _ = r.select_attend()
    assert int(cnt[1, 1]) == 2048 and idx[1, 1].cpu().numpy().tolist() == list(range(10000, 12048))


@pytest.mark.parametrize("G,L,k,run", [(4, 32768, 2048, 0), (2, 20000, 1000, 1500),
                                       (1, 16400, 64, 0)])
def test_fused_gqa_one_sweep_rows_take_segments(G, L, k, run):
    """Few rows of one sweep but over 16384 slots also take the segment
    candidates (the exact top-k of every row against the oracle); a run of
    top-scoring tokens in row (1, 1) overflows its segments, so that row is
    selected from its scores."""
    st = W.make_gqa_paged(tag=770 + G, B=2, H=2, G=G, L=L, k=k, sink=4, local=64,
                          seq_len=[L, L - 333])
    if run:
        qf = (st.q[1, G].astype(np.uint32) << 16).view(np.float32)   # head (h = 1, g = 0)
        kb = (((qf * 4).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
        blocks = st.kv.block_table[1]
        for t in range(5000, 5000 + run):
            st.kv.k[blocks[t // 16], 1, t % 16] = kb
    r = Run(st)
    assert S.sparsekv_segments(r.kv, G, k) > 0
    assert _check_gqa(st) == 0
    if run:
        _, idx, cnt, _ = r.select_attend()
        assert int(cnt[1, 1]) == k and idx[1, 1].cpu().numpy().tolist() == list(range(5000, 5000 + k))


def test_fused_gqa_long_list_overflow_fallback():
    """Every key of sequence 0 ties: its list overflows and each attending
    workgroup selects from the row itself (lowest positions win)."""
    st = W.make_gqa_paged(tag=731, B=2, H=1, G=2, L=40960, k=1500, sink=4, local=64)
    blocks = st.kv.block_table[0]
    st.kv.k[blocks] = st.kv.k[blocks[0], :, 0:1, :]
    assert _check_gqa(st) == 0
    r = Run(st)
    _, idx, cnt, _ = r.select_attend()
    assert int(cnt[0, 0]) == 1500 and idx[0, 0].cpu().numpy().tolist() == list(range(4, 1504))


def test_fused_gqa_long_many_rows_token_table():
    """128 rows: the one-workgroup-per-row finish + attention."""
    st = W.make_token_pool(tag=740, B=16, H=8, L=40000, k=2048, sink=4, local=128)
    assert _check_gqa(st) == 0


def test_fused_gqa_long_many_rows_g8_k4096_ragged():
    """128 rows, G = 8, k = 4096 (the most the kernel stages), ragged
    sequence lengths and a paged pool."""
    seq = [33024 - 1531 * (b % 5) for b in range(16)]
    st = W.make_gqa_paged(tag=741, B=16, H=8, G=8, L=33024, k=4096, sink=4, local=64, seq_len=seq)
    assert _check_gqa(st) == 0


def test_fused_gqa_long_many_rows_list_overflow_fallback():
    """128 rows, one of them all ties: that row's list overflows and its
    workgroup selects from the row itself."""
    st = W.make_gqa_paged(tag=742, B=16, H=8, G=1, L=40960, k=1500, sink=4, local=64)
    blocks = st.kv.block_table[3]
    st.kv.k[blocks, 5] = st.kv.k[blocks[0], 5, 0:1, :]
    rows = [(3, 5), (3, 4), (0, 0), (15, 7)]
    assert _check_gqa(st, rows=rows) == 0
    r = Run(st)
    _, idx, cnt, _ = r.select_attend()
    assert int(cnt[3, 5]) == 1500 and idx[3, 5].cpu().numpy().tolist() == list(range(4, 1504))


@pytest.mark.parametrize("n_blocks", [188, 625])
def test_fused_gqa_long_many_rows_tied_run(n_blocks):
    """128 rows, one query head; in one row the first 16 n_blocks tokens tie
    for the top score, and the k taken must be the lowest positions.  With
    3,008 tied tokens the row's own listing holds them all (at most 4,096
    keys) and resolves the tie; with 10,000 it would overflow, so the row is
    selected from the scores alone."""
    st = W.make_gqa_paged(tag=744, B=16, H=8, G=1, L=40960, k=1500, sink=4, local=64)
    qf = (st.q[3, 5].astype(np.uint32) << 16).view(np.float32)
    kb = (((qf * 4).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # bf16 of 4 q
    st.kv.k[st.kv.block_table[3][:n_blocks], 5] = kb                     # tokens 0 .. 16 n_blocks - 1
    rows = [(3, 5), (3, 4), (0, 0), (15, 7)]
    assert _check_gqa(st, rows=rows) == 0
    r = Run(st)
    _, idx, cnt, _ = r.select_attend()
    assert int(cnt[3, 5]) == 1500 and idx[3, 5].cpu().numpy().tolist() == list(range(4, 1504))


@pytest.mark.parametrize("B,H,G,L,k", [(127, 1, 2, 33024, 700), (64, 2, 3, 40000, 1024),
                                       (16, 8, 1, 36000, 33)])
def test_fused_gqa_long_rows_around_the_one_workgroup_threshold(B, H, G, L, k):
    """127 rows (8 workgroups per row and the merge) against 128 (one
    workgroup per row, no merge), with G not a power of two and a small k."""
    st = W.make_gqa_paged(tag=750 + B, B=B, H=H, G=G, L=L, k=k, sink=4, local=64)
    rows = [(b, h) for b in range(0, B, max(1, B // 8)) for h in range(H)][:24]
    assert _check_gqa(st, rows=rows) == 0


def test_fused_gqa_long_many_rows_window_edges():
    """128 rows through the one-workgroup-per-row kernel with edge windows:
    no candidates (lo == hi), fewer candidates than k, a sequence of 40
    tokens, an empty sequence, k = 1."""
    seq = [40960] * 16
    seq[3], seq[4] = 40, 0
    st = W.make_gqa_paged(tag=743, B=16, H=8, G=2, L=40960, k=2048, sink=4, local=64,
                          seq_len=seq)
    st.lo[0] = st.hi[0] = 20000             # only the sink and local tokens
    st.lo[1], st.hi[1] = 1000, 2500         # 1,500 candidates < k
    st.lo[3], st.hi[3] = 4, 20              # a short sequence
    st.lo[4], st.hi[4] = 0, 0               # an empty one
    rows = [(b, h) for b in (0, 1, 2, 3, 4, 15) for h in (0, 7)]
    assert _check_gqa(st, rows=rows) == 0
    st.k = 1
    assert _check_gqa(st, rows=rows) == 0


@pytest.mark.slow
def test_fused_gqa_long_full_size_every_row():
    """The GQA decode at L = 131072 through the fused call, all 32 rows."""
    st = W.make_gqa_paged(L=131072)
    assert _check_gqa(st) == 0


@pytest.mark.slow
def test_fused_token_pool_full_size_64_rows_over_every_head():
    st = W.make_token_pool()
    rows = [(b, (b + 4 * j) % 8) for b in range(32) for j in range(2)]
    assert _check_gqa(st, rows=rows) == 0


def test_segment_pair_equals_the_one_call_step():
    """The two halves of the segment path (sparsekv_score_segments, then
    sparsekv_select_attend_segments) give what sparsekv_select_attend gives,
    for GQA rows and for the latent step (the scan over the indexer's KV)."""
    st = W.make_gqa_paged(tag=760, B=2, H=2, G=4, L=65536, k=2048, sink=4, local=64)
    r = Run(st)
    sc1, idx1, cnt1, out1 = r.select_attend()
    kv = r.kv
    assert S.sparsekv_segments(kv, st.G, st.k) > 0
    ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, kv, st.G, st.k), DEV)
    sc = torch.empty_like(sc1)
    idx = torch.empty_like(idx1)
    cnt = torch.empty_like(cnt1)
    out = torch.empty_like(out1)
    S.sparsekv_score_segments(kv, r.q, st.G, r.lo, r.hi, st.k, sc, ws)
    S.sparsekv_select_attend_segments(kv, r.q, st.G, r.lo, r.hi, st.k, st.scale, sc, idx, cnt,
                                      out, ws)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc1) and torch.equal(idx, idx1) and torch.equal(cnt, cnt1)
    assert float((out - out1).abs().max()) <= ATTN_TOL
    # latent: the scan over the indexer's keys, the selection from its segments
    st = W.make_indexer_mla(tag=761, L=65536, k=2048, n_heads=64)
    r = Run(st)
    _, iidx, icnt, iout, _ = _indexer(r)
    ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, r.kv, st.G, st.k), DEV)
    sc = torch.empty((1, 1, 65536), dtype=torch.float32, device=DEV)
    idx = torch.empty_like(iidx)
    cnt = torch.empty_like(icnt)
    out = torch.empty_like(iout)
    S.sparsekv_score_segments(r.skv, r.sq, st.score_G, r.lo, r.hi, st.k, sc, ws)
    S.sparsekv_select_attend_segments(r.kv, r.q, st.G, r.lo, r.hi, st.k, st.scale, sc, idx, cnt,
                                      out, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, iidx) and torch.equal(cnt, icnt)
    assert float((out - iout).abs().max()) <= ATTN_TOL


def test_scan_scores_at_an_unaligned_address():
    """The scan stages a row segment's scores in LDS and writes them out with
    16-byte stores when the row starts on a 16-byte boundary, one by one
    otherwise: scores written 4 bytes past such a boundary equal the aligned
    ones, on the histogram path and on the segment-candidate path."""
    st = W.make_gqa_paged(tag=780, B=2, H=2, G=4, L=20000, k=500, sink=4, local=64,
                          seq_len=[20000, 19001])
    r = Run(st)
    B, H, L = r.kv.B, r.kv.H, r.kv.L_max
    n_ws = S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, r.kv, st.G, st.k)
    ref = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    base = torch.full((B * H * L + 1,), 7.0, dtype=torch.float32, device=DEV)
    odd = base[1:].view(B, H, L)
    assert odd.data_ptr() % 16 == 4
    ws = S.workspace(n_ws, DEV)
    S.sparsekv_score_hist(r.kv, r.q, st.G, r.lo, r.hi, ref, ws)
    ws.zero_()
    S.sparsekv_score_hist(r.kv, r.q, st.G, r.lo, r.hi, odd, ws)
    torch.cuda.synchronize()
    assert torch.equal(odd, ref) and float(base[0]) == 7.0
    assert S.sparsekv_segments(r.kv, st.G, st.k) > 0
    base.fill_(7.0)
    S.sparsekv_score_segments(r.kv, r.q, st.G, r.lo, r.hi, st.k, odd, S.workspace(n_ws, DEV))
    torch.cuda.synchronize()
    assert torch.equal(odd, ref) and float(base[0]) == 7.0
