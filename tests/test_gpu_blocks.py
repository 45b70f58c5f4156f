"""GPU parity of block-summary scoring (per-block min / max key summaries,
Quest's bound as the block score, exact top-K blocks, their tokens attended
with the sink and local tokens) against the float64 oracle, through the C ABI.

Bars: summaries equal the oracle's min / max exactly (extremes of bf16 keys
are bf16); block scores within gamma_{2d} * max_g sum_i |q_gi| max(|mn_i|,
|mx_i|) (one fp32 dot product of 2d exact bf16 products); the selected block
set equal to the oracle's up to near ties; the token list exact where the
selection is; attention within 2e-3."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import blocks as BL
from oracle import dense as D

from gpu_helpers import ATTN_TOL, DEV, check_selection, gamma, say

pytestmark = pytest.mark.gpu


def _summarize_all(kv_d, st):
    summ = S.block_summary_pool(kv_d)
    for b in range(st.kv.B):
        S.sparsekv_block_summarize(kv_d, b, 0, st.kv.L_max // 16, summ)
    return summ


def _summary_rows(summ, st, b, h):
    """(mx, mn) rows of sequence b, head h, per logical block, from the pool."""
    kv = st.kv
    d = kv.d_k
    pool = summ.view(torch.int16).cpu().numpy().view(np.uint16)
    n_rows = pool.size // (2 * d)
    pool = pool[: n_rows * 2 * d].reshape(-1, kv.H, 16, 2 * d)
    out = {}
    for j in range(kv.L_max // 16):
        p = int(kv.block_table[b, j])
        if p < 0:
            continue
        row = D.to_f64(pool[p // 16, h, p % 16], "bf16")
        out[j] = (row[:d], row[d:])
    return out


def _check_block_step(st, K, rows, attend=True):
    kv = st.kv
    say("case", st.name, "B", kv.B, "H", kv.H, "G", st.G, "d", kv.d_k, "L", kv.L_max, "K", K)
    kv_d = S.kv_to_device(kv, DEV)
    q = S.to_device(st.q, DEV, True)
    lo = S.to_device(st.lo.astype(np.int32), DEV)
    hi = S.to_device(st.hi.astype(np.int32), DEV)
    summ = _summarize_all(kv_d, st)
    sc, bidx, bcnt, tok = S.sparsekv_block_select(kv_d, summ, q, st.G, lo, hi, K)
    out = None
    if attend:
        out = S.sparsekv_gather_attend(kv_d, q, st.G, tok, 16 * K, lo, hi, st.scale)
        out = out.cpu().numpy()
    torch.cuda.synchronize()
    sc, bidx, bcnt, tok = (x.cpu().numpy() for x in (sc, bidx, bcnt, tok))
    swaps = 0
    for b, h in rows:
        mn, mx, live = BL.block_summaries(kv, b, h)
        got = _summary_rows(summ, st, b, h)
        for j in np.nonzero(live)[0]:
            assert np.array_equal(got[j][0], mx[j]), (b, h, j, "max")
            assert np.array_equal(got[j][1], mn[j]), (b, h, j, "min")
        s_ref, blk_ref, tok_ref, out_ref = BL.block_step_row(st, K, b, h)
        g = sc[b, h].astype(np.float64)
        dead = ~np.isfinite(s_ref)
        assert np.array_equal(np.isneginf(g), dead), (b, h)
        qg = np.abs(D.to_f64(st.q[b, h * st.G:(h + 1) * st.G], "bf16"))
        for j in np.nonzero(~dead)[0]:
            bound = gamma(2 * kv.d_k) * (qg @ np.maximum(np.abs(mn[j]), np.abs(mx[j]))).max()
            assert abs(g[j] - s_ref[j]) <= bound + 1e-30, (b, h, j, g[j], s_ref[j], bound)
        assert bcnt[b, h] == blk_ref.size
        sw = check_selection(s_ref, blk_ref, bidx[b, h], bcnt[b, h])
        swaps += sw
        lb, hb = BL.block_window(int(st.lo[b]), int(st.hi[b]))
        chosen = bidx[b, h][: bcnt[b, h]]
        assert np.all((chosen >= lb) & (chosen < hb))
        # the token list follows from the chosen blocks exactly
        seq = int(kv.seq_len[b])
        exp = np.full(16 * K, -1, np.int64)
        for u, j in enumerate(chosen):
            t = 16 * int(j) + np.arange(16)
            ok = (t < seq) & (kv.block_table[b, j] >= 0)
            exp[16 * u:16 * u + 16] = np.where(ok, t, -1)
        assert np.array_equal(tok[b, h].astype(np.int64), exp), (b, h)
        if sw == 0:
            assert np.array_equal(np.sort(tok[b, h][tok[b, h] >= 0]), tok_ref)
            if out is not None:
                err = np.abs(out[b, h * st.G:(h + 1) * st.G] - out_ref).max()
                assert err <= ATTN_TOL, (b, h, err)
    say("  swaps", swaps)
    return swaps


def _rows(st):
    return [(b, h) for b in range(st.kv.B) for h in range(st.kv.H)]


@pytest.mark.parametrize("G", [1, 4, 8])
def test_blocks_small_ragged(G):
    st = W.make_gqa_paged(tag=950 + G, B=2, H=3, G=G, L=2048, k=256, sink=4, local=64,
                          seq_len=[2048, 1509])
    assert _check_block_step(st, 16, _rows(st)) == 0


@pytest.mark.parametrize("d", [32, 64])
def test_blocks_head_dims(d):
    st = W.make_gqa_paged(tag=960 + d, B=2, H=2, G=2, d=d, L=1024, k=64, sink=5, local=37,
                          seq_len=[1024, 700])
    assert _check_block_step(st, 8, _rows(st), attend=False) == 0


def test_blocks_unmapped_and_short_rows():
    """Unmapped blocks inside the window, a sequence shorter than K blocks
    (count < K, -1 padding), a window edge inside a block on both sides."""
    st = W.make_gqa_paged(tag=970, B=3, H=2, G=4, L=1024, k=64, sink=7, local=29,
                          seq_len=[1024, 997, 150])
    st.kv.block_table[0, [3, 10, 11, 40]] = -1
    st.kv.block_table[1, [1, 61]] = -1
    assert _check_block_step(st, 12, _rows(st)) == 0


def test_blocks_full_size_every_row():
    """4 sequences x 8 KV heads x 4 query heads, d = 128, 32768 tokens
    (2048 blocks per row), top-128 blocks; oracle on all 32 rows."""
    st = W.make_gqa_paged(tag=2, B=4, H=8, G=4, L=32768, k=2048, sink=4, local=64)
    assert _check_block_step(st, 128, [(b, h) for b in range(4) for h in range(8)]) == 0


def test_blocks_incremental_summaries_match_rebuild():
    """Decode appends tokens to the last block: re-summarising only the
    blocks that changed gives the pool a full rebuild gives."""
    st = W.make_gqa_paged(tag=980, B=2, H=2, G=2, L=512, k=32, sink=4, local=16,
                          seq_len=[300, 161])
    kv_d = S.kv_to_device(st.kv, DEV)
    summ = _summarize_all(kv_d, st)
    new_len = np.array([307, 177], np.int32)
    kv_d.seq_len.copy_(torch.from_numpy(new_len))
    for b, (old, new) in enumerate(zip(st.kv.seq_len, new_len)):
        S.sparsekv_block_summarize(kv_d, b, int(old) // 16, (int(new) + 15) // 16, summ)
    fresh = _summarize_all(kv_d, st)
    torch.cuda.synchronize()
    st.kv.seq_len = new_len
    for b in range(2):
        for h in range(2):
            a, f = _summary_rows(summ, st, b, h), _summary_rows(fresh, st, b, h)
            mn, mx, live = BL.block_summaries(st.kv, b, h)
            for j in np.nonzero(live)[0]:
                assert np.array_equal(a[j][0], f[j][0]) and np.array_equal(a[j][1], f[j][1])
                assert np.array_equal(a[j][0], mx[j]) and np.array_equal(a[j][1], mn[j])


def test_blocks_rejects_unsupported():
    st = W.make_gqa_paged(tag=990, B=1, H=1, G=1, L=2064, k=16, sink=4, local=16)
    kv_d = S.kv_to_device(st.kv, DEV)
    summ = S.block_summary_pool(kv_d)
    q = S.to_device(st.q, DEV, True)
    lo = S.to_device(st.lo.astype(np.int32), DEV)
    hi = S.to_device(st.hi.astype(np.int32), DEV)
    with pytest.raises(S.SkvError) as e:      # L_max not a multiple of 256
        S.sparsekv_block_select(kv_d, summ, q, 1, lo, hi, 4, ws=S.workspace(1 << 20, DEV))
    assert e.value.status == S.SKV_EUNSUPPORTED
    with pytest.raises(S.SkvError) as e:      # block range past the table
        S.sparsekv_block_summarize(kv_d, 0, 0, 2064 // 16 + 1, summ)
    assert e.value.status == S.SKV_EINVAL


def test_blocks_summarize_last_follows_decode_appends():
    """One token appended per step to every sequence (across a block edge):
    re-summarising the block of each sequence's last token keeps the pool
    equal to the oracle's summaries of the grown history."""
    st = W.make_gqa_paged(tag=985, B=3, H=5, G=1, d=64, L=512, k=32, sink=4, local=16,
                          seq_len=[62, 15, 300])
    kv_d = S.kv_to_device(st.kv, DEV)
    summ = _summarize_all(kv_d, st)
    lens = st.kv.seq_len.astype(np.int32).copy()
    for _ in range(4):
        lens = lens + 1
        kv_d.seq_len.copy_(torch.from_numpy(lens))
        S.sparsekv_block_summarize_last(kv_d, summ)
    torch.cuda.synchronize()
    st.kv.seq_len = lens
    for b in range(3):
        for h in range(5):
            got = _summary_rows(summ, st, b, h)
            mn, mx, live = BL.block_summaries(st.kv, b, h)
            for j in np.nonzero(live)[0]:
                assert np.array_equal(got[j][0], mx[j]), (b, h, j)
                assert np.array_equal(got[j][1], mn[j]), (b, h, j)
