"""GPU parity of the fused decode step (sparsekv_select_attend: score scan,
then exact top-k fused with the gather + split attention) against the
float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D

from gpu_helpers import ATTN_TOL, DEV, Run, check_scores, check_selection, say

pytestmark = pytest.mark.gpu


def _fused_vs_oracle(st, rows=None):
    say("fused case", st.name, "B", st.kv.B, "H", st.kv.H, "G", st.G, "L", st.kv.L_max, "k", st.k,
        "mode", st.kv.mode)
    B, H = st.kv.B, st.kv.H
    rows = [(b, h) for b in range(B) for h in range(H)] if rows is None else rows
    r = Run(st)
    sc, idx, cnt, out = [t.cpu().numpy() for t in r.select_attend()]
    check_scores(st, sc, rows)
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
    # the separate calls give the same selection
    _, idx2, cnt2, _ = r.step(fused=True)
    assert np.array_equal(idx, idx2.cpu().numpy()) and np.array_equal(cnt, cnt2.cpu().numpy())
    return swaps


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fused_gqa_paged_ragged(G):
    st = W.make_gqa_paged(tag=400 + G, B=3, H=3, G=G, L=4096, k=300, sink=4, local=64,
                          seq_len=[4096, 2500, 777])
    assert _fused_vs_oracle(st) == 0


def test_fused_contiguous_and_token_table():
    st = W.make_gqa_paged(tag=410, B=2, H=2, G=4, L=2048, k=200, sink=4, local=32,
                          seq_len=[2048, 1999])
    bt = st.kv.block_table
    t = np.arange(st.kv.L_max)
    tt = (bt[:, t // 16] * 16 + t % 16).astype(np.int32)
    tt[np.random.default_rng(3).random(tt.shape) < 0.25] = -1
    st.kv.token_table, st.kv.block_table = tt, None
    assert _fused_vs_oracle(st) == 0
    st = W.make_gqa_paged(tag=411, B=2, H=2, G=4, L=1008, k=64, seq_len=[1008, 611])
    for name in ("k", "v"):
        pool = getattr(st.kv, name)
        logical = pool[st.kv.block_table]
        setattr(st.kv, name, np.ascontiguousarray(logical.transpose(0, 2, 1, 3, 4).reshape(2, 2, 1008, 128)))
    st.kv.block, st.kv.block_table = 0, None
    assert _fused_vs_oracle(st) == 0


def test_fused_windows_k_ge_candidates_ties_and_empty():
    st = W.make_gqa_paged(tag=412, B=3, H=2, G=4, L=512, k=512, sink=4, local=64)
    st.lo = np.array([4, 100, 0], np.int32)
    st.hi = np.array([448, 100, 512], np.int32)            # row 1: no candidates
    assert _fused_vs_oracle(st) == 0
    st.k = 1
    assert _fused_vs_oracle(st) == 0
    # exact ties: integer keys, all-ones query
    st = W.make_gqa_paged(tag=413, B=1, H=2, G=2, L=1024, k=100, sink=0, local=0)
    vals = np.random.default_rng(5).integers(-1, 2, size=st.kv.k.shape).astype(np.float32)
    st.kv.k = W.f32_to_bf16_bits(vals)
    st.q = W.f32_to_bf16_bits(np.ones_like(D.bf16_bits_to_f64(st.q), dtype=np.float32))
    st.score_kv, st.score_q = st.kv, st.q
    r = Run(st)
    _, idx, _, out = r.select_attend()
    ref = D.step(st)
    for h in range(2):
        assert idx.cpu().numpy()[0, h].tolist() == sorted(ref["idx"][0, h].tolist())
    assert np.abs(out.cpu().numpy() - ref["out"]).max() <= ATTN_TOL


def test_fused_unmapped_blocks_and_large_window():
    st = W.make_gqa_paged(tag=414, B=2, H=2, G=4, L=8192, k=1000, sink=300, local=900,
                          seq_len=[8192, 6000])
    st.kv.block_table[0, [2, 3, 100, 511]] = -1
    st.kv.block_table[1, [0, 40]] = -1
    assert _fused_vs_oracle(st) == 0


def test_fused_repeated_calls_share_one_workspace():
    st = W.make_gqa_paged(tag=415, B=2, H=4, G=4, L=8192, k=700, seq_len=[8192, 5000])
    r = Run(st)
    ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT_ATTEND, r.kv, 4, st.k), DEV)
    first = [t.clone() for t in r.select_attend(ws=ws)]
    for _ in range(3):
        again = r.select_attend(ws=ws)
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    rows = st.kv.B * st.kv.H
    assert torch.count_nonzero(ws[: rows * 4096 * 4]).item() == 0    # histograms back to zero


@pytest.mark.slow
def test_fused_full_size_every_row():
    """The fused step on the full GQA decode (L = 32768), all 32 rows."""
    st = W.make_gqa_paged()
    assert _fused_vs_oracle(st) == 0


def test_fused_rejects_unsupported_shapes():
    st = W.make_gqa_paged(tag=416, B=1, H=1, G=16, L=256, k=16)
    r = Run(st)
    with pytest.raises(S.SkvError):
        r.select_attend()
