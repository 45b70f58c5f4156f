"""GPU parity of the dense-path kernels (score scan, exact top-k, gather +
split-k attention) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D

from gpu_helpers import ATTN_TOL, DEV, Run, check_scores, check_selection, say

pytestmark = pytest.mark.gpu


def _all_rows(st):
    return [(b, h) for b in range(st.score_kv.B) for h in range(st.score_kv.H)]


def _end_to_end(st, rows=None, check_all_rows=True, attend=True, fused=True):
    rows = _all_rows(st) if rows is None else rows
    say("case", st.name, "B", st.kv.B, "H", st.kv.H, "G", st.G, "L", st.kv.L_max, "k", st.k,
        "mode", st.kv.mode)
    r = Run(st)
    if attend:
        sc, idx, cnt, out = r.step(fused=fused)
        out = out.cpu().numpy()
    else:
        sc = r.score()
        idx, cnt = r.topk(sc)
        out = None
    sc, idx, cnt = sc.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    worst = check_scores(st, sc, rows)
    ref = D.step(st, rows=rows)
    swaps = 0
    for b, h in rows:
        s_ref = ref["scores"][b, h]
        sel = ref["idx"][b, h][: ref["count"][b, h]]
        assert cnt[b, h] == ref["count"][b, h]
        sw = check_selection(s_ref, sel, idx[b, h], cnt[b, h])
        swaps += sw
        if sw == 0 and out is not None:
            hs = range(h * st.G, (h + 1) * st.G)
            err = np.abs(out[b, list(hs)] - ref["out"][b, list(hs)]).max()
            assert err <= ATTN_TOL, (b, h, err)
    say("  worst score err / bound", worst, "swaps", swaps)
    if check_all_rows:
        B, H = st.score_kv.B, st.score_kv.H
        assert out is None or np.all(np.isfinite(out))
        for b in range(B):
            for h in range(H):
                got = idx[b, h][: cnt[b, h]]
                assert np.all((got >= st.lo[b]) & (got < st.hi[b]))
    return swaps


def test_single_head_fp32_full():
    st = W.make_single_head()
    assert _end_to_end(st) == 0
    # planted keys are mostly recovered (reported, not a parity criterion)
    r = Run(st)
    _, idx, cnt, _ = r.step()
    got = set(idx.cpu().numpy()[0, 0].tolist())
    say("  planted recovered", len(got & set(st.meta["planted"].tolist())), "of 8")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_paged_small(G):
    st = W.make_gqa_paged(tag=100 + G, B=2, H=3, G=G, L=2048, k=256, sink=4, local=64,
                          seq_len=[2048, 1509])
    assert _end_to_end(st) == 0
    assert _end_to_end(st, fused=False) == 0


def test_gqa_paged_g16_mfma_cross_lane_max():
    """G = 16 spreads the group over all four C row-groups of the MFMA tile;
    scoring and selection only (the vector attention path stops at G = 8)."""
    st = W.make_gqa_paged(tag=116, B=1, H=2, G=16, L=1024, k=128, sink=4, local=64)
    assert _end_to_end(st, attend=False) == 0


@pytest.mark.parametrize("tag", [201, 202])
def test_select_equals_score_then_topk(tag):
    """The fused scan + top-k returns the same scores and the same selection as
    the two separate calls (several calls reuse one workspace)."""
    st = W.make_gqa_paged(tag=tag, B=2, H=2, G=4, L=8192, k=700, sink=4, local=64,
                          seq_len=[8192, 5000])
    r = Run(st)
    ws = S.workspace(S.sparsekv_workspace_size(S.SKV_OP_SELECT, r.skv, 4, st.k), DEV)
    for _ in range(3):
        sc1, idx1, cnt1 = S.sparsekv_select(r.skv, r.sq, 4, r.lo, r.hi, st.k, ws=ws)
        sc2 = r.score()
        idx2, cnt2 = S.sparsekv_topk(sc2, r.lo, r.hi, st.k, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(sc1, sc2)
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2)
    # the counters at the front of the workspace are back to zero
    rows = 4
    al = lambda x: (x + 255) // 256 * 256
    zero_region = al(rows * 4096 * 4)
    assert torch.count_nonzero(ws[:zero_region]).item() == 0


def test_token_pool_small():
    st = W.make_token_pool(tag=120, B=3, H=2, L=4096, k=256, sink=4, local=128)
    assert _end_to_end(st) == 0


def test_contiguous_bf16_and_fp32_g4():
    st = W.make_gqa_paged(tag=121, B=2, H=2, G=4, L=1024, k=64)
    # re-lay the paged pool as contiguous [B][H][L][d]
    for name in ("k", "v"):
        pool = getattr(st.kv, name)
        logical = pool[st.kv.block_table]                    # [B][nb][H][16][d]
        cont = np.ascontiguousarray(logical.transpose(0, 2, 1, 3, 4).reshape(2, 2, 1024, 128))
        setattr(st.kv, name, cont)
    st.kv.block, st.kv.block_table = 0, None
    assert _end_to_end(st) == 0
    st32 = W.make_single_head(tag=122, L=3000, d=64, k=100)
    assert _end_to_end(st32) == 0


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_scan_slices_cross_rows_and_ragged_lengths(G):
    """Row lengths that are not a multiple of the per-workgroup slice, so
    workgroup slices of the persistent scan straddle rows; ragged seq_len
    (including one shorter than a chunk)."""
    st = W.make_gqa_paged(tag=150 + G, B=3, H=5, G=G, L=1040, k=100, sink=4, local=16,
                          seq_len=[1040, 777, 33])
    assert _end_to_end(st, attend=G <= 16) == 0


def test_scan_contiguous_ragged_tail_chunk():
    """Contiguous store with L_max = 1000 (last chunk of each row is partial)."""
    st = W.make_gqa_paged(tag=157, B=2, H=2, G=4, L=1008, k=64, seq_len=[1008, 611])
    Lc = 1000
    for name in ("k", "v"):
        pool = getattr(st.kv, name)
        logical = pool[st.kv.block_table]                    # [B][nb][H][16][d]
        cont = logical.transpose(0, 2, 1, 3, 4).reshape(2, 2, 1008, 128)[:, :, :Lc]
        setattr(st.kv, name, np.ascontiguousarray(cont))
    st.kv.block, st.kv.block_table, st.kv.L_max = 0, None, Lc
    st.kv.seq_len = np.array([1000, 611], np.int32)
    st.hi = (st.kv.seq_len - 64).astype(np.int32)
    assert _end_to_end(st) == 0


def test_scan_token_table_gqa_and_unmapped_blocks():
    """G = 4 through a per-token table with holes, and through a block table
    with unmapped (negative) blocks."""
    st = W.make_gqa_paged(tag=158, B=2, H=3, G=4, L=2048, k=200, sink=4, local=64,
                          seq_len=[2048, 1500])
    bt = st.kv.block_table
    t = np.arange(st.kv.L_max)
    tt = (bt[:, t // 16] * 16 + t % 16).astype(np.int32)
    holes = np.random.default_rng(9).random(tt.shape) < 0.3
    tt[holes] = -1
    tt[:, :4] = bt[:, :1] * 16 + np.arange(4)                # keep the sink live
    st.kv.token_table, st.kv.block_table = tt, None
    assert _end_to_end(st) == 0
    st = W.make_gqa_paged(tag=159, B=2, H=3, G=4, L=2048, k=200, sink=4, local=64,
                          seq_len=[2048, 1500])
    st.kv.block_table[0, [3, 4, 50, 127]] = -1
    st.kv.block_table[1, [0, 20]] = -1
    assert _end_to_end(st) == 0


@pytest.mark.parametrize("d", [64, 128, 256])
def test_scan_single_query_head_dims_and_tables(d):
    """G = 1 (vector-ALU dot in the persistent scan) for d = 64, 128, 256,
    through the block table and through a token table with holes."""
    st = W.make_gqa_paged(tag=170 + d // 64, B=2, H=3, G=1, d=d, L=1040, k=90, sink=4, local=16,
                          seq_len=[1040, 517])
    assert _end_to_end(st, attend=d == 128) == 0
    bt = st.kv.block_table
    t = np.arange(st.kv.L_max)
    tt = (bt[:, t // 16] * 16 + t % 16).astype(np.int32)
    tt[np.random.default_rng(d).random(tt.shape) < 0.4] = -1
    tt[:, :4] = bt[:, :1] * 16 + np.arange(4)
    st.kv.token_table, st.kv.block_table = tt, None
    assert _end_to_end(st, attend=d == 128) == 0


@pytest.mark.parametrize("d,attend", [(64, False), (256, True)])
def test_scan_other_head_dims(d, attend):
    st = W.make_gqa_paged(tag=160 + d // 64, B=2, H=2, G=4, d=d, L=1024, k=100, sink=4, local=16,
                          seq_len=[1024, 999])
    assert _end_to_end(st, attend=attend) == 0


def test_edges_k_ge_candidates_empty_window_and_k1():
    st = W.make_gqa_paged(tag=130, B=3, H=2, G=4, L=512, k=512, sink=4, local=64)
    st.lo = np.array([4, 100, 0], np.int32)
    st.hi = np.array([448, 100, 512], np.int32)            # row 1: no candidates
    assert _end_to_end(st) == 0
    st.k = 1
    assert _end_to_end(st) == 0


def test_all_dead_tokens_give_zero_output():
    st = W.make_token_pool(tag=131, B=2, H=2, L=256, k=32, sink=4, local=16)
    st.kv.token_table[1, :] = -1
    st.lo[1], st.hi[1] = 256, 256
    r = Run(st)
    sc, idx, cnt, out = r.step()
    assert int(cnt[1, 0]) == 0 and int(cnt[1, 1]) == 0
    assert np.all(out.cpu().numpy()[1] == 0)
    assert np.all(np.isneginf(sc.cpu().numpy()[1]))
    assert _end_to_end(st, rows=[(0, 0), (0, 1)], check_all_rows=False) == 0


def test_exact_ties_lowest_index_wins():
    """Integer-valued keys and an all-ones query make exact score ties; the
    selected set must equal the oracle's exactly (lowest index first)."""
    st = W.make_gqa_paged(tag=132, B=1, H=2, G=1, L=1024, k=100, sink=0, local=0)
    rng = np.random.default_rng(5)
    vals = rng.integers(-1, 2, size=st.kv.k.shape).astype(np.float32)
    st.kv.k = W.f32_to_bf16_bits(vals)
    st.q = W.f32_to_bf16_bits(np.ones_like(D.bf16_bits_to_f64(st.q), dtype=np.float32))
    st.score_kv, st.score_q = st.kv, st.q
    r = Run(st)
    sc, idx, cnt, _ = r.step()
    idx = idx.cpu().numpy()
    ref = D.step(st)
    for h in range(2):
        assert idx[0, h].tolist() == sorted(ref["idx"][0, h].tolist())


# --------------------------------------------------------------- top-k alone
@pytest.mark.parametrize("L,k,seed", [(1000, 37, 0), (4096, 2048, 1), (32768, 2048, 2),
                                      (40000, 700, 3), (131072, 2048, 4), (5000, 4999, 5),
                                      (32768, 2048, 6), (70001, 3000, 7), (32767, 1000, 8),
                                      (32765, 2048, 9), (4097, 100, 10), (200003, 2500, 11),
                                      (150001, 2048, 12)])
def test_topk_kernel_on_oracle_inputs(L, k, seed):
    """Synthetic rows with ties, -0.0 / +0.0, -inf and windows; the GPU set must
    equal the oracle's set exactly.  Row lengths that are not multiples of 4
    put row and window starts at every offset from a 16-byte boundary."""
    say("topk", L, k, seed)
    rng = np.random.default_rng(seed)
    B, H = 2, 2
    s = W.normal_f32(W.seed_of(1000 + seed), 0, (B, H, L)) * 10
    s[0, 1] = np.round(s[0, 1])                              # many exact ties
    s[1, 0, ::7] = -0.0
    s[1, 0, 3::7] = 0.0
    s[1, 1, rng.random(L) < 0.3] = -np.inf                   # dead tokens
    if seed >= 6:
        s[0, 0] = 1.5                                        # one value: every key ties
    lo = np.array([3, 0], np.int32)
    hi = np.array([L - 5, L], np.int32)
    sd = torch.from_numpy(s).to(DEV)
    idx, cnt = S.sparsekv_topk(sd, S.to_device(lo, DEV), S.to_device(hi, DEV), k)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = D.select_topk(s[b, h].astype(np.float64), int(lo[b]), int(hi[b]), k)
            assert cnt[b, h] == ref.size
            assert idx[b, h, : ref.size].tolist() == sorted(ref.tolist()), (b, h)
            assert np.all(idx[b, h, ref.size:] == -1)


@pytest.mark.parametrize("B,H,L,k", [(32, 8, 65536, 2048), (16, 4, 131072, 2048),
                                     (8, 4, 131072, 4000), (1, 1, 131072, 2048),
                                     (1, 2, 131072, 14000), (1, 2, 131072, 15500),
                                     (1, 1, 131072, 20000)])
def test_topk_listing_slice_sizes(B, H, L, k):
    """Many rows take 8192-slot listing slices, fewer rows smaller ones (4096,
    2048, 1024 slots); every row's set equals the oracle's, windows ragged.
    Large k put the list (each slice's share padded to 4 entries) near and
    past its 16,384-entry capacity, where the row is selected from the
    scores instead."""
    say("topk slices", B, H, L, k)
    s = W.normal_f32(W.seed_of(1100 + B), 0, (B, H, L)) * 10
    lo = (np.arange(B, dtype=np.int32) * 37) % 1000
    hi = (L - (np.arange(B, dtype=np.int32) * 53) % 999).astype(np.int32)
    sd = torch.from_numpy(s).to(DEV)
    idx, cnt = S.sparsekv_topk(sd, S.to_device(lo, DEV), S.to_device(hi, DEV), k)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = D.select_topk(s[b, h].astype(np.float64), int(lo[b]), int(hi[b]), k)
            assert cnt[b, h] == ref.size
            assert idx[b, h, : ref.size].tolist() == sorted(ref.tolist()), (b, h)


# ------------------------------------------------------------ attention alone
@pytest.mark.parametrize("G", [1, 4, 8])
def test_attend_kernel_on_oracle_selection(G):
    st = W.make_gqa_paged(tag=140 + G, B=2, H=2, G=G, L=4096, k=512, sink=4, local=64,
                          seq_len=[4096, 3001])
    ref = D.step(st)
    r = Run(st)
    idx = torch.from_numpy(ref["idx"].astype(np.int32)).to(DEV)
    out = r.attend(idx).cpu().numpy()
    err = np.abs(out - ref["out"]).max()
    say("  attend G", G, "max err", err)
    assert err <= ATTN_TOL


# ----------------------------------------------------- full-size workloads
@pytest.mark.slow
def test_gqa_paged_full_size_every_row():
    """All 32 (sequence, KV head) rows of the GQA decode at L = 32768."""
    st = W.make_gqa_paged()
    assert _end_to_end(st) == 0


@pytest.mark.slow
def test_gqa_paged_long_context_every_row():
    """The GQA decode at L = 131072, all 32 rows: rows longer than one
    workgroup's sweep go through the sliced top-k."""
    st = W.make_gqa_paged(L=131072)
    assert _end_to_end(st) == 0


def _token_pool_rows():
    """64 of the 256 rows: two KV heads of every sequence, each head 8 times."""
    return [(b, (b + 4 * j) % 8) for b in range(32) for j in range(2)]


@pytest.mark.slow
def test_token_pool_full_size_64_rows_over_every_head():
    st = W.make_token_pool()
    rows = _token_pool_rows()
    assert sorted(set(h for _, h in rows)) == list(range(8))
    assert _end_to_end(st, rows=rows) == 0


# ------------------------------------------- indexer + shared-latent attention
@pytest.mark.parametrize("L,k,heads", [(4096, 256, 128), (2048, 300, 16), (1024, 77, 64)])
def test_indexer_mla_small(L, k, heads):
    st = W.make_indexer_mla(tag=300 + heads, L=L, k=k, n_heads=heads)
    assert _end_to_end(st) == 0


def test_mla_with_sink_local_and_ragged_tail():
    st = W.make_indexer_mla(tag=310, L=2048, k=200, n_heads=32)
    st.lo = np.array([4], np.int32)
    st.hi = np.array([2048 - 70], np.int32)
    assert _end_to_end(st) == 0


def test_mla_attend_kernel_on_oracle_selection():
    st = W.make_indexer_mla(tag=311, L=8192, k=1000, n_heads=128)
    ref = D.step(st)
    r = Run(st)
    idx = torch.from_numpy(ref["idx"].astype(np.int32)).to(DEV)
    out = r.attend(idx).cpu().numpy()
    err = np.abs(out - ref["out"]).max()
    say("  mla max err", err)
    assert err <= ATTN_TOL


@pytest.mark.slow
def test_indexer_mla_full_size():
    st = W.make_indexer_mla()
    assert _end_to_end(st) == 0


@pytest.mark.parametrize("L,k,seed", [(20962, 100, 0), (20962, 256, 1), (4096, 1, 2),
                                      (30000, 200, 3), (777, 256, 4)])
def test_topk_small_k_narrow_score_range(L, k, seed):
    """Small k over rows of one sweep whose scores span one octave (like the
    rerank estimates of a retrieval): exact ties, dead slots and ragged
    windows; the set equals the oracle's exactly."""
    say("topk small", L, k, seed)
    rng = np.random.default_rng(50 + seed)
    B, H = 2, 4
    s = (1.0 + 0.5 * rng.random((B, H, L))).astype(np.float32)
    s[0, 1] = np.round(s[0, 1] * 64) / 64                   # exact ties
    s[1, 2, rng.random(L) < 0.4] = -np.inf                   # dead slots
    s[1, 3, : L // 2] = 1.25                                 # a tied block
    lo = np.array([0, 5], np.int32)
    hi = np.array([L, L - 3], np.int32)
    sd = torch.from_numpy(s).to(DEV)
    idx, cnt = S.sparsekv_topk(sd, S.to_device(lo, DEV), S.to_device(hi, DEV), k)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = D.select_topk(s[b, h].astype(np.float64), int(lo[b]), int(hi[b]), k)
            assert cnt[b, h] == ref.size
            assert idx[b, h, : ref.size].tolist() == sorted(ref.tolist()), (b, h)
            assert np.all(idx[b, h, ref.size:] == -1)
