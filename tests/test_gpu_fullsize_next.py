"""Full-size checks of the later rows, in the configurations bench.py times,
on outputs the oracle can compute one by one: token-table compaction of the
full token pool (the library's plans equal the oracle's for sampled
sequences, the pool and table after applying every plan equal the oracle's
apply on those sequences' rows, the I1 hash of sampled sequences equals the
oracle's before and after, no duplicate slot), and a full-size decode with
the 512-token Update Buffer (the flushed entries equal the oracle's encoding
of those keys, the histogram grows by exactly their centroid counts, and the
retrieval after the flush stays inside the grown region)."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import compact as C
from oracle import lloyd
from oracle import paris as P

from gpu_helpers import DEV, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_compaction_full_token_pool():
    st = W.make_token_pool(spare_blocks=2048)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    say("compaction full size", st.name, "blocks", n_blocks)
    kv_d = S.kv_to_device(kv, DEV)
    sample = [0, 13, 31]
    h_gpu, c_gpu = S.sparsekv_live_hash(kv_d)
    h_gpu = h_gpu.cpu().numpy().view(np.uint64)
    for b in sample:
        assert (int(h_gpu[b]), int(c_gpu[b])) == C.live_hash(kv, b), b
    before = h_gpu.copy()
    free = [int(x) for x in st.meta["free_blocks"]]
    counts = C.occupancy(kv.token_table, kv.seq_len, n_blocks).astype(np.int32)
    moved = {}
    for b in range(kv.B):
        moves, src, n_dst = S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, b, free,
                                                    len(free), 0.25, 64, counts=counts)
        if b in sample:
            r_moves, r_src, r_dst = C.plan(kv.token_table, kv.seq_len, n_blocks, b, free,
                                           len(free), 0.25, 64)
            assert [tuple(m[1:]) for m in moves.tolist()] == r_moves and src.tolist() == r_src
            moved[b] = r_moves
        assert len(moves) > 0 and len(src) > n_dst
        S.sparsekv_compact_apply(kv_d, torch.from_numpy(moves).to(DEV))
        # the host table and counts follow, as a caller's would
        for (_, t, s_, d_) in moves.tolist():
            kv.token_table[b, t] = d_
        for p_ in src:
            counts[p_] = 0
        for j, p_ in enumerate(free[:n_dst]):
            counts[p_] = min(16, len(moves) - 16 * j)
        free = free[n_dst:]
    torch.cuda.synchronize()
    tt = kv_d.token_table.cpu().numpy()
    assert np.array_equal(tt, kv.token_table)
    # the moved rows of the sampled sequences landed where the oracle puts them
    k_d = kv_d.k.view(torch.int16)
    v_d = kv_d.v.view(torch.int16)
    for b, mv in moved.items():
        for (t, s_, d_) in mv[:: max(1, len(mv) // 64)]:
            for arr, dev_arr in ((kv.k, k_d), (kv.v, v_d)):
                got = dev_arr[d_ // 16, :, d_ % 16].cpu().numpy().view(np.uint16)
                assert np.array_equal(got, arr[s_ // 16, :, s_ % 16]), (b, t)
    h_after, c_after = S.sparsekv_live_hash(kv_d)
    h_after = h_after.cpu().numpy().view(np.uint64)
    assert np.array_equal(h_after, before)                        # I1, every sequence
    assert S.sparsekv_check_unique(kv_d, n_blocks).cpu().tolist() == [0, 0]   # I2


def test_update_buffer_flush_full_size():
    p = W.make_paris()
    lv, th = lloyd.codebook_f32(8)
    cb = S.new_codebook(torch.from_numpy(p.signs).to(DEV))
    U = 512
    L0 = p.L - 600
    n0 = L0 - p.sink - p.local
    say("update buffer full size", p.name, "L0", L0, "n0", n0)
    kvn = p.kv()
    kvn.seq_len = np.array([L0], np.int32)
    kv = S.kv_to_device(kvn, DEV)
    cap = p.L - p.sink - p.local
    index = S.new_index(p.H, cap, device=DEV)
    S.sparsekv_encode(cb, kv, 0, p.sink, p.sink + n0, index)
    hist0 = index.hist.cpu().numpy().copy()
    flushed = 0
    for i in range(600):
        seq = L0 + 1 + i
        kv.seq_len.fill_(seq)
        flushed += S.sparsekv_update_buffer(cb, kv, 0, seq, p.sink, p.local, U, index)
    torch.cuda.synchronize()
    assert flushed == 1 and index.n == n0 + U
    t0 = p.sink + n0
    ids = index.ids[:, n0:n0 + U].cpu().numpy()
    codes = index.codes[:, n0:n0 + U].cpu().numpy()
    w = index.w[:, n0:n0 + U].cpu().numpy()
    for h in range(p.H):
        r_ids, r_codes, r_w, _ = P.encode_keys(p.keys[h, t0:t0 + U], p.signs, p.n_sub, lv, th)
        assert np.array_equal(ids[h], r_ids) and np.array_equal(codes[h], r_codes), h
        assert np.array_equal(w[h].view(np.uint32), r_w.view(np.uint32)), h
        grown = index.hist[h].cpu().numpy() - hist0[h]
        assert np.array_equal(grown, P.histogram(r_ids, 256)), h
    assert np.array_equal(index.pos[n0:n0 + U].cpu().numpy(), np.arange(t0, t0 + U))
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, _ = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final)
    idx, n_cand = idx.cpu().numpy(), n_cand.cpu().numpy()
    assert np.all(n_cand == p.k_final)
    assert np.all((idx >= p.sink) & (idx < p.sink + index.n))
