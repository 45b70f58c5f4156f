"""GPU parity of token-table compaction (sparsekv_compact_apply) and of the
I1 / I2 checks (sparsekv_live_hash, sparsekv_check_unique) against the
oracle: the pool and the token table after applying the library's plans are
byte-identical to the oracle's, the hashes and duplicate counts equal the
oracle's before and after, and a decode step over the compacted pool gives
bit-identical scores, selection and attention."""
import copy

import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import compact as C

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def _hashes(kv_d):
    h, c = S.sparsekv_live_hash(kv_d)
    return h.cpu().numpy().view(np.uint64).tolist(), c.cpu().numpy().tolist()


def _oracle_hashes(kv):
    r = [C.live_hash(kv, b) for b in range(kv.B)]
    return [x[0] for x in r], [x[1] for x in r]


def _pool_bytes(kv_d):
    return (kv_d.k.view(torch.int16).cpu().numpy().view(np.uint16),
            kv_d.v.view(torch.int16).cpu().numpy().view(np.uint16),
            kv_d.token_table.cpu().numpy())


@pytest.mark.parametrize("d,max_src", [(128, 8), (64, 64)])
def test_compaction_matches_oracle_and_keeps_invariants(d, max_src):
    st = W.make_token_pool(tag=90 + d, B=3, H=2, d=d, L=1024, k=64, sink=4, local=32,
                           spare_blocks=96)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    say("compact", st.name, "d", d, "max_src", max_src, "n_blocks", n_blocks)
    kv_d = S.kv_to_device(kv, DEV)
    assert _hashes(kv_d) == _oracle_hashes(kv)
    assert S.sparsekv_check_unique(kv_d, n_blocks).cpu().tolist() == [0, 0]
    h0 = _hashes(kv_d)
    ref = copy.deepcopy(kv)
    free = list(st.meta["free_blocks"])
    total = 0
    for b in range(kv.B):
        tt_host = kv_d.token_table.cpu().numpy()
        moves, src, n_dst = S.sparsekv_compact_plan(tt_host, kv.seq_len, n_blocks, b, free,
                                                    len(free), 0.25, max_src)
        r_moves, r_src, r_dst = C.plan(ref.token_table, ref.seq_len, n_blocks, b, free, len(free),
                                       0.25, max_src)
        assert [tuple(m[1:]) for m in moves.tolist()] == r_moves and src.tolist() == r_src
        assert len(moves) > 0 and len(src) > n_dst
        S.sparsekv_compact_apply(kv_d, torch.from_numpy(moves).to(DEV))
        C.apply(ref, b, r_moves)
        free = free[n_dst:] + src.tolist()        # freed sources return to the pool
        total += len(moves)
    torch.cuda.synchronize()
    k, v, tt = _pool_bytes(kv_d)
    assert np.array_equal(tt, ref.token_table)
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
    assert _hashes(kv_d) == h0 == _oracle_hashes(ref)                   # I1
    assert S.sparsekv_check_unique(kv_d, n_blocks).cpu().tolist() == [0, 0]   # I2
    say("  moved", total)


def test_decode_step_identical_after_compaction():
    st = W.make_token_pool(tag=95, B=2, H=2, d=128, L=2048, k=128, sink=4, local=64,
                           spare_blocks=200)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    kv_d = S.kv_to_device(kv, DEV)
    q = S.to_device(st.q, DEV, True)
    lo = S.to_device(st.lo.astype(np.int32), DEV)
    hi = S.to_device(st.hi.astype(np.int32), DEV)

    def step():
        sc, idx, cnt = S.sparsekv_select(kv_d, q, 1, lo, hi, st.k)
        out = S.sparsekv_gather_attend(kv_d, q, 1, idx, st.k, lo, hi, st.scale)
        torch.cuda.synchronize()
        return [x.cpu().numpy() for x in (sc, idx, cnt, out)]

    before = step()
    free = list(st.meta["free_blocks"])
    moved = 0
    for _ in range(3):                    # several rounds per sequence
        for b in range(kv.B):
            moves, src, n_dst = S.sparsekv_compact_plan(kv_d.token_table.cpu().numpy(), kv.seq_len,
                                                        n_blocks, b, free, len(free), 0.25, 32)
            if len(moves):
                S.sparsekv_compact_apply(kv_d, torch.from_numpy(moves).to(DEV))
                free = free[n_dst:] + src.tolist()
                moved += len(moves)
    after = step()
    say("compacted", moved, "tokens")
    assert moved > 0
    for a, b_ in zip(before, after):
        assert np.array_equal(a.view(np.uint8), b_.view(np.uint8))


def test_checks_detect_broken_invariants():
    st = W.make_token_pool(tag=97, B=2, H=2, d=64, L=512, k=16, sink=4, local=16, spare_blocks=8)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    kv_d = S.kv_to_device(kv, DEV)
    h0 = _hashes(kv_d)
    live = np.nonzero(kv.token_table[1] >= 0)[0]
    s = int(kv.token_table[1, live[3]])
    # one bit of a live value row (I1 broken for sequence 1 only)
    kv.v[s // 16, 1, s % 16, 5] ^= 1
    kv_d.v.view(torch.int16)[s // 16, 1, s % 16, 5] ^= 1
    h1 = _hashes(kv_d)
    assert h1[0][0] == h0[0][0] and h1[0][1] != h0[0][1] and h1[1] == h0[1]
    assert h1 == _oracle_hashes(kv)
    # two live tokens on one slot, one slot outside the pool (I2 broken)
    kv.token_table[1, live[4]] = kv.token_table[1, live[5]]
    kv.token_table[0, np.nonzero(kv.token_table[0] >= 0)[0][0]] = n_blocks * 16 + 3
    kv_d.token_table.copy_(torch.from_numpy(kv.token_table))
    got = S.sparsekv_check_unique(kv_d, n_blocks).cpu().tolist()
    assert got == list(C.duplicate_slots(kv.token_table, kv.seq_len, n_blocks)) == [1, 1]


@pytest.mark.parametrize("layout", ["paged", "contiguous", "latent"])
def test_live_hash_every_layout(layout):
    """sparsekv_live_hash against the oracle on a block-table pool (with an
    unmapped block), contiguous storage and a latent pool without values."""
    if layout == "paged":
        st = W.make_gqa_paged(tag=992, B=2, H=3, G=2, d=128, L=512, k=16, sink=4, local=16,
                              seq_len=[512, 301])
        st.kv.block_table[1, 2] = -1
        kv = st.kv
    elif layout == "contiguous":
        kv = W.make_paris(tag=993, H=2, G=1, L=1000, sink=4, local=16).kv()
        kv.seq_len = np.array([777], np.int32)
    else:
        kv = W.make_indexer_mla(tag=994, L=1024, n_heads=16, k=64).kv
    kv_d = S.kv_to_device(kv, DEV)
    assert _hashes(kv_d) == _oracle_hashes(kv)


def test_apply_skips_moves_outside_the_table_or_pool():
    """Moves whose sequence, token or slots fall outside the table or the pool
    are skipped before any address is formed and counted into err; the valid
    moves of the same launch are applied exactly as the oracle applies them."""
    st = W.make_token_pool(tag=97, B=2, H=2, d=128, L=512, k=16, sink=4, local=16,
                           spare_blocks=16)
    kv = st.kv
    n_blocks = kv.k.shape[0]
    n_slots = n_blocks * 16
    kv_d = S.kv_to_device(kv, DEV)
    free = list(st.meta["free_blocks"])
    moves, src, n_dst = S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, 0, free,
                                                len(free), 0.0, 4)
    assert len(moves) > 0
    ref = copy.deepcopy(kv)
    C.apply(ref, 0, [tuple(m[1:]) for m in moves.tolist()])
    good = moves.tolist()
    t_dead = int(np.nonzero(kv.token_table[1] < 0)[0][0])
    bad = [[0, good[0][1], good[0][2], n_slots],        # dst past the pool
           [0, good[0][1], n_slots + 5, good[0][3]],    # src past the pool
           [1, t_dead, -3, good[0][3]],                 # negative src
           [2, 0, good[0][2], good[0][3]],              # sequence past B
           [0, kv.L_max, good[0][2], good[0][3]]]       # token past L_max
    mixed = np.array(bad[:2] + good + bad[2:], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("compact skip", len(good), "valid moves,", len(bad), "invalid")
    S.sparsekv_compact_apply(kv_d, torch.from_numpy(mixed).to(DEV), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == len(bad)
    k, v, tt = _pool_bytes(kv_d)
    assert np.array_equal(tt, ref.token_table)
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
