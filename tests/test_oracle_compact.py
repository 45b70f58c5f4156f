"""Pins of the compaction oracle (no GPU): the page's worked example of the
relocation stages, the gates that reject a plan (threshold, headroom, net
freeing, shared blocks), token conservation and unique mapping after
applying a plan to a token pool, and the hash's primitive and properties."""
import json
import os

import numpy as np

import workloads as W
from oracle import compact as C
from oracle import dense as D

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _table(blocks_live, B=1, extra=None):
    """Sequence 0 holds blocks 0..len-1 with the given live counts (its
    tokens t = 16 j + e, the first n of each block live)."""
    nb = len(blocks_live)
    tt = np.full((B, 16 * nb), -1, np.int32)
    for j, n in enumerate(blocks_live):
        for e in range(n):
            tt[0, 16 * j + e] = 16 * j + e
    if extra:
        for (b, t, slot) in extra:
            tt[b, t] = slot
    return tt, np.full(B, 16 * nb, np.int32)


def test_worked_example_of_the_page():
    g = GOLD["waste_ratio"]
    assert abs(C.waste_ratio(g["n_live"]) - g["F"]) < 1e-12
    tt, sl = _table(g["n_live"])
    n_blocks = 3 + g["free_blocks"] + g["headroom_blocks"]
    free = list(range(3, n_blocks))
    moves, src, dst = C.plan(tt, sl, n_blocks, 0, free, g["free_blocks"] + g["headroom_blocks"],
                             0.25, 8)
    assert len(moves) == g["T_live"]
    assert len(dst) == g["target_blocks"] and len(src) - len(dst) == g["net_freed"]
    assert sorted(src) == [0, 1, 2] and dst == [3]
    # logical order kept, the target block filled from offset 0
    assert [m[0] for m in moves] == sorted(m[0] for m in moves)
    assert [m[2] for m in moves] == list(range(48, 48 + 12))


def test_gates_reject_or_shrink():
    # net freeing: 9 + 8 live -> 2 targets for 2 sources, then 1 for 1: no plan
    tt, sl = _table([9, 8])
    assert C.plan(tt, sl, 6, 0, [2, 3, 4, 5], 4, 0.0, 8) == ([], [], [])
    # 7 + 8 + 9 = 24 -> 2 targets for 3 sources
    tt, sl = _table([9, 8, 7])
    moves, src, dst = C.plan(tt, sl, 6, 0, [3, 4, 5], 3, 0.0, 8)
    assert len(moves) == 24 and sorted(src) == [0, 1, 2] and dst == [3, 4]
    # headroom: only one target may be consumed -> the fullest candidates go
    tt, sl = _table([10, 10, 10, 4, 3])
    moves, src, dst = C.plan(tt, sl, 8, 0, [5, 6, 7], 1, 0.0, 8)
    assert sorted(src) == [3, 4] and dst == [5] and len(moves) == 7
    assert C.plan(tt, sl, 8, 0, [5, 6, 7], 0, 0.0, 8) == ([], [], [])
    # max_src caps the candidates (lowest utilisation first)
    moves, src, dst = C.plan(tt, sl, 8, 0, [5, 6, 7], 3, 0.0, 2)
    assert sorted(src) == [3, 4]
    # threshold: F = 1 - (16 + 16 + 15) / 48 is below 0.25 -> no plan
    tt, sl = _table([16, 16, 15, 0])
    assert C.plan(tt, sl, 6, 0, [4, 5], 2, 0.25, 8) == ([], [], [])


def test_shared_block_is_not_a_source():
    # block 1 also holds a live token of sequence 1: only blocks 0 and 2 move
    tt, sl = _table([2, 3, 4], B=2, extra=[(1, 0, 16 + 15)])
    sl[1] = 1
    moves, src, dst = C.plan(tt, sl, 5, 0, [3, 4], 2, 0.0, 8)
    assert sorted(src) == [0, 2] and dst == [3] and len(moves) == 6


def _pool(tag=81, B=3, L=512, spare=40):
    st = W.make_token_pool(tag=tag, B=B, H=2, d=64, L=L, k=32, sink=4, local=16,
                           spare_blocks=spare)
    return st.kv, list(st.meta["free_blocks"])


def test_apply_conserves_tokens_and_mapping():
    kv, free = _pool()
    n_blocks = kv.k.shape[0]
    before = [D.logical_kv(kv, b, h) for b in range(kv.B) for h in range(kv.H)]
    hashes = [C.live_hash(kv, b) for b in range(kv.B)]
    used = 0
    for b in range(kv.B):
        moves, src, dst = C.plan(kv.token_table, kv.seq_len, n_blocks, b, free[used:],
                                 len(free) - used, 0.25, 6)
        assert moves and len(src) > len(dst)
        C.apply(kv, b, moves)
        used += len(dst)
        # the freed sources hold no live token of any sequence any more
        occ = C.occupancy(kv.token_table, kv.seq_len, n_blocks)
        assert all(occ[p] == 0 for p in src) and all(occ[p] > 0 for p in dst)
    after = [D.logical_kv(kv, b, h) for b in range(kv.B) for h in range(kv.H)]
    for (t0, k0, v0), (t1, k1, v1) in zip(before, after):          # I1
        assert np.array_equal(t0, t1) and np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert C.duplicate_slots(kv.token_table, kv.seq_len, n_blocks) == (0, 0)   # I2
    assert [C.live_hash(kv, b) for b in range(kv.B)] == hashes


def test_hash_primitive_and_sensitivity():
    # SplitMix64 outputs for seed 0 (Steele, Lea and Flood 2014): the finaliser
    # applied to 1, 2, 3 times the golden-gamma increment 0x9e3779b97f4a7c15
    gamma = np.uint64(0x9E3779B97F4A7C15)
    with np.errstate(over="ignore"):
        st = np.array([gamma * np.uint64(i) for i in (1, 2, 3)], np.uint64)
    assert [int(x) for x in C.mix64(st)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                             0x06C45D188009454F]
    kv, free = _pool(tag=82, B=1, L=256, spare=4)
    h0 = C.live_hash(kv, 0)
    assert h0[1] == int((kv.token_table[0] >= 0).sum())
    live = np.nonzero(kv.token_table[0] >= 0)[0]
    dead = np.nonzero(kv.token_table[0] < 0)[0]
    s = int(kv.token_table[0, live[5]])
    kv.k[s // 16, 1, s % 16, 7] ^= 1                     # one bit of a live key
    assert C.live_hash(kv, 0) != h0
    kv.k[s // 16, 1, s % 16, 7] ^= 1
    assert C.live_hash(kv, 0) == h0
    # a dead slot's bytes do not count
    occupied = set(int(x) for x in kv.token_table[0][live])
    spare_slot = next(x for x in range(16 * kv.k.shape[0]) if x not in occupied)
    kv.v[spare_slot // 16, 0, spare_slot % 16, 3] ^= 5
    assert C.live_hash(kv, 0) == h0
    # moving a token with its rows leaves the hash alone; pointing it at
    # another token's rows (without the copy) does not
    f = int(free[0]) * 16
    for arr in (kv.k, kv.v):
        arr[f // 16, :, 0] = arr[s // 16, :, s % 16]
    kv.token_table[0, live[5]] = f
    assert C.live_hash(kv, 0) == h0
    kv.token_table[0, live[5]] = kv.token_table[0, live[6]]
    assert C.live_hash(kv, 0) != h0
    assert C.duplicate_slots(kv.token_table, kv.seq_len, kv.k.shape[0]) == (1, 0)
    # a dead token revived changes the count
    kv.token_table[0, live[5]] = f
    kv.token_table[0, dead[0]] = f + 1
    assert C.live_hash(kv, 0)[1] == h0[1] + 1


def test_hash_same_for_every_addressing_mode():
    """The hash follows the logical view: a paged pool read through its
    block table, the same pool through the equivalent token table, and the
    same keys and values laid out contiguously hash alike."""
    import dataclasses
    st = W.make_gqa_paged(tag=991, B=2, H=2, G=2, d=64, L=256, k=16, sink=4, local=16,
                          seq_len=[256, 173])
    kv = st.kv
    kv.block_table[0, 5] = -1                        # an unmapped block: 16 dead tokens
    tt = np.full((2, 256), -1, np.int32)
    Kc = np.zeros((2, 2, 256, 64), np.uint16)
    Vc = np.zeros((2, 2, 256, 64), np.uint16)
    for b in range(2):
        for t in range(int(kv.seq_len[b])):
            p = int(kv.block_table[b, t // 16])
            if p >= 0:
                tt[b, t] = p * 16 + t % 16
                Kc[b, :, t] = kv.k[p, :, t % 16]
                Vc[b, :, t] = kv.v[p, :, t % 16]
    via_bt = [C.live_hash(kv, b) for b in range(2)]
    via_tt = [C.live_hash(dataclasses.replace(kv, block_table=None, token_table=tt), b)
              for b in range(2)]
    assert via_bt == via_tt
    # contiguous storage has no dead tokens inside seq_len: compare sequence 1,
    # whose blocks are all mapped
    contig = dataclasses.replace(kv, k=Kc, v=Vc, block=0, block_table=None, token_table=None)
    assert C.live_hash(contig, 1) == via_bt[1]
    assert via_bt[0][1] == int(kv.seq_len[0]) - 16
