"""The library's host-side relocation planner against the oracle's plan
(no GPU: the planner is host code in libsparsekv.so), on token pools and on
random tables with shared blocks, every gate and several batch sizes."""
import numpy as np
import pytest

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import compact as C


def _same(tt, sl, n_blocks, b, free, n_free, theta, max_src, counts=None):
    ref_moves, ref_src, ref_dst = C.plan(tt, sl, n_blocks, b, free, n_free, theta, max_src)
    moves, src, n_dst = S.sparsekv_compact_plan(tt, sl, n_blocks, b, free, n_free, theta, max_src,
                                                counts=counts)
    got = [(int(t), int(s_), int(d_)) for (_, t, s_, d_) in moves]
    assert got == ref_moves
    assert np.all(moves[:, 0] == b)
    assert src.tolist() == ref_src and n_dst == len(ref_dst)
    return len(got)


def test_waste_ratio_matches_eq1():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = rng.integers(0, 17, size=int(rng.integers(1, 40)))
        assert abs(S.sparsekv_waste_ratio(n) - C.waste_ratio(n)) < 1e-12


@pytest.mark.parametrize("max_src,theta", [(1, 0.25), (6, 0.25), (64, 0.0), (64, 0.6)])
def test_plan_matches_oracle_on_token_pools(max_src, theta):
    st = W.make_token_pool(tag=83, B=4, H=1, d=64, L=1024, k=16, sink=4, local=16,
                           spare_blocks=50)
    kv = st.kv
    free = list(st.meta["free_blocks"])
    n_blocks = kv.k.shape[0]
    for b in range(kv.B):
        for n_free in (0, 1, 3, len(free)):
            _same(kv.token_table, kv.seq_len, n_blocks, b, free, n_free, theta, max_src)
    counts = C.occupancy(kv.token_table, kv.seq_len, n_blocks).astype(np.int32)
    assert _same(kv.token_table, kv.seq_len, n_blocks, 2, free, len(free), theta, max_src,
                 counts=counts) >= 0


def test_plan_matches_oracle_on_random_tables_with_shared_blocks():
    rng = np.random.default_rng(11)
    for trial in range(60):
        B, L, n_blocks = int(rng.integers(1, 4)), 16 * int(rng.integers(2, 12)), 40
        slots = rng.permutation(n_blocks * 16)[: B * L].reshape(B, L)
        # keep some slots inside shared blocks: scatter, then kill at random
        tt = np.where(rng.random((B, L)) < rng.uniform(0.2, 0.9), slots, -1).astype(np.int32)
        sl = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
        used = set((tt[tt >= 0] // 16).tolist())
        free = [p for p in range(n_blocks) if p not in used]
        for b in range(B):
            _same(tt, sl, n_blocks, b, free, int(rng.integers(0, len(free) + 1)),
                  float(rng.choice([0.0, 0.25, 0.5])), int(rng.integers(1, 10)))


def _pool_with_free():
    st = W.make_token_pool(tag=84, B=2, H=1, d=64, L=512, k=16, sink=4, local=16, spare_blocks=8)
    kv = st.kv
    return kv, kv.k.shape[0], [int(x) for x in st.meta["free_blocks"]]


def test_plan_rejects_free_blocks_outside_the_pool():
    kv, n_blocks, free = _pool_with_free()
    for bad in (-1, n_blocks, n_blocks + 100):
        with pytest.raises(S.SkvError) as e:
            S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, 0, free[:3] + [bad],
                                    4, 0.0, 8)
        assert e.value.status == S.SKV_EINVAL


def test_plan_rejects_free_blocks_that_hold_live_tokens_or_repeat():
    kv, n_blocks, free = _pool_with_free()
    live_block = int(kv.token_table[0][kv.token_table[0] >= 0][0]) // 16
    for fb in ([live_block] + free[:2], free[:2] + [free[0]]):
        with pytest.raises(S.SkvError) as e:
            S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, 0, fb, len(fb), 0.0, 8)
        assert e.value.status == S.SKV_EINVAL
    # the entries past n_free are not part of the plan's input
    moves, src, n_dst = S.sparsekv_compact_plan(kv.token_table, kv.seq_len, n_blocks, 0,
                                                free + [live_block], len(free), 0.0, 8)
    assert n_dst <= len(free)
