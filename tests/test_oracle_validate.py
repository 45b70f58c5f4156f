"""Pins of the validation reference (no GPU): clean workloads give no flag,
and each hand-made corruption raises exactly its own flag."""
import copy

import numpy as np

import workloads as W
from oracle import validate as V


def _token():
    st = W.make_token_pool(tag=501, B=2, H=1, d=64, L=256, k=16, sink=4, local=16,
                           spare_blocks=4)
    return st, st.kv.k.shape[0]


def _paged():
    st = W.make_gqa_paged(tag=502, B=2, H=1, G=2, d=64, L=256, k=16, sink=4, local=16)
    return st, st.kv.k.shape[0]


def test_clean_workloads_give_no_flag():
    for st, nb in (_token(), _paged()):
        idx = np.array([[[st.lo[b] + 1, st.lo[b] + 3, -1]] for b in range(st.kv.B)])
        assert V.validate(st.kv, nb, st.lo, st.hi, idx) == 0
    st = W.make_single_head(L=512)
    assert V.validate(st.kv, 0, st.lo, st.hi) == 0


def test_each_corruption_raises_its_flag():
    st, nb = _token()
    kv = copy.deepcopy(st.kv)
    kv.seq_len[1] = kv.L_max + 1
    assert V.validate(kv, nb) == V.BAD_SEQ_LEN
    assert V.validate(st.kv, nb, np.array([5, 0]), np.array([4, 10])) == V.BAD_WINDOW
    assert V.validate(st.kv, nb, np.array([0, 0]), np.array([10, 257])) == V.BAD_WINDOW
    kv = copy.deepcopy(st.kv)
    t = int(np.nonzero(kv.token_table[0] >= 0)[0][3])
    kv.token_table[0, t] = 16 * nb                     # one past the pool
    assert V.validate(kv, nb) == V.BAD_SLOT
    assert V.validate(kv, 0) == 0                      # no pool size: no upper bound
    kv.token_table[0, t] = -2
    assert V.validate(kv, 0) == V.BAD_SLOT
    kv = copy.deepcopy(st.kv)
    live1 = np.nonzero(kv.token_table[1] >= 0)[0]
    kv.token_table[1, live1[5]] = kv.token_table[0][kv.token_table[0] >= 0][7]
    assert V.validate(kv, nb) == V.DUP_SLOT
    kv.seq_len[1] = int(live1[5])                      # the duplicate is past seq_len now
    assert V.validate(kv, nb) == 0
    assert V.validate(st.kv, nb, idx=np.array([[[1, 256]]])) == V.BAD_IDX
    assert V.validate(st.kv, nb, idx=np.array([[[1, -2]]])) == V.BAD_IDX
    assert V.validate(st.kv, nb, idx=np.array([[[7, 3, 7, -1]], [[1, 2, -1, -1]]])) == V.DUP_IDX
    assert V.validate(st.kv, nb, idx=np.array([[[7, -1, -1]], [[7, -1, -1]]])) == 0


def test_block_table_checks():
    st, nb = _paged()
    kv = copy.deepcopy(st.kv)
    kv.block_table[1, 3] = nb
    assert V.validate(kv, nb) == V.BAD_SLOT
    kv.block_table[1, 3] = -1                          # unmapped: allowed
    assert V.validate(kv, nb) == 0
    kv.block_table[1, 3] = kv.block_table[0, 9]
    assert V.validate(kv, nb) == V.DUP_SLOT
    kv.seq_len[1] = 3 * 16                             # block 3 lies past seq_len
    assert V.validate(kv, nb) == 0
    kv.block_table[1, 3] = -5
    kv.seq_len[1] = 3 * 16 + 1
    assert V.validate(kv, nb) == V.BAD_SLOT
