"""The validation of device-resident data (sparsekv_validate) against the
oracle's reference, flag for flag, on clean workloads and on hand-made
corruptions of the tables, windows and selected positions.  Only the
validation pass sees the corrupt tables: it reads the tables, never the
pools.  The checking build (libsparsekv_debug.so) runs the same checks in
front of every call: a clean step leaves its flag word at zero, and a
reversed window -- which every kernel clamps to an empty window -- is
reported."""
import copy

import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D
from oracle import validate as V

from gpu_helpers import ATTN_TOL, DEV, say

pytestmark = pytest.mark.gpu


def _gpu_flags(kv_np, lo=None, hi=None, idx=None):
    kv = S.kv_to_device(kv_np, DEV)
    t = lambda a: None if a is None else S.to_device(np.asarray(a, np.int32), DEV)
    f = S.sparsekv_validate(kv, t(lo), t(hi), t(idx))
    torch.cuda.synchronize()
    return int(f.item())


def _both(kv_np, lo=None, hi=None, idx=None):
    nb = kv_np.k.shape[0] if kv_np.block else 0
    ref = V.validate(kv_np, nb, lo, hi, idx)
    got = _gpu_flags(kv_np, lo, hi, idx)
    say("  flags oracle", ref, "gpu", got)
    assert got == ref
    return got


def test_clean_workloads_pass():
    st = W.make_token_pool(tag=601, B=3, H=2, d=64, L=1024, k=32, sink=4, local=16, spare_blocks=7)
    idx = np.array([[[st.lo[b] + 2, st.lo[b] + 9, -1] for _ in range(2)] for b in range(3)])
    assert _both(st.kv, st.lo, st.hi, idx) == 0
    st = W.make_gqa_paged(tag=602, B=2, H=2, G=2, d=64, L=512, k=16, sink=4, local=16,
                          seq_len=[512, 301])
    assert _both(st.kv, st.lo, st.hi) == 0
    st = W.make_single_head(L=777 * 4)
    assert _both(st.kv, st.lo, st.hi) == 0


def test_corruptions_match_the_reference():
    st = W.make_token_pool(tag=603, B=2, H=1, d=64, L=512, k=16, sink=4, local=16, spare_blocks=4)
    nb = st.kv.k.shape[0]
    kv = copy.deepcopy(st.kv)
    t = int(np.nonzero(kv.token_table[0] >= 0)[0][3])
    kv.token_table[0, t] = 16 * nb
    assert _both(kv) == S.SKV_FLAG_BAD_SLOT
    kv.token_table[0, t] = -3
    assert _both(kv) == S.SKV_FLAG_BAD_SLOT
    kv = copy.deepcopy(st.kv)
    live1 = np.nonzero(kv.token_table[1] >= 0)[0]
    kv.token_table[1, live1[5]] = kv.token_table[0][kv.token_table[0] >= 0][7]
    assert _both(kv) == S.SKV_FLAG_DUP_SLOT
    kv = copy.deepcopy(st.kv)
    kv.seq_len[1] = kv.L_max + 3
    assert _both(kv) & S.SKV_FLAG_BAD_SEQ_LEN
    assert _both(st.kv, np.array([9, 0]), np.array([4, 10])) == S.SKV_FLAG_BAD_WINDOW
    idx = np.array([[[1, 512, -1]], [[5, 5, -1]]])
    assert _both(st.kv, idx=idx) == S.SKV_FLAG_BAD_IDX | S.SKV_FLAG_DUP_IDX
    pg = W.make_gqa_paged(tag=604, B=2, H=1, G=1, d=64, L=256, k=16, sink=4, local=16)
    kv = copy.deepcopy(pg.kv)
    kv.block_table[1, 2] = kv.block_table[0, 5]
    assert _both(kv) == S.SKV_FLAG_DUP_SLOT
    kv.block_table[1, 2] = kv.k.shape[0] + 1
    assert _both(kv) == S.SKV_FLAG_BAD_SLOT
    kv.block_table[1, 2] = -1
    assert _both(kv) == 0


def test_debug_build_checks_every_call():
    st = W.make_gqa_paged(tag=605, B=2, H=2, G=4, L=2048, k=128, sink=4, local=64)
    try:
        S.use_debug_library(True)
        assert S.sparsekv_is_debug_build()
        kv = S.kv_to_device(st.kv, DEV)
        q = S.to_device(st.q, DEV, True)
        lo = S.to_device(st.lo.astype(np.int32), DEV)
        hi = S.to_device(st.hi.astype(np.int32), DEV)
        S.sparsekv_debug_status()                         # start from a clear word
        _, idx, cnt, out = S.sparsekv_select_attend(kv, q, st.G, lo, hi, st.k, st.scale)
        _, idx2, cnt2 = S.sparsekv_select(kv, q, st.G, lo, hi, st.k)
        S.sparsekv_gather_attend(kv, q, st.G, idx2, st.k, lo, hi, st.scale)
        assert S.sparsekv_debug_status() == 0
        ref = D.step(st)
        assert np.abs(out.cpu().numpy() - ref["out"]).max() <= ATTN_TOL
        # a reversed window of sequence 1: reported; the kernels clamp it
        bad_lo = S.to_device(np.array([4, 1500], np.int32), DEV)
        bad_hi = S.to_device(np.array([1984, 1000], np.int32), DEV)
        S.sparsekv_select_attend(kv, q, st.G, bad_lo, bad_hi, st.k, st.scale)
        assert S.sparsekv_debug_status() == S.SKV_FLAG_BAD_WINDOW
        assert S.sparsekv_debug_status() == 0             # cleared by the read
    finally:
        S.use_debug_library(False)
