"""Pins of the float64 step oracle against brute force, closed forms and
library routines (no GPU)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import workloads as W
from oracle import closed_forms as cf
from oracle import dense as D

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


# ----------------------------------------------------------------- addressing
def _coded_pool(n_blocks, H, d):
    """fp32 pool whose element (pb, h, off, j) = pb*1000 + h*100 + off + j/8:
    every row names its own physical coordinates."""
    pb, h, off, j = np.meshgrid(np.arange(n_blocks), np.arange(H), np.arange(16), np.arange(d),
                                indexing="ij")
    return (pb * 1000.0 + h * 100.0 + off + j / 8.0).astype(np.float32)


def test_block_table_addressing_reads_the_named_block():
    B, H, d, L = 2, 3, 8, 64
    n_blocks = B * L // 16
    pool = _coded_pool(n_blocks, H, d)
    perm = np.random.default_rng(0).permutation(n_blocks).astype(np.int32)
    bt = perm.reshape(B, L // 16)
    kv = W.KV(k=pool, v=pool, dtype="f32", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
              block_table=bt, seq_len=np.array([L, 37], np.int32))
    for b in range(B):
        for h in range(H):
            t, K, V = D.logical_kv(kv, b, h)
            assert t.tolist() == list(range(int(kv.seq_len[b])))
            want = bt[b, t // 16] * 1000.0 + h * 100.0 + t % 16
            np.testing.assert_array_equal(K[:, 0], want)
            np.testing.assert_array_equal(K[:, 5] - K[:, 0], 0.625)
            np.testing.assert_array_equal(V, K)


def test_token_table_addressing_and_dead_tokens():
    B, H, d, L = 2, 2, 4, 48
    n_blocks = 8
    pool = _coded_pool(n_blocks, H, d)
    rng = np.random.default_rng(1)
    tt = np.full((B, L), -1, np.int32)
    slots = rng.permutation(n_blocks * 16)
    live = rng.random((B, L)) < 0.6
    tt[live] = slots[: live.sum()]
    kv = W.KV(k=pool, v=pool, dtype="f32", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
              token_table=tt, seq_len=np.array([L, L], np.int32))
    for b in range(B):
        for h in range(H):
            t, K, _ = D.logical_kv(kv, b, h)
            assert t.tolist() == np.nonzero(live[b])[0].tolist()
            slot = tt[b, t]
            np.testing.assert_array_equal(K[:, 0], (slot // 16) * 1000.0 + h * 100.0 + slot % 16)


def test_unmapped_block_equals_token_table_with_dead_tokens():
    """A negative block-table entry makes its 16 tokens dead: the logical KV
    equals the one read through the per-token table with those tokens at -1."""
    B, H, d, L = 2, 2, 4, 64
    n_blocks = B * L // 16
    pool = _coded_pool(n_blocks, H, d)
    bt = np.random.default_rng(2).permutation(n_blocks).astype(np.int32).reshape(B, L // 16)
    bt[0, 1] = -1
    bt[1, 3] = -7
    seq = np.array([L, 60], np.int32)
    kvb = W.KV(k=pool, v=pool, dtype="f32", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
               block_table=bt, seq_len=seq)
    t = np.arange(L)
    tt = np.where(bt[:, t // 16] >= 0, bt[:, t // 16] * 16 + t % 16, -1).astype(np.int32)
    kvt = W.KV(k=pool, v=pool, dtype="f32", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
               token_table=tt, seq_len=seq)
    for b in range(B):
        for h in range(H):
            tb, Kb, _ = D.logical_kv(kvb, b, h)
            tk, Kt, _ = D.logical_kv(kvt, b, h)
            np.testing.assert_array_equal(tb, tk)
            np.testing.assert_array_equal(Kb, Kt)
    dead0 = set(range(16, 32))
    assert dead0.isdisjoint(D.logical_kv(kvb, 0, 0)[0].tolist())
    q = np.ones((B, H, d), np.float32)
    s0 = D.scores_row(kvb, q, 1, 0, 0)
    assert np.all(np.isneginf(s0[16:32])) and np.all(np.isfinite(s0[:16]))


def test_contiguous_addressing_and_latent_value():
    B, H, L, d = 2, 2, 10, 6
    k = np.arange(B * H * L * d, dtype=np.float32).reshape(B, H, L, d)
    kv = W.KV(k=k, v=None, dtype="f32", B=B, H=H, d_k=d, d_v=4, block=0, L_max=L,
              seq_len=np.array([L, 7], np.int32))
    t, K, V = D.logical_kv(kv, 1, 1)
    assert t.tolist() == list(range(7))
    np.testing.assert_array_equal(K, k[1, 1, :7])
    np.testing.assert_array_equal(V, k[1, 1, :7, :4])


def test_bf16_decode_exact():
    x = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 65280.0], np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(D.bf16_bits_to_f64(bits), x.astype(np.float64))


# ------------------------------------------------------------------- scoring
def _plain_kv(L, d, H=1, B=1, seed=0, seq_len=None):
    k = np.random.default_rng(seed).standard_normal((B, H, L, d)).astype(np.float32)
    v = np.random.default_rng(seed + 1).standard_normal((B, H, L, d)).astype(np.float32)
    sl = np.full(B, L, np.int32) if seq_len is None else np.asarray(seq_len, np.int32)
    return W.KV(k=k, v=v, dtype="f32", B=B, H=H, d_k=d, d_v=d, block=0, L_max=L, seq_len=sl)


def test_scores_basis_query_reads_one_coordinate():
    kv = _plain_kv(20, 8, seq_len=[15])
    q = np.zeros((1, 1, 8), np.float32)
    q[0, 0, 3] = 1.0
    s = D.scores_row(kv, q, 1, 0, 0)
    np.testing.assert_array_equal(s[:15], kv.k[0, 0, :15, 3])
    assert np.all(np.isneginf(s[15:]))


def test_scores_group_max():
    kv = _plain_kv(12, 8, H=2)
    q = np.zeros((1, 4, 8), np.float32)           # G = 2 per KV head
    q[0, 2, 1], q[0, 3, 1] = 1.0, -1.0            # head 1: max(k, -k) = |k|
    s = D.scores_row(kv, q, 2, 0, 1)
    np.testing.assert_array_equal(s, np.abs(kv.k[0, 1, :, 1]))


# ----------------------------------------------------------------- selection
def _brute_topk(s, lo, hi, k):
    """The unique k-subset S of finite candidates with, for i in S, j not in S:
    s_i > s_j or (s_i == s_j and i < j)."""
    cand = [t for t in range(lo, hi) if np.isfinite(s[t])]
    kk = min(k, len(cand))
    found = []
    for S in itertools.combinations(cand, kk):
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in S for j in cand if j not in S)
        if ok:
            found.append(set(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 11))
    s = rng.integers(-3, 4, size=L).astype(np.float64)      # many ties
    s[rng.random(L) < 0.2] = -np.inf                        # dead tokens
    lo = int(rng.integers(0, L))
    hi = int(rng.integers(lo, L + 1))
    k = int(rng.integers(1, 6))
    got = D.select_topk(s, lo, hi, k)
    assert set(got.tolist()) == _brute_topk(s, lo, hi, k)
    assert len(got) == len(set(got.tolist()))


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([0.0, -0.0, 0.0, -0.0, -1.0])
    assert D.select_topk(s, 0, 5, 2).tolist() == [0, 1]
    s2 = np.array([-0.0, 0.0])
    assert D.select_topk(s2, 0, 2, 1).tolist() == [0]


# ----------------------------------------------------------------- attention
def test_equal_logits_give_mean_of_attended_values():
    kv = _plain_kv(16, 4)
    q = np.zeros((1, 1, 4), np.float32)
    sel = [3, 7, 9]
    o = D.attend_row(kv, q, 1, 0, 0, sel, 2, 14, 0.3)
    A = [0, 1, 3, 7, 9, 14, 15]                      # sink t<2, selected, local t>=14
    np.testing.assert_allclose(o[0], kv.v[0, 0, A].astype(np.float64).mean(axis=0), rtol=1e-13)


def test_two_token_softmax_by_hand():
    k = np.zeros((1, 1, 2, 2), np.float32)
    k[0, 0, 0] = [1.0, 0.0]
    k[0, 0, 1] = [0.0, 2.0]
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    kv = W.KV(k=k, v=v, dtype="f32", B=1, H=1, d_k=2, d_v=2, block=0, L_max=2,
              seq_len=np.array([2], np.int32))
    q = np.array([[[1.0, 1.0]]], np.float32)
    o = D.attend_row(kv, q, 1, 0, 0, [0, 1], 0, 2, 0.5)     # logits 0.5, 1.0
    p1 = 1.0 / (1.0 + math.exp(-0.5))
    np.testing.assert_allclose(o[0], [1 - p1, p1], rtol=1e-14)


def test_mask_is_exactly_selected_sink_local():
    """V rows = one-hot of the logical position: the output is the probability
    vector itself, so its support must be exactly A restricted to live tokens."""
    L = 32
    rng = np.random.default_rng(3)
    kpool = rng.standard_normal((2, 1, 16, 8)).astype(np.float32)
    vpool = np.eye(L, dtype=np.float32).reshape(2, 1, 16, L)
    tt = np.arange(L, dtype=np.int32).reshape(1, L).copy()
    tt[0, [1, 10, 20]] = -1                                  # dead tokens
    kv = W.KV(k=kpool, v=vpool, dtype="f32", B=1, H=1, d_k=8, d_v=L, block=16, L_max=L,
              token_table=tt, seq_len=np.array([L], np.int32))
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    sel = [5, 6, 11]
    o = D.attend_row(kv, q, 1, 0, 0, sel, 3, 19, 1.0)
    support = set(np.nonzero(o[0] > 0)[0].tolist())
    assert support == {0, 2, 5, 6, 11, 19, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31}
    np.testing.assert_allclose(o[0].sum(), 1.0, rtol=1e-14)


def test_k_equals_L_is_dense_attention():
    """Selecting every candidate reproduces plain dense softmax attention
    (scipy.special.softmax), for a GQA group."""
    B, H, G, d, L = 1, 2, 3, 16, 40
    st = W.make_gqa_paged(tag=901, B=2, H=H, G=G, d=d, L=48, k=48, sink=0, local=0)
    res = D.step(st)
    for b in range(2):
        for h in range(H):
            t, K, V = D.logical_kv(st.kv, b, h)
            qg = D.bf16_bits_to_f64(st.q[b, h * G:(h + 1) * G])
            p = softmax(st.scale * qg @ K.T, axis=1)
            np.testing.assert_allclose(res["out"][b, h * G:(h + 1) * G], p @ V, rtol=1e-12,
                                       atol=1e-13)
            assert res["count"][b, h] == 48


def test_one_dominant_key_returns_its_value():
    kv = _plain_kv(30, 8)
    q = (kv.k[0, 0, 17] * 50).reshape(1, 1, 8)
    o = D.attend_row(kv, q, 1, 0, 0, [17, 3], 0, 30, 1.0)
    np.testing.assert_allclose(o[0], kv.v[0, 0, 17], atol=1e-10)


def test_empty_attention_set_gives_zero():
    kv = _plain_kv(8, 4)
    q = np.ones((1, 1, 4), np.float32)
    o = D.attend_row(kv, q, 1, 0, 0, [-1, -1], 0, 8, 1.0)
    assert np.all(o == 0)


# -------------------------------------------------------------- closed forms
def test_waste_ratio_worked_example():
    g = GOLD["waste_ratio"]
    assert cf.waste_ratio(g["n_live"], g["S"]) == pytest.approx(g["F"])
    assert sum(g["n_live"]) == g["T_live"]
    assert math.ceil(g["T_live"] / g["S"]) == g["target_blocks"]


def test_oasis_budget_example():
    g = GOLD["oasis_budget"]
    assert g["K_blocks"] * g["block"] == g["selected_tokens"]
    assert (g["K_blocks"] + 1) * g["block"] == g["with_local_tokens"]
    assert round(100 * cf.read_fraction(g["with_local_tokens"], g["context"]), 1) == g["fraction_pct"]


def test_ulacache_read_volume_example():
    g = GOLD["ulacache_read"]
    mib = cf.read_bytes(g["k"], g["s_kv_KiB"] * 1024) / 2**20
    assert mib == g["read_MiB"]
    assert round(1000 * mib / 1024 / g["link_GiB_s"], 2) == g["time_ms"]
    assert round((1 - g["hit"]) * mib) == g["read_MiB_with_hit"]


def test_generated_pool_bytes_match_kv_closed_form():
    """M_KV = B L N_layer 2 N_kv d_h s for the generated pools (one layer)."""
    st = W.make_gqa_paged(tag=902, B=2, H=3, G=2, d=32, L=64, k=8)
    assert st.kv.k.nbytes + st.kv.v.nbytes == cf.kv_bytes(2, 64, 1, 3, 32, 2)
    s1 = W.make_single_head(tag=903, L=256, d=16, k=4)
    assert s1.kv.k.nbytes + s1.kv.v.nbytes == cf.kv_bytes(1, 256, 1, 1, 16, 4)


def test_token_pool_generator_half_dead_waste():
    st = W.make_token_pool(tag=904, B=3, H=2, d=16, L=512, k=16, sink=4, local=16)
    tt = st.kv.token_table
    n_live_blocks = []
    for b in range(3):
        assert (tt[b] >= 0).sum() == 256                  # exactly half live
        s = tt[b][tt[b] >= 0]
        assert len(np.unique(s)) == s.size                # unique mapping (I2)
        n_live_blocks += np.bincount(s // 16, minlength=1)[np.unique(s // 16)].tolist()
        live = np.nonzero(tt[b] >= 0)[0]
        assert (live < st.lo[b]).sum() == 4 and (live >= st.hi[b]).sum() == 16
    # blocks keep their holes: the intra-block waste ratio is ~0.5 (Eq. (1))
    assert 0.45 < cf.waste_ratio(n_live_blocks, 16) < 0.55
