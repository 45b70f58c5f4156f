"""Pins of the block-summary oracle (no GPU): Quest's bound holds for every
block, a one-token block scores exactly its token, the block selection
equals a brute-force search over all K-subsets, and selecting every block of
a window without sink / local reproduces dense attention over its tokens."""
import itertools

import numpy as np
import scipy.special

import workloads as W
from oracle import blocks as BL
from oracle import dense as D


def _small(tag=900, L=256, G=2, seq=None):
    return W.make_gqa_paged(tag=tag, B=2, H=2, G=G, L=L, k=16, sink=0, local=0,
                            seq_len=seq or [L, L - 37])


def test_bound_over_every_token_of_the_block():
    st = _small()
    for b in range(2):
        for h in range(2):
            s_blk = BL.block_scores(st.kv, st.q, st.G, b, h)
            s_tok = D.scores_row(st.kv, st.q, st.G, b, h)
            for j in range(s_blk.size):
                toks = s_tok[16 * j:16 * j + 16]
                toks = toks[np.isfinite(toks)]
                if toks.size:
                    assert s_blk[j] >= toks.max() - 1e-9 * (1 + abs(toks.max()))
                else:
                    assert s_blk[j] == -np.inf


def test_one_token_block_scores_its_token():
    # seq_len 16 j + 1: the last block holds one live token
    st = _small(tag=901, L=128, seq=[97, 49])
    for b, last in ((0, 96), (1, 48)):
        for h in range(2):
            s_blk = BL.block_scores(st.kv, st.q, st.G, b, h)
            s_tok = D.scores_row(st.kv, st.q, st.G, b, h)
            assert abs(s_blk[last // 16] - s_tok[last]) <= 1e-12 * (1 + abs(s_tok[last]))


def test_selection_equals_brute_force_subsets():
    rng = np.random.default_rng(7)
    for trial in range(20):
        n, K = 9, 3
        s = np.round(rng.standard_normal(n) * 2) / 2        # ties likely
        s[rng.random(n) < 0.2] = -np.inf
        lo, hi = 16 * int(rng.integers(0, 2)), 16 * int(rng.integers(6, 10))
        got = BL.select_blocks(s, lo, hi, K)
        lb, hb = lo // 16, hi // 16
        cand = [j for j in range(lb, hb) if np.isfinite(s[j])]
        best = None
        for sub in itertools.combinations(cand, min(K, len(cand))):
            key = (sorted((-s[j] for j in sub)), sorted(sub))
            if best is None or key < best[0]:
                best = (key, sub)
        assert sorted(got.tolist()) == sorted(best[1])


def test_all_blocks_equal_dense_attention():
    st = _small(tag=902, L=160, seq=[160, 121])
    st.lo = np.zeros(2, np.int32)
    st.hi = np.array([160, 121], np.int32)
    for b in range(2):
        for h in range(2):
            nb = (int(st.kv.seq_len[b]) + 15) // 16
            s, blk, tok, out = BL.block_step_row(st, nb, b, h)
            t, K, V = D.logical_kv(st.kv, b, h)
            qg = D.to_f64(st.q[b, h * st.G:(h + 1) * st.G], st.kv.dtype)
            inb = t < 16 * (int(st.hi[b]) // 16)
            p = scipy.special.softmax(st.scale * (qg @ K[inb].T), axis=1)
            ref = p @ V[inb]
            # tokens of the partial last block are neither candidates nor local here
            assert np.array_equal(tok, t[inb])
            assert np.abs(out - ref).max() < 1e-12


def test_window_keeps_partial_boundary_blocks_out():
    assert BL.block_window(4, 32704) == (1, 2044)
    assert BL.block_window(0, 32) == (0, 2)
    assert BL.block_window(20, 30) == (2, 2)
