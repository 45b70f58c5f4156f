"""Block-summary scoring of the history, in float64 (test infrastructure only).

Source: OasisKV reading notes, section 3.2 (compressed key summaries, after
Quest): every logical block of 16 tokens keeps, per KV head, the
coordinate-wise minimum and maximum of its keys (two vectors instead of 16);
a query ranks all blocks by scanning the summaries alone, without reading a
key, and the top-K blocks per KV head (K = 128, i.e. 2,048 tokens, plus the
active local block; section 4.3 / 5.1) are attended.

Reading where the page is silent (the block score formula): the plainest
score consistent with "rank blocks from min / max summaries" is Quest's upper
bound of q . k over the block,
    score_j = sum_i max(q_i mn_ji, q_i mx_ji)  >=  max_{t in block j} q . k_t,
with the GQA group taking the max over its query heads, as for token scores.
Candidate blocks are those lying wholly inside the window [lo, hi); ties go
to the lower block index; the tokens of the selected blocks are attended with
the sink (t < lo) and local (t >= hi) tokens, as in the token-level step.
"""
from __future__ import annotations

import numpy as np

from oracle import dense as D

BLOCK = 16


def block_summaries(kv, b: int, h: int):
    """(mn, mx, live) for the logical blocks j < ceil(L_max / 16) of sequence
    b, KV head h: coordinate-wise min / max over the block's live keys
    (float64), live[j] = the block holds a live key."""
    t, K, _ = D.logical_kv(kv, b, h)
    nb = (kv.L_max + BLOCK - 1) // BLOCK
    mn = np.full((nb, kv.d_k), np.inf)
    mx = np.full((nb, kv.d_k), -np.inf)
    live = np.zeros(nb, bool)
    for i, tt in enumerate(t):
        j = tt // BLOCK
        mn[j] = np.minimum(mn[j], K[i])
        mx[j] = np.maximum(mx[j], K[i])
        live[j] = True
    return mn, mx, live


def block_scores(kv, q: np.ndarray, G: int, b: int, h: int) -> np.ndarray:
    """score_j = max_g sum_i max(q_gi mn_ji, q_gi mx_ji); -inf for blocks
    without a live key."""
    mn, mx, live = block_summaries(kv, b, h)
    qg = D.to_f64(q[b, h * G:(h + 1) * G], kv.dtype)      # [G][d]
    s = np.full(mn.shape[0], -np.inf)
    for j in np.nonzero(live)[0]:
        s[j] = max(np.maximum(qg * mn[j], qg * mx[j]).sum(axis=1))
    return s


def block_window(lo: int, hi: int):
    """Candidate blocks: those lying wholly inside [lo, hi)."""
    lb = (lo + BLOCK - 1) // BLOCK
    return lb, max(lb, hi // BLOCK)


def select_blocks(s: np.ndarray, lo: int, hi: int, K: int) -> np.ndarray:
    """The K best candidate blocks by (-score, j) (full sort), rank order."""
    lb, hb = block_window(lo, hi)
    return D.select_topk(s, lb, hb, K)


def expand(kv, b: int, blocks) -> np.ndarray:
    """Logical tokens of the selected blocks, live ones only, ascending."""
    t, _ = D.live_slots(kv, b)
    keep = np.isin(t // BLOCK, np.asarray(blocks, np.int64))
    return np.sort(t[keep])


def block_step_row(st, K: int, b: int, h: int):
    """Scores, selected blocks, attended tokens and output of one (b, h) row."""
    s = block_scores(st.kv, st.q, st.G, b, h)
    blk = select_blocks(s, int(st.lo[b]), int(st.hi[b]), K)
    tok = expand(st.kv, b, blk)
    out = D.attend_row(st.kv, st.q, st.G, b, h, tok, int(st.lo[b]), int(st.hi[b]), st.scale)
    return s, blk, tok, out
