"""Definition of one top-k sparse-attention decode step, in float64.

Test infrastructure (see the package docstring): never imported by the
product path.

Sources
-------
* Problem statement — ParisKV close-reading, section 一 (paper Sec. 3,
  Eqs. (1)-(3)): for one head, s_i = <k_i, q>, o = sum_i softmax(s)_i v_i;
  a small set C(q) is chosen and softmax is recomputed over the full-precision
  KV inside it.
* Exact top-k after all scores — ECHO-OSDI26 wiki page, "问题与动机" and
  observation 5: exact selection needs every index score first; prediction
  never changes the final exact top-k.
* Addressing — vToken reading notes, section 3.4, Eq. (2):
  slot = token_table[t].block_id * S + token_table[t].offset, and the
  PagedAttention block table of its background section (16-token blocks,
  logical block -> physical block).
* Sink / local windows — ParisKV close-reading, section 2.5 (Sink and Local
  regions attended densely, retrieval region searched); the eviction policy
  family (StreamingLLM) in vToken's background section.

Readings where the pages are silent (ties -> lower logical index; GQA
selection score = max over the group; disjoint sink / candidates / local
regions; fp32 output) are the plainest ones the pages support.

Layouts (shared with the GPU path only through the caller's arrays)
------------------------------------------------------------------
paged / token-table pools: [n_blocks][H][16][d]; contiguous: [B][H][L_max][d].
bf16 values are carried as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact bf16 -> float64: the 16 bits are the top half of an fp32."""
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    raise ValueError(dtype)


def live_slots(kv, b: int):
    """Logical positions t < seq_len[b] that are live, and their physical
    slot (paged / token modes) or row (contiguous mode)."""
    L = int(kv.seq_len[b])
    t = np.arange(L, dtype=np.int64)
    if kv.token_table is not None:                 # token-level table, Eq. (2)
        slot = kv.token_table[b, :L].astype(np.int64)
        keep = slot >= 0
        return t[keep], slot[keep]
    if kv.block_table is not None:                 # block table, 16-token blocks
        blk = kv.block_table[b, t // 16].astype(np.int64)
        keep = blk >= 0                            # negative entry: unmapped block, dead
        return t[keep], (blk * 16 + t % 16)[keep]
    return t, t                                    # contiguous storage


def logical_kv(kv, b: int, h: int):
    """Dense logical (t, K_t, V_t) of sequence b, KV head h, for live t.

    Returns (t, K [n, d_k], V [n, d_v]) in float64.  When kv.v is None the
    value is the first d_v dims of the key row (shared latent)."""
    t, slot = live_slots(kv, b)
    if kv.block:                                   # pool [n_blocks][H][16][d]
        pb, off = slot // 16, slot % 16
        Kr = kv.k[pb, h, off]
        Vr = kv.v[pb, h, off] if kv.v is not None else None
    else:                                          # [B][H][L_max][d]
        Kr = kv.k[b, h, slot]
        Vr = kv.v[b, h, slot] if kv.v is not None else None
    K = to_f64(Kr, kv.dtype)
    V = to_f64(Vr, kv.dtype) if Vr is not None else K[:, : kv.d_v]
    return t, K, V


def scores_row(kv, q: np.ndarray, G: int, b: int, h: int) -> np.ndarray:
    """s[t] = max over the G query heads of KV head h of q_g . K_t, for every
    logical t < L_max; -inf for dead tokens and t >= seq_len[b]."""
    t, K, _ = logical_kv(kv, b, h)
    qg = to_f64(q[b, h * G:(h + 1) * G], kv.dtype)      # [G][d_k]
    s = np.full(kv.L_max, -np.inf)
    if t.size:
        s[t] = (K @ qg.T).max(axis=1)
    return s


def select_topk(s: np.ndarray, lo: int, hi: int, k: int) -> np.ndarray:
    """The k largest s[t] among candidates t in [lo, hi) with s finite, ties to
    the lower t, by a full sort on the key (-s, t).  Returns the selected
    logical positions in rank order (len = min(k, #candidates))."""
    t = np.arange(lo, max(lo, hi), dtype=np.int64)
    st = s[lo:max(lo, hi)]
    keep = np.isfinite(st)
    t, st = t[keep], st[keep] + 0.0                # + 0.0 maps -0.0 to +0.0
    order = np.lexsort((t, -st))
    return t[order[:k]]


def attend_row(kv, q: np.ndarray, G: int, b: int, h: int, sel, lo: int, hi: int,
               scale: float) -> np.ndarray:
    """Dense-then-masked softmax attention for the G query heads of KV head h.

    A = selected ∪ {live t < lo} ∪ {live t >= hi}.  Logits over all L_max
    logical positions, -inf outside A, subtract the max, exp, normalise,
    o = sum_t p_t V_t.  Returns [G][d_v] float64 (zeros if A is empty)."""
    t, K, V = logical_kv(kv, b, h)
    qg = to_f64(q[b, h * G:(h + 1) * G], kv.dtype)
    L = kv.L_max
    in_a = np.zeros(L, bool)
    sel = np.asarray(sel, np.int64)
    in_a[sel[sel >= 0]] = True
    live = np.zeros(L, bool)
    live[t] = True
    pos = np.arange(L)
    in_a |= live & ((pos < lo) | (pos >= hi))
    in_a &= live
    out = np.zeros((G, kv.d_v))
    if not in_a.any():
        return out
    Kfull = np.zeros((L, kv.d_k))
    Vfull = np.zeros((L, kv.d_v))
    Kfull[t] = K
    Vfull[t] = V
    z = scale * (qg @ Kfull.T)                     # [G][L]
    z[:, ~in_a] = -np.inf
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p @ Vfull


def step_row(st, b: int, h: int):
    """Selection and output of one (b, h) row of a Step."""
    s = scores_row(st.score_kv, st.score_q, st.score_G, b, h)
    sel = select_topk(s, int(st.lo[b]), int(st.hi[b]), st.k)
    out = attend_row(st.kv, st.q, st.G, b, h, sel, int(st.lo[b]), int(st.hi[b]), st.scale)
    return s, sel, out


def step(st, rows=None):
    """Whole step (or the listed (b, h) rows).

    Returns dict with scores [B][H][L_max], idx [B][H][k] (rank order, -1
    padded), count [B][H], out [B][H*G][d_v] (float64; rows not computed
    are NaN)."""
    kv = st.kv
    B, H = st.score_kv.B, st.score_kv.H
    Ha = kv.H
    scores = np.full((B, H, st.score_kv.L_max), np.nan)
    idx = np.full((B, H, st.k), -1, np.int64)
    count = np.zeros((B, H), np.int64)
    out = np.full((B, Ha * st.G, kv.d_v), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(H)]
    for b, h in rows:
        s = scores_row(st.score_kv, st.score_q, st.score_G, b, h)
        sel = select_topk(s, int(st.lo[b]), int(st.hi[b]), st.k)
        scores[b, h] = s
        idx[b, h, : sel.size] = sel
        count[b, h] = sel.size
        # attention heads that read this selection (an indexer with one head
        # drives every attention KV head of its layer)
        for ha in ([h] if H == Ha else range(Ha)):
            o = attend_row(kv, st.q, st.G, b, ha, sel, int(st.lo[b]), int(st.hi[b]), st.scale)
            out[b, ha * st.G:(ha + 1) * st.G] = o
    return {"scores": scores, "idx": idx, "count": count, "out": out}


def attend_given(st, idx: np.ndarray, rows=None) -> np.ndarray:
    """Attention output for a given selection idx [B][H_sel][k] (-1 skipped),
    e.g. the GPU's own set, so a legitimate near-tie swap cannot fail the
    output comparison."""
    kv = st.kv
    B, Hs = idx.shape[0], idx.shape[1]
    out = np.full((B, kv.H * st.G, kv.d_v), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hs)]
    for b, h in rows:
        for ha in ([h] if Hs == kv.H else range(kv.H)):
            out[b, ha * st.G:(ha + 1) * st.G] = attend_row(
                kv, st.q, st.G, b, ha, idx[b, h], int(st.lo[b]), int(st.hi[b]), st.scale)
    return out
