"""Token-table compaction (lazy relocation) and its invariant checks
(test infrastructure only).

Source: vToken reading notes, section 3.3 (the reclamation back end: stage 1
eligibility by the intra-block waste ratio F of Eq. (1) against theta_F,
stage 2 headroom-aware admission, stage 3 relocation planning, stage 4 the
copy), section 3.2 (apply_moves rewrites the token-table positions after the
copy), section 3.5 (invariants I1 token conservation, I2 unique mapping, I4
a plan must free strictly more blocks than it consumes; shared blocks are
left alone) and section 4.6 (I1 / I2 are checked by hashing the retained
token ids and their K/V contents before and after every migration).

Readings where the page is silent:
  * F is taken over the blocks holding the sequence's live tokens
    (N = their number), n_b counting live tokens of every sequence;
  * eligible source blocks are the sequence's private blocks (all their live
    tokens belong to it) that are not full; they are taken lowest
    utilisation first (ties: lower block id), at most max_src of them;
  * targets are the caller's free blocks in the order given; `n_free` of
    them may be consumed (free pool plus evacuation headroom);
  * when the plan would not free strictly more blocks than it consumes, or
    needs more targets than may be consumed, the fullest candidate is dropped
    and the plan recomputed (the page shrinks the candidate set); an empty
    set means no plan;
  * moves take the sources' live tokens in ascending logical order and fill
    target block after target block: move i goes to
    free_blocks[i // 16] * 16 + i % 16;
  * the page names no hash; the one used is a sum, modulo 2^64, of one term
    per stored 64-bit word of every live token's K row (and V row when
    values are stored separately), over all heads:
        s    = mix64((t * H + h) * R + r),
        term = mix64((s + (j + 1) * gamma) ^ w_j),
    t the logical token, h the head, r the row (0 = K, 1 = V; R rows), w_j
    the row's 64-bit word j (its 32-bit words 2j and 2j + 1, low first),
    gamma = 0x9e3779b97f4a7c15 and mix64 the SplitMix64 finaliser (Steele,
    Lea and Flood, "Fast splittable pseudorandom number generators", 2014):
        z ^= z >> 30; z *= 0xbf58476d1ce4e5b9; z ^= z >> 27;
        z *= 0x94d049bb133111eb; z ^= z >> 31.
    One mix per 8 stored bytes keeps a GPU pass over the pool bound by
    memory.  The sum is independent of where a token is stored and of the
    order the terms are added in, and changes when a live token, its
    position or one stored word changes (barring a 2^-64 coincidence).
"""
from __future__ import annotations

import math

import numpy as np

S = 16
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
GAMMA = np.uint64(0x9E3779B97F4A7C15)


def waste_ratio(n_live) -> float:
    """Eq. (1): F = 1 - sum_i n_i / (N S) over N allocated blocks."""
    n = np.asarray(n_live, np.float64)
    return 1.0 - n.sum() / (n.size * S)


def occupancy(token_table: np.ndarray, seq_len: np.ndarray, n_blocks: int) -> np.ndarray:
    """Live tokens per physical block over every sequence."""
    counts = np.zeros(n_blocks, np.int64)
    for b in range(token_table.shape[0]):
        row = token_table[b, : int(seq_len[b])]
        row = row[row >= 0]
        np.add.at(counts, row // S, 1)
    return counts


def plan(token_table: np.ndarray, seq_len: np.ndarray, n_blocks: int, b: int, free_blocks,
         n_free: int, theta_F: float, max_src: int):
    """Relocation plan for sequence b.  Returns (moves [(t, src, dst)],
    sources, targets), empty when stage 1 or the gates reject."""
    counts = occupancy(token_table, seq_len, n_blocks)
    L = int(seq_len[b])
    row = token_table[b, :L].astype(np.int64)
    live_t = np.nonzero(row >= 0)[0]
    blk = row[live_t] // S
    own = np.bincount(blk, minlength=n_blocks)
    mine = np.nonzero(own)[0]
    if mine.size == 0 or waste_ratio(counts[mine]) <= theta_F:     # stage 1
        return [], [], []
    cand = [p for p in mine if own[p] == counts[p] and counts[p] < S]   # private, not full
    cand.sort(key=lambda p: (counts[p], p))
    cand = cand[:max_src]
    while cand:                                                   # stages 2 and 3
        T = int(sum(counts[p] for p in cand))
        n_tgt = math.ceil(T / S)
        if len(cand) > n_tgt and n_tgt <= min(n_free, len(free_blocks)):
            break
        cand = cand[:-1]
    if not cand:
        return [], [], []
    src = set(int(p) for p in cand)
    toks = [int(t) for t, p in zip(live_t, blk) if int(p) in src]   # ascending t
    moves = [(t, int(row[t]), int(free_blocks[i // S]) * S + i % S) for i, t in enumerate(toks)]
    return moves, sorted(src), [int(x) for x in free_blocks[: math.ceil(len(toks) / S)]]


def apply(kv, b: int, moves):
    """Copy the moved tokens' K (and V) rows of every head to their targets,
    then point the token table at them (the sources keep their bytes)."""
    for t, src, dst in moves:
        for arr in (kv.k, kv.v):
            if arr is not None:
                arr[dst // S, :, dst % S] = arr[src // S, :, src % S]
        kv.token_table[b, t] = dst


def mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * M1
        z = z ^ (z >> np.uint64(27))
        z = z * M2
        z = z ^ (z >> np.uint64(31))
    return z


def live_hash(kv, b: int) -> tuple[int, int]:
    """(hash, live count) of sequence b's retained tokens, from the logical
    view: the table (token or block table, or none for contiguous storage)
    decides which t are live and where their rows are."""
    from .dense import live_slots
    live_t, slots = live_slots(kv, b)
    live_t, slots = live_t[live_t < kv.L_max], slots[live_t < kv.L_max]
    rows = [kv.k] + ([kv.v] if kv.v is not None else [])
    R = len(rows)
    total = np.uint64(0)
    for r, arr in enumerate(rows):
        if kv.block:
            data = arr[slots // S, :, slots % S]             # [n][H][d] as stored
        else:
            data = np.moveaxis(arr[b][:, slots], 0, 1)       # [H][n][d] -> [n][H][d]
        words = np.ascontiguousarray(data).view(np.uint64)   # [n][H][W64], little endian
        n, H, W = words.shape
        t = live_t.astype(np.uint64)[:, None, None]
        h = np.arange(H, dtype=np.uint64)[None, :, None]
        j1 = np.arange(1, W + 1, dtype=np.uint64)[None, None, :]
        with np.errstate(over="ignore"):
            seed = mix64((t * np.uint64(H) + h) * np.uint64(R) + np.uint64(r))
            terms = mix64((seed + j1 * GAMMA) ^ words)
            total = total + terms.sum(dtype=np.uint64)
    return int(total), int(live_t.size)


def duplicate_slots(token_table: np.ndarray, seq_len: np.ndarray, n_blocks: int) -> tuple[int, int]:
    """I2 check over every sequence: (live tokens whose slot another live
    token already claims, live tokens whose slot lies outside the pool)."""
    seen = np.zeros(n_blocks * S, np.int64)
    bad = 0
    for b in range(token_table.shape[0]):
        row = token_table[b, : int(seq_len[b])]
        row = row[row >= 0].astype(np.int64)
        out = row >= n_blocks * S
        bad += int(out.sum())
        np.add.at(seen, row[~out], 1)
    dup = int(np.maximum(seen - 1, 0).sum())
    return dup, bad
