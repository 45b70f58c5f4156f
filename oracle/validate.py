"""Validation of the device-resident data a decode step takes on trust, as a
plain CPU reference.

Test infrastructure (see the package docstring): never imported by the
product path.

Sources
-------
* Invariant I2 — vToken reading notes, section 3.5: every live token's
  mapping points at a valid slot inside the pool and no two live tokens map
  to one slot; section 4.6 checks the invariants around every migration.
* Slot mapping — vToken reading notes, section 3.4, Eq. (2) (token table)
  and the PagedAttention block table of its background section (a logical
  16-token block -> a physical block; a negative entry: unmapped).
* Windows — ParisKV close-reading, section 2.5: sink [0, lo), retrieval
  [lo, hi), local [hi, seq_len).

The checks read only seq_len, the tables, the windows and the selected
positions; never the K/V pools.  Flags are OR-ed bits:

  BAD_SEQ_LEN  1   seq_len[b] outside [0, L_max]
  BAD_WINDOW   2   not 0 <= lo[b] <= hi[b] <= seq_len[b]
  BAD_SLOT     4   a mapping of a token t < seq_len[b] that is neither a
                   valid slot nor "dead": token table entry < -1 or >= 16 n;
                   block table entry < -1 or >= n (n = pool blocks; the
                   upper bounds only when n is given)
  DUP_SLOT     8   two live tokens map to one slot (token table) or two
                   logical blocks to one physical block (block table);
                   only when n is given
  BAD_IDX     16   a selected position outside [-1, L_max)
  DUP_IDX     32   a row of selected positions names a position twice

Reading where the pages are silent: a block-table entry of -1 marks an
unmapped block (its 16 tokens dead); any other negative entry is invalid;
a sequence's block-table entries are checked for the blocks holding its
first seq_len[b] tokens only.
"""
from __future__ import annotations

import numpy as np

BAD_SEQ_LEN, BAD_WINDOW, BAD_SLOT, DUP_SLOT, BAD_IDX, DUP_IDX = 1, 2, 4, 8, 16, 32


def validate(kv, n_blocks: int = 0, lo=None, hi=None, idx=None) -> int:
    """Flags of the checks above for a KV description (numpy arrays, the
    fields of workloads.KV), optional windows lo, hi [B] and optional selected
    positions idx [B][H][k]."""
    flags = 0
    B, L = kv.B, kv.L_max
    seq = np.asarray(kv.seq_len, np.int64)
    if np.any((seq < 0) | (seq > L)):
        flags |= BAD_SEQ_LEN
    if lo is not None and hi is not None:
        lo, hi = np.asarray(lo, np.int64), np.asarray(hi, np.int64)
        s = np.clip(seq, 0, L)
        if np.any((lo < 0) | (lo > hi) | (hi > s)):
            flags |= BAD_WINDOW
    claims = {}
    for b in range(B):
        n = int(min(max(seq[b], 0), L))
        if kv.token_table is not None:
            for t in range(n):
                e = int(kv.token_table[b, t])
                if e < -1 or (n_blocks and e >= 16 * n_blocks):
                    flags |= BAD_SLOT
                elif e >= 0 and n_blocks:
                    if e in claims:
                        flags |= DUP_SLOT
                    claims[e] = (b, t)
        elif kv.block_table is not None:
            for j in range((n + 15) // 16):
                e = int(kv.block_table[b, j])
                if e < -1 or (n_blocks and e >= n_blocks):
                    flags |= BAD_SLOT
                elif e >= 0 and n_blocks:
                    if e in claims:
                        flags |= DUP_SLOT
                    claims[e] = (b, j)
    if idx is not None:
        idx = np.asarray(idx, np.int64)
        if np.any((idx < -1) | (idx >= L)):
            flags |= BAD_IDX
        for row in idx.reshape(-1, idx.shape[-1]):
            live = row[(row >= 0) & (row < L)]
            if live.size != np.unique(live).size:
                flags |= DUP_IDX
    return flags
