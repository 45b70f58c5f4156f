"""Update buffer of the compressed path and its multi-step decode loop
(test infrastructure only).

Source: ParisKV close-reading, section 2.5 (paper Sec. 4.2.1, Fig. 5) and
section 2.1 (paper Sec. 4, Figs. 2 and 5): the history is split into a Sink
region and a Local region attended densely, a Retrieval region held in the
compressed index, and an Update Buffer for the newest tokens.  New tokens
enter the buffer; once it is full they move into Local as one batch, and the
Local tokens pushed out by them are encoded and join Retrieval, which spreads
the cost of updating the index over `update` steps (256 or 512 tokens in the
page's experiments).

Readings where the page is silent:
  * layout: Sink [0, sink) | Retrieval [sink, sink + n) | Local, `local`
    tokens | buffer; the buffer's tokens are attended densely like Local
    (they are the newest context and stay on the GPU);
  * "full" means the buffer holds `update` tokens, i.e. the dense tail
    [sink + n, seq_len) has reached local + update tokens; the flush then
    happens before the step's retrieval, so a step attends densely to
    between `local` and local + update - 1 tail tokens;
  * after prefill the index covers [sink, L0 - local) and the buffer is
    empty (as in the one-step workload);
  * the index of a grown Retrieval region is the per-key encoding of every
    key in it, its histogram the count over all of them: appending entries
    adds their counts (the encoding of a key does not depend on the others).

Retrieval and attention of each step are the one-step definitions
(oracle.paris.retrieve over the current n entries, oracle.dense.attend_row
with lo = sink, hi = sink + n).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import paris as P


def flushes(seq_len: int, n: int, sink: int, local: int, update: int) -> int:
    """Number of full buffers at length seq_len with n tokens in Retrieval:
    each full buffer moves `update` tokens from Local into Retrieval."""
    f = 0
    while seq_len - (sink + n + f * update) >= local + update:
        f += 1
    return f


def append_entries(p, index: dict, t0: int, t1: int, levels, thresh) -> dict:
    """The index grown by the keys at positions [t0, t1) of every KV head,
    each encoded on its own; the histogram gains their centroid counts."""
    ids, codes, w = [], [], []
    for h in range(p.H):
        i_, c_, w_, _ = P.encode_keys(p.keys[h, t0:t1], p.signs, p.n_sub, levels, thresh)
        ids.append(i_)
        codes.append(c_)
        w.append(w_)
    ids, codes, w = np.stack(ids), np.stack(codes), np.stack(w)
    add = np.stack([P.histogram(ids[h], 1 << p.m) for h in range(p.H)])
    return {"ids": np.concatenate([index["ids"], ids], axis=1),
            "codes": np.concatenate([index["codes"], codes], axis=1),
            "w": np.concatenate([index["w"], w], axis=1),
            "hist": index["hist"] + add,
            "pos": np.concatenate([index["pos"], np.arange(t0, t1, dtype=np.int64)])}


def prefill_index(p, L0: int, levels, thresh) -> dict:
    """Index after a prefill of L0 tokens: Retrieval = [sink, L0 - local)."""
    return P.build_index(at_length(p, L0), levels, thresh)


def at_length(p, seq_len: int, n: int | None = None):
    """The workload viewed at sequence length seq_len with n entries in
    Retrieval (default: the prefill layout, n = seq_len - sink - local):
    Paris.n is L - sink - local, so L = seq_len and local = the dense tail."""
    n = seq_len - p.sink - p.local if n is None else n
    return dataclasses.replace(p, L=seq_len, local=seq_len - p.sink - n)


def decode_step(p, index: dict, n: int, seq_len: int, q: np.ndarray, levels, thresh,
                update: int):
    """One decode step at the new length seq_len (the appended token is
    seq_len - 1): apply the buffer rule, then retrieve with query q.
    Returns (index, n, flushed, retrieval result of oracle.paris.retrieve)."""
    f = flushes(seq_len, n, p.sink, p.local, update)
    if f:
        t0 = p.sink + n
        index = append_entries(p, index, t0, t0 + f * update, levels, thresh)
        n += f * update
    view = dataclasses.replace(at_length(p, seq_len, n), q=q)
    return index, n, f, P.retrieve(view, index, levels)
