"""Pins of the update-buffer oracle (no GPU): the flush rule against its
closed form and a hand-worked example, the region layout it keeps, and an
index grown by flushes against the index built in one pass."""
import numpy as np
import pytest

import workloads as W
from oracle import lloyd
from oracle import paris as P
from oracle import update as U


def _closed_form_n(seq, n0, sink, local, update):
    # tail = seq - sink - n0 tokens after the prefill; every `update` tokens
    # beyond `local` make one full buffer
    return n0 + update * max(0, (seq - sink - n0 - local) // update)


def test_flush_rule_matches_closed_form_and_keeps_layout():
    rng = np.random.default_rng(3)
    for _ in range(200):
        sink, local, update = int(rng.integers(0, 9)), int(rng.integers(0, 40)), int(rng.integers(1, 20))
        L0 = sink + local + int(rng.integers(0, 100))
        n = n0 = L0 - sink - local
        total = 0
        appends = 4 * update + 2
        for seq in range(L0 + 1, L0 + appends + 1):
            f = U.flushes(seq, n, sink, local, update)
            assert f in (0, 1)                      # one token appended per step
            n += f * update
            total += f
            assert n == _closed_form_n(seq, n0, sink, local, update)
            tail = seq - sink - n                   # Local + buffer, attended densely
            assert local <= tail < local + update
        assert total == appends // update


def test_hand_worked_example():
    """sink 4, Local 8, buffer 4, prefill 20 tokens: Retrieval [4, 12), dense
    tail [12, 20).  Appending tokens 20, 21, 22 fills the buffer to 3; token
    23 makes it full (tail 12 = 8 + 4), so tokens 12..15 (the oldest Local
    ones) are encoded: Retrieval [4, 16), tail [16, 24)."""
    n = 20 - 4 - 8
    got = []
    for seq in range(21, 30):
        n += U.flushes(seq, n, 4, 8, 4) * 4
        got.append(n)
    assert got == [8, 8, 8, 12, 12, 12, 12, 16, 16]
    # several tokens at once: 9 more tokens after seq 20 -> two full buffers
    assert U.flushes(29, 8, 4, 8, 4) == 2


def test_grown_index_equals_one_pass_index():
    p = W.make_paris(tag=61, H=2, G=2, L=1400, sink=4, local=64)
    lv, th = lloyd.codebook_f32(8)
    L0, update = 1000, 48
    index = U.prefill_index(p, L0, lv, th)
    n = L0 - p.sink - p.local
    assert index["ids"].shape[1] == n
    flushed = 0
    qs = W.paris_step_queries(p, 3)
    for i, seq in enumerate(range(L0 + 1, 1400)):
        if i % 97 == 0:          # a full decode step now and then: flush, then retrieve
            index, n, f, res = U.decode_step(p, index, n, seq, qs[i % 3], lv, th, update)
            for h in range(p.H):
                assert np.all((res["idx"][h] >= p.sink) & (res["idx"][h] < p.sink + n))
        else:                    # otherwise only the buffer rule
            f = U.flushes(seq, n, p.sink, p.local, update)
            if f:
                index = U.append_entries(p, index, p.sink + n, p.sink + n + f * update, lv, th)
                n += f * update
        flushed += f
    assert flushed == (1399 - L0) // update
    one = P.build_index(U.at_length(p, 1399, n), lv, th)
    for key in ("ids", "codes", "hist", "pos"):
        assert np.array_equal(index[key], one[key]), key
    assert np.array_equal(index["w"].view(np.uint32), one["w"].view(np.uint32))
    # the histogram counts every entry once per subspace
    assert np.all(index["hist"].sum(axis=2) == n)
