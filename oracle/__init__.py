"""CPU oracle for the sparse top-k decode step — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the GPU path
computes, written from the pages' definitions.  It shares no code with the
HIP library and imports nothing from it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it; the product path never routes through it.

Modules
-------
dense         exact definition of the step (score every key, exact top-k with
              the lowest index winning ties, dense-then-masked softmax), in
              float64, with its own logical->physical addressing.
paris         ParisKV compressed-code retrieval (normalise, SRHT, fixed
              sign-pattern centroids, collision vote, 4-bit rerank, top-k),
              as an exact fp32 operation sequence in numpy.
blocks        block-summary scoring (per-block coordinate-wise min / max of
              the keys, Quest's upper bound as the block score, exact top-K
              blocks, attention over their tokens), float64.
update        the compressed path's Update Buffer (full buffers move into
              Local, the Local tokens they push out are encoded into the
              index) and its multi-step decode loop.
compact       token-table compaction: waste ratio, relocation plan (threshold,
              headroom, net-freeing gates), applying moves, and the I1 / I2
              checks (a position-independent hash of the retained tokens,
              duplicate-slot counts).
validate      the checks of device-resident data a step takes on trust
              (sequence lengths, windows, table entries inside the pool, no
              slot mapped twice, selected positions in range and distinct).
lloyd         Lloyd-Max levels for |u_j| under the Beta prior, float64.
closed_forms  byte / capacity formulas the pages state.

Pinning: every function is pinned by ``tests/test_oracle_*.py`` against
brute force, closed forms, library routines or the pages' worked examples.
The Recall@100 *values* the pages print come from real-model traces and are
parity unpinned against the pages; recall here is pinned only by definition.
"""
