"""Closed forms the pages state — test infrastructure (see package docstring).

* kv_bytes: OasisKV reading notes, section 1, Eq. (1):
  M_KV(B, L) = B * L * N_layer * 2 N_kv d_h * s  (also vToken's per-token
  2 L H D dtype in its background section).
* waste_ratio: vToken reading notes, section 2, Eq. (1):
  F = 1 - sum_i n_i / (N S).
* read_bytes / read_fraction: UlaCache article, section 二: a sparse step
  reads about k * s_kv bytes, rho_read = k / L.
* n_candidates: ParisKV close-reading, section 2.5 (paper Sec. 4.3):
  C = ceil(beta * n).
* codebook_size: ParisKV close-reading, section 2.2 (paper Eq. (5)): |Omega| = 2^m.
"""
from __future__ import annotations

import math


def kv_bytes(B: int, L: int, n_layer: int, n_kv: int, d_h: int, s: int) -> int:
    return B * L * n_layer * 2 * n_kv * d_h * s


def waste_ratio(n_live, S: int) -> float:
    n_live = list(n_live)
    return 1.0 - sum(n_live) / (len(n_live) * S)


def read_bytes(k: int, s_kv: int) -> int:
    return k * s_kv


def read_fraction(k: int, L: int) -> float:
    return k / L


def n_candidates(beta: float, n: int) -> int:
    return int(math.ceil(beta * n))


def codebook_size(m: int) -> int:
    return 2 ** m
