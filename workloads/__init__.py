"""Seeded synthetic inputs for the sparse decode step (shared by tests, bench and
the oracle's callers).

This module draws numbers and lays them out in the storage formats the step
reads; it contains none of the method's arithmetic (no scoring, selection,
softmax, rotation or coding).  Large arrays come from the counter-based C
generator in ``gen.c`` (Philox4x32-10 + Box-Muller), so a pool of several GB
is produced in seconds with identical bytes on every machine; small discrete
draws (permutations, liveness, planted indices, outlier channels, signs) come
from ``numpy.random.default_rng`` seeded by ``SeedSequence``.

The five workloads mirror the shapes the pages measure on (long-context decode
over a paged or token-level KV pool, a DSA-style indexer over a latent KV, and
ParisKV's compressed-code retrieval); see each ``make_*`` docstring.  bf16
tensors are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libskvgen.so")
_lib = None

# Sub-stream ids, in the fixed order: K, V, q, planted/outlier channels,
# permutation, liveness, SRHT signs, noise.
S_K, S_V, S_Q, S_PLANT, S_PERM, S_LIVE, S_SIGN, S_NOISE = range(8)


def build_lib(force: bool = False) -> str:
    """Compile gen.c into libskvgen.so (plain gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _gen():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, sz, vp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
        lib.skvgen_normal_f32.argtypes = [u64, u64, u64, sz, vp, u64, vp]
        lib.skvgen_normal_bf16.argtypes = [u64, u64, u64, sz, vp, u64, vp]
        lib.skvgen_lognormal_keys_bf16.argtypes = [u64, u64, u64, u64, sz, ctypes.c_int, ctypes.c_double, vp]
        lib.skvgen_u64.argtypes = [u64, u64, u64, sz, vp]
        lib.skvgen_philox.argtypes = [u64, u64, u64, vp]
        _lib = lib
    return _lib


def seed_of(tag: int) -> int:
    """64-bit Philox key derived from a workload tag via SeedSequence."""
    w = np.random.SeedSequence(tag).generate_state(2, dtype=np.uint32)
    return int(w[0]) | (int(w[1]) << 32)


def rngs_of(tag: int):
    """The eight numpy sub-generators of a workload tag (fixed order)."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(tag).spawn(8)]


def philox_words(seed: int, stream: int, idx: int) -> np.ndarray:
    out = np.zeros(4, np.uint32)
    _gen().skvgen_philox(seed, stream, idx, out.ctypes.data)
    return out


def normal_f32(seed, stream, shape, scale=None, offset=0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    sc = None
    period = 1
    if scale is not None:
        scale = np.ascontiguousarray(scale, np.float32)
        sc, period = scale.ctypes.data, scale.size
    _gen().skvgen_normal_f32(seed, stream, offset, n, sc, period, out.ctypes.data)
    return out.reshape(shape)


def normal_bf16(seed, stream, shape, scale=None, offset=0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    sc = None
    period = 1
    if scale is not None:
        scale = np.ascontiguousarray(scale, np.float32)
        sc, period = scale.ctypes.data, scale.size
    _gen().skvgen_normal_bf16(seed, stream, offset, n, sc, period, out.ctypes.data)
    return out.reshape(shape)


def lognormal_keys_bf16(seed, s_dir, s_norm, n_keys, d, sigma, key0=0) -> np.ndarray:
    out = np.empty((n_keys, d), np.uint16)
    _gen().skvgen_lognormal_keys_bf16(seed, s_dir, s_norm, key0, n_keys, d, sigma, out.ctypes.data)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (input storage only)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# --------------------------------------------------------------------------
# Containers
# --------------------------------------------------------------------------
@dataclass
class KV:
    """Caller-owned KV storage as the step reads it.

    paged / token-table layout (block == 16): k, v are pools
    [n_blocks][H][16][d]; contiguous (block == 0): [B][H][L_max][d].
    v is None when the value is the first d_v dims of k (shared MLA latent).
    """
    k: np.ndarray
    v: Optional[np.ndarray]
    dtype: str  # "bf16" (uint16 bits) or "f32"
    B: int
    H: int
    d_k: int
    d_v: int
    block: int
    L_max: int
    block_table: Optional[np.ndarray] = None  # int32 [B][L_max/16]
    token_table: Optional[np.ndarray] = None  # int32 [B][L_max], -1 = dead
    seq_len: Optional[np.ndarray] = None      # int32 [B]

    @property
    def mode(self) -> str:
        if self.token_table is not None:
            return "token"
        if self.block_table is not None:
            return "paged"
        return "contiguous"


@dataclass
class Step:
    """One decode step: score with (score_kv, score_q, score_G), select top-k in
    [lo, hi), attend with (kv, q, G) over selected + sink (< lo) + local (>= hi)."""
    name: str
    kv: KV
    q: np.ndarray
    G: int
    score_kv: KV
    score_q: np.ndarray
    score_G: int
    lo: np.ndarray
    hi: np.ndarray
    k: int
    scale: float
    meta: dict = field(default_factory=dict)


@dataclass
class Paris:
    """Compressed-code retrieval workload (one sequence, contiguous KV)."""
    name: str
    keys: np.ndarray     # bf16 bits [H][L][d]
    values: np.ndarray   # bf16 bits [H][L][d]
    q: np.ndarray        # bf16 bits [H*G][d]
    signs: np.ndarray    # int8 [d], +-1 (SRHT diagonal)
    H: int
    G: int
    d: int
    L: int
    n_sub: int
    m: int
    sink: int
    local: int
    rho: float
    beta: float
    k_final: int
    scale: float

    @property
    def n(self) -> int:
        return self.L - self.sink - self.local

    def kv(self) -> KV:
        return KV(k=self.keys.reshape(1, self.H, self.L, self.d),
                  v=self.values.reshape(1, self.H, self.L, self.d), dtype="bf16", B=1, H=self.H,
                  d_k=self.d, d_v=self.d, block=0, L_max=self.L,
                  seq_len=np.array([self.L], np.int32))


def live_tokens(kv: KV, b: int) -> np.ndarray:
    """Logical positions t < seq_len[b] of sequence b that the storage holds:
    a token-table entry >= 0, a block-table entry >= 0 for block t // 16, or
    any t of contiguous storage (a layout property, used for accounting)."""
    n = int(min(int(kv.seq_len[b]), kv.L_max))
    t = np.arange(n, dtype=np.int64)
    if kv.token_table is not None:
        return t[kv.token_table[b, :n] >= 0]
    if kv.block_table is not None:
        return t[kv.block_table[b, t // 16] >= 0]
    return t


def block_occupancy(token_table: np.ndarray, seq_len: np.ndarray, n_blocks: int) -> np.ndarray:
    """Live tokens per physical 16-token block of a token-table pool."""
    slots = [token_table[b, : int(seq_len[b])] for b in range(token_table.shape[0])]
    s = np.concatenate(slots) if slots else np.zeros(0, np.int32)
    s = s[s >= 0].astype(np.int64)
    return np.bincount(s // 16, minlength=n_blocks).astype(np.int32)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
def make_single_head(tag=1, L=4096, d=128, k=64, n_planted=8, noise=0.1) -> Step:
    """Single head, batch 1, fp32 contiguous K/V ~ N(0,1); the query is the
    normalised sum of `n_planted` distinct planted keys plus N(0, noise^2)
    per coordinate; top-k over all L, attention over the selected set only."""
    seed = seed_of(tag)
    r = rngs_of(tag)
    K = normal_f32(seed, S_K, (1, 1, L, d))
    V = normal_f32(seed, S_V, (1, 1, L, d))
    planted = np.sort(r[S_PLANT].choice(L, size=n_planted, replace=False))
    s = K[0, 0, planted].astype(np.float64).sum(axis=0)
    eps = normal_f32(seed, S_NOISE, (d,)).astype(np.float64) * noise
    q = (s / np.sqrt((s * s).sum()) + eps).astype(np.float32).reshape(1, 1, d)
    kv = KV(k=K, v=V, dtype="f32", B=1, H=1, d_k=d, d_v=d, block=0, L_max=L,
            seq_len=np.array([L], np.int32))
    return Step("single_head_L%d" % L, kv, q, 1, kv, q, 1, np.array([0], np.int32),
                np.array([L], np.int32), k, 1.0, meta={"planted": planted})


def make_gqa_paged(tag=2, B=4, H=8, G=4, d=128, L=32768, k=2048, sink=4, local=64,
                   n_outlier=4, outlier_scale=8.0, seq_len=None) -> Step:
    """GQA decode over a 16-token paged pool [n_blocks][H][16][d] (bf16),
    physical block order a seeded permutation reached through a per-sequence
    block table; K/V ~ N(0,1) with `n_outlier` channels per KV head scaled by
    `outlier_scale` (on K and V, before bf16 rounding); q ~ N(0,1)."""
    assert L % 16 == 0
    seed = seed_of(tag)
    r = rngs_of(tag)
    nb_seq = L // 16
    n_blocks = B * nb_seq
    ch_scale = np.ones((H, 16, d), np.float32)
    outl = np.stack([np.sort(r[S_PLANT].choice(d, size=n_outlier, replace=False)) for _ in range(H)])
    for h in range(H):
        ch_scale[h, :, outl[h]] = outlier_scale
    Kp = normal_bf16(seed, S_K, (n_blocks, H, 16, d), scale=ch_scale)
    Vp = normal_bf16(seed, S_V, (n_blocks, H, 16, d), scale=ch_scale)
    q = normal_bf16(seed, S_Q, (B, H * G, d))
    perm = r[S_PERM].permutation(n_blocks).astype(np.int32)
    bt = perm.reshape(B, nb_seq).copy()
    if seq_len is None:
        seq_len = np.full(B, L, np.int32)
    seq_len = np.asarray(seq_len, np.int32)
    kv = KV(k=Kp, v=Vp, dtype="bf16", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
            block_table=bt, seq_len=seq_len)
    lo = np.full(B, sink, np.int32)
    hi = (seq_len - local).astype(np.int32)
    return Step("gqa_paged_B%d_L%d" % (B, L), kv, q, G, kv, q, G, lo, hi, k, 1.0 / np.sqrt(d),
                meta={"outliers": outl})


def make_token_pool(tag=3, B=32, H=8, d=128, L=65536, k=2048, sink=4, local=128,
                    dead_frac=0.5, spare_blocks=0) -> Step:
    """Token-level eviction pool: a 16-token paged pool with permuted blocks;
    exactly `dead_frac` of each sequence's tokens are dead, drawn uniformly
    without replacement and left as holes inside their blocks; a token table
    maps live logical tokens to physical slots (-1 = dead).  Sink = the first
    `sink` live tokens, local = the last `local` live tokens; G = 1.
    `spare_blocks` free blocks follow the sequences' blocks in the pool
    (meta["free_blocks"]); the rest of the workload does not depend on it."""
    assert L % 16 == 0
    seed = seed_of(tag)
    r = rngs_of(tag)
    nb_seq = L // 16
    n_blocks = B * nb_seq + spare_blocks
    Kp = normal_bf16(seed, S_K, (n_blocks, H, 16, d))
    Vp = normal_bf16(seed, S_V, (n_blocks, H, 16, d))
    q = normal_bf16(seed, S_Q, (B, H, d))
    perm = r[S_PERM].permutation(B * nb_seq).astype(np.int64)
    n_dead = int(round(L * dead_frac))
    tt = np.empty((B, L), np.int32)
    lo = np.empty(B, np.int32)
    hi = np.empty(B, np.int32)
    t = np.arange(L, dtype=np.int64)
    for b in range(B):
        dead = r[S_LIVE].permutation(L)[:n_dead]
        live = np.ones(L, bool)
        live[dead] = False
        slots = perm[b * nb_seq + t // 16] * 16 + t % 16
        tt[b] = np.where(live, slots, -1).astype(np.int32)
        live_idx = np.nonzero(live)[0]
        lo[b] = live_idx[sink] if sink < live_idx.size else L
        hi[b] = live_idx[live_idx.size - local] if local > 0 else L
    kv = KV(k=Kp, v=Vp, dtype="bf16", B=B, H=H, d_k=d, d_v=d, block=16, L_max=L,
            token_table=tt, seq_len=np.full(B, L, np.int32))
    return Step("token_pool_B%d_L%d" % (B, L), kv, q, 1, kv, q, 1, lo, hi, k, 1.0 / np.sqrt(d),
                meta={"free_blocks": np.arange(B * nb_seq, n_blocks, dtype=np.int64)})


def make_indexer_mla(tag=4, L=131072, d_idx=128, d_lat=576, d_v=512, n_heads=128, k=2048) -> Step:
    """DSA-style decode, batch 1: a separate bf16 indexer key cache (one
    indexer head, d_idx) and a shared bf16 latent KV (d_lat; value = first
    d_v dims) read by `n_heads` query heads; both are 16-token paged pools
    shuffled by one seeded permutation; no sink / local."""
    assert L % 16 == 0
    seed = seed_of(tag)
    r = rngs_of(tag)
    n_blocks = L // 16
    Ki = normal_bf16(seed, S_K, (n_blocks, 1, 16, d_idx))
    Kl = normal_bf16(seed, S_V, (n_blocks, 1, 16, d_lat))
    q = normal_bf16(seed, S_Q, (1, n_heads, d_lat))
    qi = normal_bf16(seed, S_NOISE, (1, 1, d_idx))
    perm = r[S_PERM].permutation(n_blocks).astype(np.int32)
    bt = perm.reshape(1, n_blocks).copy()
    sl = np.array([L], np.int32)
    idx_kv = KV(k=Ki, v=None, dtype="bf16", B=1, H=1, d_k=d_idx, d_v=d_idx, block=16, L_max=L,
                block_table=bt, seq_len=sl)
    lat_kv = KV(k=Kl, v=None, dtype="bf16", B=1, H=1, d_k=d_lat, d_v=d_v, block=16, L_max=L,
                block_table=bt, seq_len=sl)
    return Step("indexer_mla_L%d" % L, lat_kv, q, n_heads, idx_kv, qi, 1,
                np.array([0], np.int32), np.array([L], np.int32), k, 1.0 / np.sqrt(d_lat))


def make_paris(tag=5, H=8, G=4, d=128, L=1048576, n_sub=16, sink=4, local=512, rho=0.02,
               beta=0.02, k_final=100, sigma=0.5) -> Paris:
    """Compressed-code retrieval workload, batch 1: keys k = n * g/|g| with
    g ~ N(0, I_d) and n ~ LogNormal(0, sigma); values ~ N(0,1); contiguous
    [H][L][d] bf16; q ~ N(0,1) for H*G query heads; seeded +-1 SRHT signs."""
    seed = seed_of(tag)
    r = rngs_of(tag)
    keys = lognormal_keys_bf16(seed, S_K, S_NOISE, H * L, d, sigma).reshape(H, L, d)
    values = normal_bf16(seed, S_V, (H, L, d))
    q = normal_bf16(seed, S_Q, (H * G, d))
    signs = np.where(r[S_SIGN].integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)
    return Paris("paris_L%d" % L, keys, values, q, signs, H, G, d, L, n_sub, d // n_sub, sink,
                 local, rho, beta, k_final, 1.0 / np.sqrt(d))


def paris_step_queries(p: Paris, steps: int, tag=5) -> np.ndarray:
    """Per-step query heads for a multi-step decode over a Paris workload:
    [steps][H*G][d] bf16 ~ N(0,1), drawn from the query stream after the
    workload's own query."""
    hg = p.H * p.G
    return normal_bf16(seed_of(tag), S_Q, (steps, hg, p.d), offset=hg * p.d)


# Full-size workloads by id (1..5), as measured in the bench and the
# full-size parity tests.
FULL = {
    1: make_single_head,
    2: make_gqa_paged,
    3: make_token_pool,
    4: make_indexer_mla,
    5: make_paris,
}
