"""ParisKV compressed-code retrieval, as an exact fp32 operation sequence.

Test infrastructure (see the package docstring).

Source: ParisKV close-reading (notes on arXiv 2602.07721v3):
  section 2.2 (paper Sec. 4.1.1-4.1.2, Eqs. (5)-(6)) normalise keys and query,
      rotate both by one shared orthogonal SRHT, split D into B subspaces of
      m = D/B dims, fixed centroids Omega = {(+-1/sqrt m, ...)} (|Omega| = 2^m),
      store the centroid maximising <u_b, omega>;
  section 2.3 (paper Sec. 4.2.2, App. B.2.1, Eq. (15)) per subspace keep the
      top-rho fraction of keys by query-centroid similarity, give tier weights
      6..1 at cumulative 5/15/30/50/75/100 % of that set, sum over subspaces,
      keep the top beta*n by a small-integer histogram (bucket top-k);
  section 2.4 (paper Sec. 4.1.3, Eqs. (7)-(10), Prop. 4.1) 1 sign + 3 magnitude
      bits per coordinate, alpha = <v, u>, w = |k| r_b / alpha,
      est = |q| sum_b w_b <v_b, q~_b>;
  section 2.5 (paper Sec. 4.3) C = ceil(beta n) candidates are reranked and
      only the final top-k are fetched.

Because the method is an approximation, this module follows its steps in the
pages' order, written as one fixed fp32 sequence (numpy float32: IEEE
round-to-nearest-even, correctly rounded sqrt and division, no fused
multiply-add) so that another implementation can reproduce every bit:

  tree_sum      pairwise, element j plus element j + half, halving to 1;
  norm          sqrt(tree_sum(x*x));  x^ = x / |x|  (|x| = 0 -> x^ = 0);
  SRHT          y = x^ * sigma, Sylvester-order Walsh-Hadamard butterflies
                h = 1, 2, ..., D/2 with (a, b) -> (a + b, a - b), then
                times fp32(1/sqrt(D));
  subspace b    r_b = sqrt(tree_sum over m of y^2), u = y_b / r_b (r_b = 0 ->
                u = 0, w = 0);  id bit j = [u_j < 0] (coordinate 0 = LSB;
                -0.0 and 0 count as positive); nibble = [u_j < 0] << 3 |
                #{thresholds t_i <= |u_j|}; coordinate 2c in the low nibble
                of byte c; v_j = +-levels[mag]; alpha = tree_sum(v*u);
                w_b = (|k| * r_b) / alpha;
  query         the same transform gives q~ and |q|;
                sim_b(c) = tree_sum_j(sgn_cj * q~_bj), sgn_cj = -1 iff bit j
                of c; centroids ranked by (-sim, c);
  tiers         T_rho = ceil(rho n), T_l = ceil(p_l T_rho) (float64),
                p = .05, .15, .30, .50, .75, 1.0; walking the ranked centroids
                with the exclusive prefix count P of the key histogram,
                LUT[b][c] = 7 - (smallest l with P < T_l), 0 if P >= T_rho;
  votes         S_i = max over the group's query heads of sum_b LUT[b][id_ib];
  candidates    top ceil(beta n) by (-S, i);
  rerank        est_i = max_g fl(|q_g| * tree_sum_b fl(w_ib * tree_sum_j
                fl(v_ibj * q~_gbj)));  final top-k by (-est, i).

Readings: tiers are assigned per centroid bucket (keys of one bucket share a
similarity and so a tier); rho defaults to beta (the page asks rho >= beta);
the index covers the retrieval region [sink, L - local); GQA takes the max
over the group for S and est.
"""
from __future__ import annotations

import math

import numpy as np

from .dense import bf16_bits_to_f64

F32 = np.float32
TIER_FRACS = (0.05, 0.15, 0.30, 0.50, 0.75, 1.0)


def bf16_to_f32(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def tree_sum(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    n = x.shape[-1]
    assert n & (n - 1) == 0
    while n > 1:
        h = n // 2
        x = x[..., :h] + x[..., h:n]
        n = h
    return x[..., 0]


def norm(x: np.ndarray) -> np.ndarray:
    return np.sqrt(tree_sum(x * x))


def normalise(x: np.ndarray):
    """(x / |x|, |x|) with x / 0 -> 0."""
    nrm = norm(x)
    safe = np.where(nrm > 0, nrm, F32(1)).astype(x.dtype)
    xh = np.where((nrm > 0)[..., None], x / safe[..., None], x.dtype.type(0))
    return xh.astype(x.dtype), nrm


def fwht(y: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform in Sylvester (natural) order."""
    D = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < D:
        z = y.reshape(lead + (D // (2 * h), 2, h))
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (D,))
        h *= 2
    return y


def srht(xh: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R x^ with R = H_D diag(sigma) / sqrt(D); works in the dtype of xh."""
    D = xh.shape[-1]
    y = xh * signs.astype(xh.dtype)
    y = fwht(y)
    return y * xh.dtype.type(1.0 / math.sqrt(D))


def encode_rotated(y: np.ndarray, knorm: np.ndarray, n_sub: int, levels, thresh,
                   unquantised: bool = False):
    """Code a batch of rotated unit keys y [n][D] (fp32) with norms knorm [n].

    Returns ids u8 [n][n_sub], codes u8 [n][D/2], w f32 [n][n_sub],
    and (for tests) v f32 [n][n_sub][m].  With unquantised=True the direction
    is kept exactly (v = u, alpha = sum u^2), used by the estimator pin."""
    n, D = y.shape
    m = D // n_sub
    yb = y.reshape(n, n_sub, m)
    r = norm(yb)                                            # [n][n_sub]
    rs = np.where(r > 0, r, F32(1))
    u = np.where((r > 0)[..., None], yb / rs[..., None], F32(0)).astype(F32)
    neg = u < 0
    bitw = (1 << np.arange(m)).astype(np.uint32)
    ids = (neg.astype(np.uint32) * bitw).sum(axis=-1).astype(np.uint8)
    a = np.abs(u)
    th = np.asarray(thresh, F32)
    mag = (a[..., None] >= th).sum(axis=-1).astype(np.uint8)  # 0..7
    nib = (neg.astype(np.uint8) << 3) | mag
    nibf = nib.reshape(n, D)
    codes = (nibf[:, 0::2] | (nibf[:, 1::2] << 4)).astype(np.uint8)
    lv = np.asarray(levels, F32)
    if unquantised:
        v = u.copy()
    else:
        v = np.where(neg, -lv[mag], lv[mag]).astype(F32)
    alpha = tree_sum(v * u)
    al = np.where(r > 0, alpha, F32(1))
    w = np.where(r > 0, (knorm[:, None] * r) / al, F32(0)).astype(F32)
    return ids, codes, w, v


def encode_keys(keys_bf16: np.ndarray, signs, n_sub, levels, thresh, unquantised=False):
    """Normalise, rotate and code keys [n][D] (bf16 bits)."""
    k = bf16_to_f32(keys_bf16)
    kh, kn = normalise(k)
    y = srht(kh, np.asarray(signs))
    return encode_rotated(y, kn, n_sub, levels, thresh, unquantised)


def histogram(ids: np.ndarray, n_cent: int) -> np.ndarray:
    """hist[b][c] = number of entries whose subspace-b centroid is c."""
    n, n_sub = ids.shape
    h = np.zeros((n_sub, n_cent), np.int64)
    for b in range(n_sub):
        h[b] = np.bincount(ids[:, b], minlength=n_cent)
    return h


def query_transform(q_bf16: np.ndarray, signs):
    """(q~ [Hq][D], |q| [Hq]) for bf16 query rows."""
    q = bf16_to_f32(q_bf16)
    qh, qn = normalise(q)
    return srht(qh, np.asarray(signs)), qn


def centroid_sims(qt: np.ndarray, n_sub: int) -> np.ndarray:
    """sim[b][c] = tree_sum_j(sgn_cj * q~_bj) for one rotated query q~ [D]."""
    D = qt.shape[-1]
    m = D // n_sub
    c = np.arange(1 << m)
    sgn = np.where((c[:, None] >> np.arange(m)) & 1, F32(-1), F32(1))   # [2^m][m]
    qb = qt.reshape(n_sub, 1, m)
    return tree_sum(sgn[None, :, :] * qb)                               # [n_sub][2^m]


def tier_bounds(n: int, rho: float):
    t_rho = int(math.ceil(rho * n))
    return t_rho, [int(math.ceil(p * t_rho)) for p in TIER_FRACS]


def lut_for_query(sims: np.ndarray, hist: np.ndarray, n: int, rho: float) -> np.ndarray:
    """Tier weight per (subspace, centroid) for one query head."""
    n_sub, n_cent = sims.shape
    t_rho, T = tier_bounds(n, rho)
    lut = np.zeros((n_sub, n_cent), np.uint8)
    cid = np.arange(n_cent)
    for b in range(n_sub):
        order = np.lexsort((cid, -(sims[b].astype(np.float64) + 0.0)))
        cnt = hist[b][order]
        P = np.concatenate([[0], np.cumsum(cnt)[:-1]])
        for r, c in enumerate(order):
            if P[r] >= t_rho:
                lut[b, c] = 0
            else:
                ell = next(i for i, t in enumerate(T) if P[r] < t)   # 0-based
                lut[b, c] = 6 - ell
    return lut


def votes(ids: np.ndarray, luts: np.ndarray) -> np.ndarray:
    """S_i = max_g sum_b luts[g][b][ids[i][b]]  (luts [G][n_sub][n_cent])."""
    G, n_sub, _ = luts.shape
    S = np.zeros(ids.shape[0], np.int64)
    for g in range(G):
        s = np.zeros(ids.shape[0], np.int64)
        for b in range(n_sub):
            s += luts[g, b][ids[:, b]]
        S = np.maximum(S, s)
    return S


def top_by(key: np.ndarray, count: int) -> np.ndarray:
    """Indices of the `count` largest keys, ties to the lower index, in rank order."""
    i = np.arange(key.shape[0])
    order = np.lexsort((i, -(key.astype(np.float64) + 0.0)))
    return order[:count]


def decode_codes(codes: np.ndarray, levels, n_sub: int) -> np.ndarray:
    """v [n][n_sub][m] from packed nibbles."""
    n = codes.shape[0]
    D = codes.shape[1] * 2
    nib = np.empty((n, D), np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    lv = np.asarray(levels, F32)
    mag = nib & 7
    v = np.where(nib >> 3, -lv[mag], lv[mag]).astype(F32)
    return v.reshape(n, n_sub, D // n_sub)


def rerank(codes_c, w_c, qt: np.ndarray, qn: np.ndarray, levels, n_sub: int,
           v_override=None) -> np.ndarray:
    """est per candidate (fp32): max over the query heads qt [G][D], qn [G]."""
    v = decode_codes(codes_c, levels, n_sub) if v_override is None else v_override
    G, D = qt.shape
    m = D // n_sub
    est = None
    for g in range(G):
        qb = qt[g].reshape(1, n_sub, m)
        t = tree_sum(v * qb)                       # [n_c][n_sub]
        x = w_c * t
        s = tree_sum(x)                            # [n_c]
        e = qn[g] * s
        est = e if est is None else np.maximum(est, e)
    return est.astype(F32)


def build_index(p, levels, thresh, unquantised=False, chunk=1 << 16):
    """Encode the retrieval region [sink, L - local) of every KV head.

    Returns dict ids [H][n][n_sub], codes [H][n][D/2], w [H][n][n_sub],
    hist [H][n_sub][2^m], pos [n] (logical ids), plus v when unquantised."""
    n = p.n
    H, D = p.H, p.d
    ids = np.empty((H, n, p.n_sub), np.uint8)
    codes = np.empty((H, n, D // 2), np.uint8)
    w = np.empty((H, n, p.n_sub), F32)
    vv = np.empty((H, n, p.n_sub, p.m), F32) if unquantised else None
    for h in range(H):
        for s0 in range(0, n, chunk):
            s1 = min(n, s0 + chunk)
            kb = p.keys[h, p.sink + s0:p.sink + s1]
            i_, c_, w_, v_ = encode_keys(kb, p.signs, p.n_sub, levels, thresh, unquantised)
            ids[h, s0:s1], codes[h, s0:s1], w[h, s0:s1] = i_, c_, w_
            if unquantised:
                vv[h, s0:s1] = v_
    hist = np.stack([histogram(ids[h], 1 << p.m) for h in range(H)])
    out = {"ids": ids, "codes": codes, "w": w, "hist": hist,
           "pos": np.arange(p.sink, p.sink + n, dtype=np.int64)}
    if unquantised:
        out["v"] = vv
    return out


def retrieve(p, index, levels, rho=None, beta=None, k_final=None):
    """Per KV head: votes S, candidates (ascending index), est, final logical ids."""
    rho = p.rho if rho is None else rho
    beta = p.beta if beta is None else beta
    k_final = p.k_final if k_final is None else k_final
    n = p.n
    qt, qn = query_transform(p.q, p.signs)
    C = min(n, int(math.ceil(beta * n)))
    res = {"S": [], "cand": [], "est": [], "idx": [], "luts": []}
    for h in range(p.H):
        gs = range(h * p.G, (h + 1) * p.G)
        luts = np.stack([lut_for_query(centroid_sims(qt[g], p.n_sub), index["hist"][h], n, rho)
                         for g in gs])
        S = votes(index["ids"][h], luts)
        cand = np.sort(top_by(S, C))
        v_over = index["v"][h][cand] if "v" in index else None
        est = rerank(index["codes"][h][cand], index["w"][h][cand], qt[list(gs)], qn[list(gs)],
                     levels, p.n_sub, v_override=v_over)
        fin = cand[top_by(est, min(k_final, cand.size))]
        res["S"].append(S)
        res["cand"].append(cand)
        res["est"].append(est)
        res["idx"].append(index["pos"][fin])
        res["luts"].append(luts)
    return res


def exact_top(p, k=100, heads=None):
    """True top-k logical ids per KV head by float64 max_g q_g . k_i over the
    index region (ties to the lower index)."""
    out = []
    q = bf16_bits_to_f64(p.q)
    for h in (range(p.H) if heads is None else heads):
        K = bf16_bits_to_f64(p.keys[h, p.sink:p.sink + p.n])
        s = (K @ q[h * p.G:(h + 1) * p.G].T).max(axis=1)
        out.append(p.sink + top_by(s, k))
    return out


def recall_at(final_ids, true_ids) -> float:
    """Recall@k = |final ∩ true| / |true| (ParisKV close-reading, section 一 and
    section 4.4: Recall@100 of the retrieved set against the exact top-100)."""
    return len(set(map(int, final_ids)) & set(map(int, true_ids))) / float(len(true_ids))
