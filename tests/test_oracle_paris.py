"""Pins of the ParisKV retrieval oracle (no GPU): explicit matrices, brute
force over the codebook, closed forms, quadrature, hand-worked tier tables and
the exact special cases the pages imply."""
import itertools
import math

import numpy as np
import pytest
from scipy.integrate import quad
from scipy.linalg import hadamard

import workloads as W
from oracle import closed_forms as cf
from oracle import lloyd
from oracle import paris as P

F32 = np.float32


def _signs(D, seed=0):
    return np.where(np.random.default_rng(seed).integers(0, 2, D) == 1, 1, -1).astype(np.int8)


# ---------------------------------------------------------------------- SRHT
def test_srht_is_hadamard_times_signs_over_sqrt_d():
    D = 128
    sg = _signs(D)
    R = hadamard(D).astype(np.float64) @ np.diag(sg.astype(np.float64)) / math.sqrt(D)
    x = np.random.default_rng(1).standard_normal((5, D))
    np.testing.assert_allclose(P.srht(x, sg), x @ R.T, rtol=0, atol=1e-12)
    x32 = x.astype(F32)
    np.testing.assert_allclose(P.srht(x32, sg), x32.astype(np.float64) @ R.T, atol=2e-6)


def test_srht_preserves_norms_and_inner_products():
    D = 128
    sg = _signs(D, 2)
    x, y = np.random.default_rng(3).standard_normal((2, 7, D))
    Rx, Ry = P.srht(x, sg), P.srht(y, sg)
    np.testing.assert_allclose((Rx * Ry).sum(-1), (x * y).sum(-1), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(Rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_tree_sum_order():
    x = np.array([1e8, 1.0, -1e8, 1.0], F32)      # (1e8 + -1e8) + (1 + 1) = 2
    assert P.tree_sum(x) == F32(2.0)
    y = np.arange(8, dtype=F32)
    assert P.tree_sum(y) == 28.0


# ------------------------------------------------------------------ codebook
def _omega(m):
    return np.array(list(itertools.product([1.0, -1.0], repeat=m)))[:, ::-1] / math.sqrt(m)


def test_codebook_size_distinct_unit_norm():
    for m in (2, 3, 8):
        om = _omega(m)
        assert om.shape[0] == cf.codebook_size(m) == 2 ** m
        assert len({tuple(r) for r in om}) == 2 ** m
        np.testing.assert_allclose(np.linalg.norm(om, axis=1), 1.0)


def test_centroid_id_is_argmax_over_all_centroids():
    m, n_sub = 8, 16
    lv, th = lloyd.codebook_f32(m)
    y = np.random.default_rng(4).standard_normal((300, m * n_sub)).astype(F32)
    ids, _, _, _ = P.encode_rotated(y, np.ones(300, F32), n_sub, lv, th)
    om = _omega(m)
    # centroid c <-> sign pattern: bit j set <=> coordinate j negative
    sgn = np.where((np.arange(2 ** m)[:, None] >> np.arange(m)) & 1, -1.0, 1.0) / math.sqrt(m)
    assert {tuple(r) for r in sgn} == {tuple(r) for r in om}
    for i in range(300):
        for b in range(n_sub):
            u = y[i, b * m:(b + 1) * m].astype(np.float64)
            assert int(np.argmax(sgn @ u)) == int(ids[i, b])


def test_mean_subspace_energy_is_m_over_d():
    """E[r_b^2] = m / D for isotropic keys (mean of Beta(m/2, (D-m)/2))."""
    D, m = 128, 8
    sg = _signs(D, 5)
    k = W.normal_f32(W.seed_of(77), 0, (100_000, D))
    kh, _ = P.normalise(k)
    y = P.srht(kh, sg).reshape(-1, D // m, m).astype(np.float64)
    r2 = (y * y).sum(-1)
    assert abs(r2.mean() - m / D) < 0.01 * m / D
    for b in range(D // m):
        assert abs(r2[:, b].mean() - m / D) < 0.02 * m / D


# ------------------------------------------------------------------ Lloyd-Max
def test_lloyd_m3_is_the_uniform_quantiser():
    """m = 3: (u_j)^2 ~ Beta(1/2, 1) makes |u_j| uniform on [0, 1], whose 8-level
    Lloyd-Max quantiser has levels (2i+1)/16 and thresholds i/8."""
    lv, th = lloyd.lloyd_max_abs_coord(3)
    np.testing.assert_allclose(lv, (2 * np.arange(8) + 1) / 16, atol=1e-12)
    np.testing.assert_allclose(th, np.arange(1, 8) / 8, atol=1e-12)


def test_lloyd_m8_fixed_point_by_quadrature():
    m = 8
    lv, th = lloyd.lloyd_max_abs_coord(m)
    f = lambda y: (1 - y * y) ** ((m - 3) / 2)
    edges = np.concatenate([[0.0], th, [1.0]])
    for i in range(8):
        a, b = edges[i], edges[i + 1]
        mean = quad(lambda y: y * f(y), a, b, epsabs=1e-14, epsrel=1e-13)[0] / \
            quad(f, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(mean - lv[i]) < 1e-10
    np.testing.assert_allclose(th, 0.5 * (lv[:-1] + lv[1:]), rtol=1e-15)
    assert np.all(np.diff(lv) > 0) and 0 < lv[0] and lv[-1] < 1
    # self-derived reference values (informational, 5 digits)
    ref = [0.04251, 0.12804, 0.21520, 0.30532, 0.40027, 0.50302, 0.61935, 0.76484]
    np.testing.assert_allclose(lv, ref, atol=1e-5)


# -------------------------------------------------------------------- coding
def test_nibbles_ids_and_weights_by_hand():
    """D = 16, n_sub = 2, m = 8, thresholds 0.1 .. 0.7, levels 0.05 .. 0.75.
    Subspace 0 holds u = y / 1 (|y| = 1); subspace 1 is all zero."""
    th = np.array([0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7], F32)
    lv = np.array([0.05, 0.15, 0.25, 0.35, 0.45, 0.55, 0.65, 0.75], F32)
    u0 = np.array([0.8, -0.0, -0.35, 0.1, 0.0, -0.05, 0.4, -0.2], np.float64)
    u0 = u0 / np.linalg.norm(u0)
    y = np.zeros((1, 16), F32)
    y[0, :8] = u0.astype(F32)
    ids, codes, w, v = P.encode_rotated(y, np.array([2.0], F32), 2, lv, th)
    u = y[0, :8] / P.norm(y[0, :8])
    neg = (u < 0)
    assert ids[0, 0] == sum(1 << j for j in range(8) if neg[j])
    assert ids[0, 0] == 0b10100100            # coords 2, 5, 7 negative; -0.0 positive
    mags = [sum(1 for t in th if abs(x) >= t) for x in u]
    nib = [(8 if neg[j] else 0) | mags[j] for j in range(8)]
    assert codes[0, :4].tolist() == [nib[0] | nib[1] << 4, nib[2] | nib[3] << 4,
                                     nib[4] | nib[5] << 4, nib[6] | nib[7] << 4]
    assert ids[0, 1] == 0 and codes[0, 4:].tolist() == [0, 0, 0, 0] and w[0, 1] == 0
    vv = np.array([(-1 if neg[j] else 1) * lv[mags[j]] for j in range(8)], F32)
    np.testing.assert_array_equal(v[0, 0], vv)
    r = P.norm(y[0, :8])
    np.testing.assert_array_equal(w[0, 0], (F32(2.0) * r) / P.tree_sum(vv * u))


def test_estimator_is_exact_without_quantisation():
    """With v = u the rerank estimate equals <k, q> (alpha = 1, radii exact)."""
    D, n_sub = 128, 16
    sg = _signs(D, 6)
    keys = W.lognormal_keys_bf16(W.seed_of(78), 0, 1, 64, D, 0.5)
    q = W.normal_bf16(W.seed_of(79), 0, (1, D))
    lv, th = lloyd.codebook_f32(8)
    ids, codes, w, v = P.encode_keys(keys, sg, n_sub, lv, th, unquantised=True)
    qt, qn = P.query_transform(q, sg)
    est = P.rerank(codes, w, qt, qn, lv, n_sub, v_override=v)
    exact = P.bf16_to_f32(keys).astype(np.float64) @ P.bf16_to_f32(q)[0].astype(np.float64)
    np.testing.assert_allclose(est, exact, rtol=2e-5, atol=2e-5 * np.abs(exact).max())


def test_quantised_estimator_is_close():
    D, n_sub = 128, 16
    sg = _signs(D, 7)
    keys = W.lognormal_keys_bf16(W.seed_of(80), 0, 1, 2000, D, 0.5)
    q = W.normal_bf16(W.seed_of(81), 0, (1, D))
    lv, th = lloyd.codebook_f32(8)
    _, codes, w, _ = P.encode_keys(keys, sg, n_sub, lv, th)
    qt, qn = P.query_transform(q, sg)
    est = P.rerank(codes, w, qt, qn, lv, n_sub).astype(np.float64)
    exact = P.bf16_to_f32(keys).astype(np.float64) @ P.bf16_to_f32(q)[0].astype(np.float64)
    assert np.corrcoef(est, exact)[0, 1] > 0.97


# --------------------------------------------------------------- collision vote
def test_tier_lut_hand_example():
    """m = 2 (4 centroids), one subspace, n = 20 keys, hist = [5, 3, 10, 2],
    rho = 0.5 -> T_rho = 10 and T = ceil(p * 10) = [1, 2, 3, 5, 8, 10].
    q~ = (-0.6, 0.8): sims c0 = 0.2, c1 = 1.4, c2 = -1.4, c3 = -0.2, so the
    ranking is c1, c0, c3, c2 with exclusive prefix counts P = 0, 3, 8, 10.
    Weights (7 - smallest l with P < T_l): c1 -> 6; c0 -> l = 4 -> 3;
    c3 -> l = 6 -> 1; c2 has P >= T_rho -> 0."""
    assert P.tier_bounds(20, 0.5) == (10, [1, 2, 3, 5, 8, 10])
    sims = P.centroid_sims(np.array([-0.6, 0.8], F32), 1)
    assert np.argsort(-sims[0]).tolist() == [1, 0, 3, 2]
    lut = P.lut_for_query(sims, np.array([[5, 3, 10, 2]]), 20, 0.5)
    assert lut[0].tolist() == [3, 6, 0, 1]


def test_tier_weights_first_bucket_is_six_and_ties_rank_by_id():
    sims = np.array([[0.5, 0.5, 0.1, 0.5]], F32)
    lut = P.lut_for_query(sims, np.array([[1, 1, 1, 1]]), 100, 1.0)
    # T_rho = 100, T = [5, 15, 30, 50, 75, 100]; ranked c0, c1, c3, c2 with P = 0, 1, 2, 3
    assert lut[0].tolist() == [6, 6, 6, 6]
    lut2 = P.lut_for_query(sims, np.array([[10, 20, 1, 40]]), 100, 1.0)
    # P: c0 0 -> 6, c1 10 -> 5 (10 < 15), c3 30 -> 3 (30 < 50), c2 70 -> 2 (70 < 75)
    assert lut2[0].tolist() == [6, 5, 2, 3]


def test_votes_sum_over_subspaces_max_over_group():
    ids = np.array([[0, 1], [1, 1], [2, 0]], np.uint8)
    luts = np.zeros((2, 2, 4), np.uint8)
    luts[0, 0] = [6, 1, 0, 0]
    luts[0, 1] = [2, 3, 0, 0]
    luts[1, 0] = [0, 0, 5, 0]
    luts[1, 1] = [4, 0, 0, 0]
    assert P.votes(ids, luts).tolist() == [max(6 + 3, 0 + 0), max(1 + 3, 0 + 0), max(0 + 2, 5 + 4)]


@pytest.mark.parametrize("seed", range(10))
def test_top_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    S = rng.integers(0, 5, size=9)
    c = int(rng.integers(1, 9))
    got = set(P.top_by(S, c).tolist())
    ok = [set(T) for T in itertools.combinations(range(9), c)
          if all(S[i] > S[j] or (S[i] == S[j] and i < j) for i in T for j in range(9) if j not in T)]
    assert ok == [got]


def test_full_budget_unquantised_pipeline_is_exact_topk():
    """beta = rho = 1 and unquantised directions: every key is a candidate and
    est = <k, q> (fp32), so the final set is the exact top-k."""
    p = W.make_paris(tag=905, H=2, G=2, d=128, L=1200, sink=4, local=16, rho=1.0, beta=1.0,
                     k_final=100)
    lv, th = lloyd.codebook_f32(8)
    idx = P.build_index(p, lv, th, unquantised=True)
    res = P.retrieve(p, idx, lv)
    true = P.exact_top(p, 100)
    for h in range(p.H):
        assert len(res["cand"][h]) == p.n
        assert P.recall_at(res["idx"][h], true[h]) >= 0.99
    assert sum(P.recall_at(res["idx"][h], true[h]) for h in range(p.H)) / p.H >= 0.995


def test_quantised_pipeline_shapes_and_budget():
    p = W.make_paris(tag=906, H=2, G=4, d=128, L=6000, sink=4, local=64)
    lv, th = lloyd.codebook_f32(8)
    idx = P.build_index(p, lv, th)
    assert idx["hist"].sum(axis=-1).tolist() == [[p.n] * 16] * 2
    res = P.retrieve(p, idx, lv)
    C = cf.n_candidates(p.beta, p.n)
    for h in range(p.H):
        assert res["cand"][h].size == C
        assert np.all(np.diff(res["cand"][h]) > 0)
        assert len(set(res["idx"][h].tolist())) == p.k_final
        assert np.all((res["idx"][h] >= p.sink) & (res["idx"][h] < p.L - p.local))
        # every candidate has a vote at least as large as every non-candidate
        S = res["S"][h]
        mask = np.zeros(p.n, bool)
        mask[res["cand"][h]] = True
        assert S[mask].min() >= S[~mask].max()


# ------------------------------------------------ histogram and zero-row pins
def test_histogram_counts_each_subspace_column_separately():
    """A hand-built id matrix whose subspaces have different counts: a
    histogram built from one column for every row, or over the flattened
    matrix, or with the axes swapped, fails this."""
    ids = np.array([[3, 0, 7],
                    [3, 1, 7],
                    [5, 1, 7],
                    [3, 1, 0],
                    [0, 2, 7]], np.uint8)
    h = P.histogram(ids, 8)
    assert h.shape == (3, 8)
    assert h[0].tolist() == [1, 0, 0, 3, 0, 1, 0, 0]
    assert h[1].tolist() == [1, 3, 1, 0, 0, 0, 0, 0]
    assert h[2].tolist() == [1, 0, 0, 0, 0, 0, 0, 4]
    assert h.sum(axis=1).tolist() == [5, 5, 5]


def test_normalise_zero_rows_give_zero_direction_and_norm():
    """Reading 17: a zero row normalises to the zero vector with norm 0 (no
    NaN), and leaves the other rows of the batch untouched."""
    x = np.zeros((3, 128), F32)
    x[1, 5] = F32(-3.0)
    x[2, :] = F32(0.5)
    xh, nrm = P.normalise(x)
    assert nrm.dtype == F32 and nrm.tolist() == [0.0, 3.0, float(np.sqrt(F32(32.0)))]
    assert np.all(xh[0] == 0) and not np.isnan(xh).any()
    assert xh[1, 5] == F32(-1.0) and np.count_nonzero(xh[1]) == 1
    np.testing.assert_allclose(np.linalg.norm(xh[2].astype(np.float64)), 1.0, rtol=1e-6)
    # a zero key encodes to id 0, codes 0 and w 0 (reading 17)
    lv, th = lloyd.codebook_f32(8)
    ids, codes, w, _ = P.encode_keys(np.zeros((1, 128), np.uint16), _signs(128, 9), 16, lv, th)
    assert not ids.any() and not codes.any() and not w.any()


def test_candidate_budget_values():
    """C = ceil(beta n), written out: the full workload's n = 1,048,060 at
    beta = 0.02 gives 20,962 (2 % of n is 20,961.2); exact multiples are
    not rounded up; beta = 1 keeps every entry."""
    assert cf.n_candidates(0.02, 1048060) == 20962
    assert cf.n_candidates(0.02, 100) == 2
    assert cf.n_candidates(0.02, 101) == 3
    assert cf.n_candidates(0.05, 2000) == 100
    assert cf.n_candidates(1.0, 777) == 777
    assert cf.n_candidates(0.1, 5) == 1
