"""Pins of the clustering and compression oracle (CPU only) against what
the page and the mathematics fix: closed forms, invariants, library
routines on special cases, brute force on tiny inputs, planted structure.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from compressed_expert_ffn_amd import synth
from oracle import cluster_oracle as C


# ------------------------------------------------------------- centroids
def test_ema_closed_form_and_untouched_experts():
    """n steps with the same batch from mu = 0 give (1 - (1 - beta)^n) xbar;
    an expert that gets no row keeps its centroid."""
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 5))
    idx = np.array([[0, 2]] * 4 + [[2, 3]] * 3)
    mu = np.zeros((5, 5))
    mu[4] = 3.0
    beta = 0.05
    for _ in range(9):
        mu = C.ema_centroids(mu, X, idx, beta)
    f = 1 - (1 - beta) ** 9
    assert np.allclose(mu[0], f * X[:4].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert np.allclose(mu[2], f * X.mean(axis=0), rtol=1e-13, atol=1e-15)
    assert np.allclose(mu[3], f * X[4:].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert (mu[1] == 0).all() and (mu[4] == 3.0).all()


# ------------------------------------------------------------ similarity
def test_cosine_matrix_against_scipy_and_zero_vector():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((6, 9))
    V[:, 0] += 2.0
    assert np.allclose(C.cosine_matrix(V), 1.0 - cdist(V, V, "cosine"), atol=1e-14)
    V[3] = 0.0
    S = C.cosine_matrix(V)
    assert S[3, 3] == 1.0 and (np.delete(S[3], 3) == 0).all() and (np.delete(S[:, 3], 3) == 0).all()
    # scale invariance and the sign of opposite vectors
    W = V.copy()
    W[1] *= 7.5
    W[2] = -V[0]
    S2 = C.cosine_matrix(W)
    assert np.isclose(S2[1, 4], S[1, 4], atol=1e-14) and np.isclose(S2[2, 0], -1.0, atol=1e-14)


def test_fused_similarity_weights_and_pruning():
    rng = np.random.default_rng(2)
    Sp = C.cosine_matrix(rng.standard_normal((5, 8)))
    St = C.cosine_matrix(rng.standard_normal((5, 8)))
    S1, _ = C.fused_distance(Sp, St, 1.0, -2.0)
    S0, _ = C.fused_distance(Sp, St, 0.0, -2.0)
    assert np.allclose(S1, Sp, atol=0) and np.allclose(S0, St, atol=0)
    S, D = C.fused_distance(Sp, St, 0.7, 0.1)
    raw = 0.7 * Sp + 0.3 * St
    off = ~np.eye(5, dtype=bool)
    assert ((S[off] == 0) == (raw[off] < 0.1)).all()
    assert np.allclose(S[off & (raw >= 0.1)], raw[off & (raw >= 0.1)], atol=1e-15)
    assert (np.diag(D) == 0).all() and np.allclose(D, 1 - S, atol=0)


def test_param_cache_refresh_rule():
    rng = np.random.default_rng(3)
    vecs = [rng.standard_normal(40) for _ in range(5)]
    S0, cache, fresh = C.param_similarity_cached(vecs, None, eps=1e-3, life=3)
    assert fresh == [0, 1, 2, 3, 4] and np.allclose(S0, C.cosine_matrix(np.stack(vecs)), atol=1e-15)
    moved = [v.copy() for v in vecs]
    moved[1] = vecs[1] + 1e-5 * rng.standard_normal(40)   # below eps: cached
    moved[2] = vecs[2] + 0.1 * rng.standard_normal(40)    # above eps: recomputed
    S1, cache, fresh = C.param_similarity_cached(moved, cache, eps=1e-3, life=3)
    assert fresh == [2]
    expect = C.cosine_matrix(np.stack([vecs[0], vecs[1], moved[2], vecs[3], vecs[4]]))
    assert np.allclose(S1, expect, atol=1e-15)
    # a row serves `life` reclusterings: the untouched rows, computed at the
    # first, are recomputed at the fourth; row 2 (recomputed at the second)
    # is still cached then
    S2, cache, fresh = C.param_similarity_cached(moved, cache, eps=1e-3, life=3)
    assert fresh == []
    S2, cache, fresh = C.param_similarity_cached(moved, cache, eps=1e-3, life=3)
    assert fresh == [0, 1, 3, 4]
    assert np.allclose(S2, C.cosine_matrix(np.stack(moved)), atol=1e-15)


# ------------------------------------------------------------ clustering
def _kmedoids_cost(D, assign, medoids):
    return sum(D[i, medoids[assign[i]]] for i in range(len(assign)))


def test_seeding_hand_example():
    """Four points on a line at 0, 1, 3, 10 (D = |a - b| / 10): seed 0 is
    floor(u0 E); seed 1 follows the running sum of squared distances."""
    p = np.array([0.0, 1.0, 3.0, 10.0])
    D = np.abs(p[:, None] - p[None, :]) / 10
    # seed 0 = floor(0.3 * 4) = 1; d^2 to it = .01, 0, .04, .81 (total .86);
    # u1 = 0.05 -> target .043: running sums .01, .01, .05 -> expert 2
    _, med = C.kmeanspp_medoids(D, 2, [0.3, 0.05], max_iter=0)
    assert list(med) == [1, 2]
    _, med = C.kmeanspp_medoids(D, 2, [0.3, 0.9], max_iter=0)   # target .774 -> expert 3
    assert list(med) == [1, 3]


@pytest.mark.parametrize("E,G,seed", [(6, 2, 0), (6, 3, 1), (8, 2, 2), (7, 3, 3)])
def test_kmedoids_fixed_point_and_global_optimum_tiny(E, G, seed):
    """The result is a k-medoids fixed point, and on well-separated tiny
    inputs it reaches the exhaustive optimum of the k-medoids cost."""
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((G, 4)) * 5
    pts = centres[np.arange(E) % G] + 0.1 * rng.standard_normal((E, 4))
    D = cdist(pts, pts) / 50
    u = rng.random(G)
    assign, med = C.kmeanspp_medoids(D, G, u)
    for i in range(E):
        assert D[i, med[assign[i]]] == min(D[i, m] for m in med)
    for g in range(G):
        mem = np.nonzero(assign == g)[0]
        costs = [D[a, mem].sum() for a in mem]
        assert D[med[g], mem].sum() == min(costs)
    best = min(sum(min(D[i, m] for m in ms) for i in range(E))
               for ms in itertools.combinations(range(E), G))
    assert math.isclose(_kmedoids_cost(D, assign, med), best, rel_tol=1e-12)


def test_planted_clusters_recovered():
    """Experts drawn around planted centres, tokens drawn around group
    directions: the fused distance splits them exactly as planted."""
    E, G = 32, 4
    bank = synth.make_expert_bank(E, G, [(24, 40), (40, 24)], rank=3, resid_scale=0.3, noise_scale=0.01)
    vecs = [np.concatenate([W[i].reshape(-1) for W in bank["W"]]) for i in range(E)]
    X, idx = synth.draw_group_tokens(bank["planted"], G, 16, 4000, 2)
    mu = np.zeros((E, 16))
    for s in range(0, 4000, 500):
        mu = C.ema_centroids(mu, X[s:s + 500], idx[s:s + 500], 0.05)
    Sp, _, _ = C.param_similarity_cached(vecs, None, 1e-3, 4)
    St = C.cosine_matrix(mu)
    _, D = C.fused_distance(Sp, St, 0.7, 0.1)
    u = np.random.default_rng(7).random(G)
    assign, med = C.kmeanspp_medoids(D, G, u)
    assign = C.rebalance(assign, D, med, E // G)
    planted = bank["planted"]
    for g in range(G):
        assert len(set(planted[assign == g])) == 1
    assert len(set(assign)) == G


def test_rebalance_sizes_and_who_moves():
    rng = np.random.default_rng(4)
    pts = rng.standard_normal((9, 3))
    D = cdist(pts, pts) / 10
    assign = np.array([0, 0, 0, 0, 0, 1, 1, 2, 2])
    med = [0, 5, 7]
    out = C.rebalance(assign, D, med, 3)
    assert (np.bincount(out, minlength=3) == 3).all()
    assert (out[5:] == assign[5:]).all()          # members of groups at or under K stay
    # the two moves, by hand: each time the cheapest (expert, target) pair
    moves = []
    a = assign.copy()
    for _ in range(2):
        sizes = np.bincount(a, minlength=3)
        cand = [(D[i, med[h]] - D[i, med[a[i]]], i, h) for i in range(9) if sizes[a[i]] > 3
                for h in range(3) if sizes[h] < 3]
        _, i, h = min(cand)
        a[i] = h
        moves.append((i, h))
    assert (out == a).all()


# ----------------------------------------------------------- compression
def test_base_is_the_mean_and_residuals_sum_to_zero():
    rng = np.random.default_rng(5)
    Ws = [rng.standard_normal((6, 4)) for _ in range(6)]
    members = np.array([[0, 3, 5], [1, 2, 4]])
    base, A, B, err = C.compress_projection(Ws, members, r=2)
    for g in range(2):
        resid = [Ws[i] - base[g] for i in members[g]]
        assert np.allclose(sum(resid), 0.0, atol=1e-14)
        # the mean minimises the summed squared distance: any shift raises it
        f0 = sum(np.linalg.norm(x) ** 2 for x in resid)
        shift = rng.standard_normal((6, 4)) * 1e-3
        assert sum(np.linalg.norm(x - shift) ** 2 for x in resid) > f0


def test_tsvd_error_is_the_eckart_young_tail():
    """||R - A B^T||_F^2 = sum of the squared singular values past r, taken
    here from the eigenvalues of R^T R (numpy's symmetric eigensolver)."""
    rng = np.random.default_rng(6)
    Ws = [rng.standard_normal((12, 9)) for _ in range(4)]
    members = np.array([[0, 1, 2, 3]])
    for r in (1, 3, 5):
        base, A, B, err = C.compress_projection(Ws, members, r)
        for j, i in enumerate(members[0]):
            R = Ws[i] - base[0]
            ev = np.sort(np.linalg.eigvalsh(R.T @ R))[::-1]
            tail = max(ev[r:].sum(), 0.0)
            got = np.linalg.norm(R - A[j] @ B[j].T) ** 2
            assert math.isclose(got, tail, rel_tol=1e-9, abs_tol=1e-12)
            assert math.isclose(err[j], math.sqrt(tail) / np.linalg.norm(Ws[i]), rel_tol=1e-9, abs_tol=1e-12)
            # singular values split evenly over the factors
            assert np.allclose(np.linalg.norm(A[j], axis=0), np.linalg.norm(B[j], axis=0), rtol=1e-12)
            assert np.allclose(np.linalg.norm(A[j], axis=0) ** 4, ev[:r], rtol=1e-9)


def test_exact_when_residuals_have_rank_r():
    rng = np.random.default_rng(7)
    centre = rng.standard_normal((10, 14))
    Ws = [centre + rng.standard_normal((10, 3)) @ rng.standard_normal((3, 14)) for _ in range(3)]
    # the group mean shifts each residual by the mean of the others: rank <= 3*3
    base, A, B, err = C.compress_projection(Ws, np.array([[0, 1, 2]]), r=9)
    assert err.max() < 1e-12
    base, A, B, err = C.compress_projection(Ws[:1], np.array([[0]]), r=2)
    assert np.array_equal(base[0], Ws[0]) and np.allclose(A, 0) and np.allclose(B, 0) and err[0] == 0


def test_error_bound_at_rank_16_and_not_at_rank_4():
    """Synthetic experts (group centre + rank-16 spread + 0.5% noise) stay
    within the 1.5% Frobenius error at r = 16 and exceed it at r = 4, as in
    the page's ablation table."""
    E, G = 8, 2
    bank = synth.make_expert_bank(E, G, [(96, 160)], rank=16, resid_scale=0.3, noise_scale=0.005)
    members = np.stack([np.nonzero(bank["planted"] == g)[0] for g in range(G)])
    Ws = list(bank["W"][0])
    _, _, _, e16 = C.compress_projection(Ws, members, 16)
    _, _, _, e4 = C.compress_projection(Ws, members, 4)
    assert e16.max() <= 0.015 < e4.min()


def test_stored_parameter_count_is_the_compression_formula():
    d_in, d_out, K, r = 48, 80, 4, 6
    rng = np.random.default_rng(8)
    Ws = [rng.standard_normal((d_in, d_out)) for _ in range(2 * K)]
    members = np.arange(2 * K).reshape(2, K)
    base, A, B, _ = C.compress_projection(Ws, members, r)
    stored = base.size + A.size + B.size
    dense = len(Ws) * d_in * d_out
    assert math.isclose(dense / stored, C.compression_ratio(d_in, d_out, K, r), rel_tol=1e-15)
