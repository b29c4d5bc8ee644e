"""Plant plausible mistakes in the clustering and compression oracle (on
the CPU, via monkeypatch) and check that a pin in test_cluster_oracle.py
catches each of them."""
import numpy as np
import pytest

from oracle import cluster_oracle as C
from tests import test_cluster_oracle as P

_orig = {name: getattr(C, name) for name in (
    "ema_centroids", "cosine_matrix", "fused_distance", "kmeanspp_medoids", "rebalance",
    "compress_projection", "param_similarity_cached")}


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError, TypeError):
        return True
    return False


def _pins():
    return [
        (P.test_ema_closed_form_and_untouched_experts, ()),
        (P.test_cosine_matrix_against_scipy_and_zero_vector, ()),
        (P.test_fused_similarity_weights_and_pruning, ()),
        (P.test_param_cache_refresh_rule, ()),
        (P.test_seeding_hand_example, ()),
        (P.test_kmedoids_fixed_point_and_global_optimum_tiny, (6, 2, 0)),
        (P.test_kmedoids_fixed_point_and_global_optimum_tiny, (7, 3, 3)),
        (P.test_planted_clusters_recovered, ()),
        (P.test_rebalance_sizes_and_who_moves, ()),
        (P.test_base_is_the_mean_and_residuals_sum_to_zero, ()),
        (P.test_tsvd_error_is_the_eckart_young_tail, ()),
        (P.test_exact_when_residuals_have_rank_r, ()),
        (P.test_error_bound_at_rank_16_and_not_at_rank_4, ()),
    ]


def _ema_swapped(mu, X, idx, beta):
    return _orig["ema_centroids"](mu, X, idx, 1.0 - beta)


def _cos_one_norm(V):
    V = np.asarray(V, dtype=np.float64)
    n = np.sqrt((V * V).sum(axis=1))
    S = (V @ V.T) / (n[:, None] ** 2)
    np.fill_diagonal(S, 1.0)
    return S


def _fused_alpha_swapped(Sp, St, alpha, tau):
    return _orig["fused_distance"](Sp, St, 1.0 - alpha, tau)


def _fused_no_prune(Sp, St, alpha, tau):
    return _orig["fused_distance"](Sp, St, alpha, -10.0)


def _seed_farthest(D, G, u, max_iter=100):
    E = D.shape[0]
    med = [min(int(u[0] * E), E - 1)]
    while len(med) < G:
        d = [min(D[i, m] for m in med) for i in range(E)]
        med.append(int(np.argmax(d)))
    # one plain k-medoids pass from those seeds (assignment only)
    assign = np.array([int(np.argmin([D[i, m] for m in med])) for i in range(E)])
    if max_iter == 0:
        assign[:] = 0
    return assign, np.array(med)


def _medoid_max_cost(D, G, u, max_iter=100):
    assign, med = _orig["kmeanspp_medoids"](D, G, u, max_iter=0)
    E = D.shape[0]
    for _ in range(max_iter):
        for i in range(E):
            assign[i] = int(np.argmin([D[i, m] for m in med]))
        new = list(med)
        for g in range(G):
            mem = [i for i in range(E) if assign[i] == g]
            if mem:
                new[g] = mem[int(np.argmax([sum(D[a, b] for b in mem) for a in mem]))]
        if list(new) == list(med):
            break
        med = np.array(new)
    return assign, np.array(med)


def _rebalance_worst(assign, D, medoids, K):
    assign = np.array(assign)
    sizes = np.bincount(assign, minlength=len(medoids))
    while (sizes > K).any():
        cand = [(-(D[i, medoids[h]] - D[i, medoids[assign[i]]]), i, h) for i in range(assign.size)
                if sizes[assign[i]] > K for h in range(len(medoids)) if sizes[h] < K]
        _, i, h = min(cand)
        sizes[assign[i]] -= 1
        sizes[h] += 1
        assign[i] = h
    return assign


def _compress_uneven(Ws, members, r):
    base, A, B, err = _orig["compress_projection"](Ws, members, r)
    nA = np.linalg.norm(A, axis=1, keepdims=True)
    nA = np.where(nA > 0, nA, 1.0)
    return base, A * nA, B / nA, err


def _compress_short_rank(Ws, members, r):
    return _orig["compress_projection"](Ws, members, max(r - 1, 0))


def _compress_sum_base(Ws, members, r):
    G, K = members.shape
    Ws2 = [np.asarray(W, dtype=np.float64) for W in Ws]
    base, A, B, err = _orig["compress_projection"](Ws2, members, r)
    return base * K / (K + 1), A, B, err


def _cache_life_plus_one(vecs, cache, eps, life):
    return _orig["param_similarity_cached"](vecs, cache, eps, life + 1)


MUTATIONS = {
    "ema_weights_swapped": ("ema_centroids", _ema_swapped),
    "cosine_one_norm": ("cosine_matrix", _cos_one_norm),
    "alpha_swapped": ("fused_distance", _fused_alpha_swapped),
    "no_tau_pruning": ("fused_distance", _fused_no_prune),
    "farthest_point_seeding": ("kmeanspp_medoids", _seed_farthest),
    "medoid_with_max_cost": ("kmeanspp_medoids", _medoid_max_cost),
    "rebalance_worst_move": ("rebalance", _rebalance_worst),
    "uneven_singular_split": ("compress_projection", _compress_uneven),
    "rank_one_short": ("compress_projection", _compress_short_rank),
    "base_not_the_mean": ("compress_projection", _compress_sum_base),
    "cache_lives_one_longer": ("param_similarity_cached", _cache_life_plus_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(C, attr, fn)
    caught = [p.__name__ for p, args in _pins() if _fails(p, *args)]
    assert caught, f"no pin caught the planted mistake {name}"
