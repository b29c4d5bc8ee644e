"""Pins of the backward oracle: central finite differences of the forward
oracle (float64, the routing held by the 1e-3 margins) for every gradient,
on tiny layers of each kind; the factored identities against scalar loops;
the gradient of each gate weight against the expert output it scales."""
import math

import numpy as np
import pytest

from compressed_expert_ffn_amd import synth
from compressed_expert_ffn_amd.workloads import Workload
from oracle import backward_oracle as BO
from oracle import moe_oracle as O
from tests.layers import make_parity_layer


def tiny(G=2, K=3, kg=1, ke=2, r=2, d=6, f=8, act="swiglu", resid="f32", T=5, bias=0.4, seed=0):
    w = Workload("tiny_bwd", 95, T=T, d=d, f=f, G=G, K=K, top_groups=kg, top_experts=ke, r=r,
                 act=act, x_dtype="f32", base_dtype="f32", resid=resid, bias_scale=bias)
    _, inputs, layer = make_parity_layer(w, seed=seed)
    # float64 copies of every parameter, so finite differences see them exactly
    L = dict(layer)
    L["X"] = np.asarray(layer["X"], dtype=np.float64)
    for key in ("W_grp", "W_exp", "group_bias", "expert_bias"):
        if L.get(key) is not None:
            L[key] = np.asarray(L[key], dtype=np.float64)
    for key in ("base", "A", "B"):
        if L.get(key) is not None and L[key][0] is not None:
            L[key] = [np.asarray(a, dtype=np.float64) for a in L[key]]
    return w, L


def loss(L, dY):
    return float((O.forward(L) * dY).sum())


def fd_check(L, dY, get, grad, n=25, h=1e-6, seed=0):
    """Compare grad (array) with central differences of entries of the
    parameter get(L) (an array inside L, perturbed in place)."""
    P = get(L)
    rng = np.random.default_rng(seed)
    flat = P.reshape(-1)
    picks = rng.choice(flat.size, size=min(n, flat.size), replace=False)
    g = np.asarray(grad).reshape(-1)
    scale = max(np.abs(g).max(), 1e-12)
    for q in picks:
        old = flat[q]
        flat[q] = old + h
        lp = loss(L, dY)
        flat[q] = old - h
        lm = loss(L, dY)
        flat[q] = old
        num = (lp - lm) / (2 * h)
        # absolute floor: rounding of the O(1) loss divided by 2h
        assert abs(num - g[q]) <= 1e-6 * scale + 1e-8, (q, num, g[q])


CASES = [
    dict(act="swiglu", kg=1, ke=2, resid="f32", r=2),
    dict(act="swiglu", kg=2, ke=2, resid="f32", r=3, G=3),
    dict(act="gelu_tanh", kg=1, ke=2, resid="f32", r=2),
    dict(act="swiglu", kg=2, ke=1, K=1, G=4, resid="none", r=0),
    dict(act="gelu_tanh", kg=2, ke=2, G=3, K=2, resid="none", r=0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c['act']}-kg{c['kg']}-{c['resid']}" for c in CASES])
def test_every_gradient_matches_finite_differences(case):
    w, L = tiny(**case)
    dY = np.random.default_rng(1).standard_normal((w.T, w.d))
    g = BO.backward(L, dY)
    fd_check(L, dY, lambda L: L["X"], g["dX"], n=30)
    fd_check(L, dY, lambda L: L["W_grp"], g["dW_grp"])
    if L.get("group_bias") is not None:
        fd_check(L, dY, lambda L: L["group_bias"], g["d_group_bias"])
    if w.K > 1:
        fd_check(L, dY, lambda L: L["W_exp"], g["dW_exp"])
        if L.get("expert_bias") is not None:
            fd_check(L, dY, lambda L: L["expert_bias"], g["d_expert_bias"])
    else:
        assert not g["dW_exp"].any() and not g["d_expert_bias"].any()
    for p in range(len(L["base"])):
        fd_check(L, dY, lambda L, p=p: L["base"][p], g["dbase"][p])
        if w.r > 0:
            fd_check(L, dY, lambda L, p=p: L["A"][p], g["dA"][p])
            fd_check(L, dY, lambda L, p=p: L["B"][p], g["dB"][p])


def test_factored_identities_by_scalar_loops():
    """d/dA_i = dW~_i B_i and d/dB_i = dW~_i^T A_i, with dW~_i from the
    expert's own dense backward, entry by entry."""
    w, L = tiny(act="swiglu", kg=1, ke=1, r=2, d=4, f=5, T=4, K=2)
    dY = np.random.default_rng(2).standard_normal((w.T, w.d))
    g = BO.backward(L, dY)
    rt = O.route(L)
    for i in range(w.E):
        rows, slots = np.nonzero(rt["idx"] == i)
        if rows.size == 0:
            continue
        Ws = O.expert_weights(L, i)
        _, dWs, _ = BO.expert_backward(L["X"][rows], Ws, "swiglu", rt["w"][rows, slots][:, None] * dY[rows])
        for p in range(3):
            A, B, dW = L["A"][p][i], L["B"][p][i], dWs[p]
            for a in range(A.shape[0]):
                for q in range(w.r):
                    v = sum(dW[a, c] * B[c, q] for c in range(B.shape[0]))
                    assert math.isclose(g["dA"][p][i][a, q], v, rel_tol=1e-12, abs_tol=1e-14)
            for c in range(B.shape[0]):
                for q in range(w.r):
                    v = sum(dW[a, c] * A[a, q] for a in range(A.shape[0]))
                    assert math.isclose(g["dB"][p][i][c, q], v, rel_tol=1e-12, abs_tol=1e-14)


def test_gate_weight_gradient_is_the_scaled_expert_output():
    w, L = tiny(act="gelu_tanh", kg=2, ke=2, G=3, K=2, r=1)
    dY = np.random.default_rng(3).standard_normal((w.T, w.d))
    g = BO.backward(L, dY)
    rt = O.route(L)
    for t in range(w.T):
        for s in range(w.k):
            i = rt["idx"][t, s]
            y = O.expert_ffn(L["X"][t:t + 1], O.expert_weights(L, i), "gelu_tanh")[0]
            assert math.isclose(g["dw"][t, s], float(dY[t] @ y), rel_tol=1e-12, abs_tol=1e-14)
