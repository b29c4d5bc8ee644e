"""CPU oracle for the backward pass of one compressed-expert MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the library may import, call or load
this module: only the tests and the benchmark's CPU-baseline leg use it.
Plain float64 NumPy: every expert is materialised densely (as the forward
oracle does), the gradient of each expert's dense weights is taken by the
chain rule of its own FFN, and then mapped onto the stored parameters
through W~_i = W_base^g + A_i B_i^T.

Sources:
[Trilemma] "Breaking the MoE LLM Trilemma: Dynamic Expert Clustering with
           Structured Compression" (papernotes.org note on arXiv
           2510.02345): the loss function / training strategy section
           trains the layer end to end (task loss of Eq. 1), and key design 2
           stores every expert as W_base^g + A_i B_i^T, so a training step
           needs d/dW_base^g = sum over the group's experts of dL/dW~_i,
           d/dA_i = dL/dW~_i B_i and d/dB_i = (dL/dW~_i)^T A_i.
[Routing]  "混合专家模型的路由机制与工程落地" (jiusizaji.com), section 1.2:
           y = sum_i G_i(x) E_i(x); the gate G is differentiable through the
           softmax over the selected logits, the top-k choice is not
           (the choice is held fixed, a zero-measure set aside).

Readings (listed in the design notes):
  B1 the loss is L = sum(dY * Y) for a given upstream gradient dY; the
     routing decisions are those of the forward pass;
  B2 INT4 residual factors are differentiated at their dequantised values
     (the quantiser itself has no gradient: straight-through);
  B3 the gate is w_{g,j} = p_g q_j (the forward oracle's reading), so
     dp_g = sum_j dw_{g,j} q_j, dq_j = dw_{g,j} p_g, and the softmax
     backward gives ds_g = p_g (dp_g - sum_g' p_g' dp_g') over the chosen
     groups (zero for the others) and likewise de_j over the chosen experts;
  B4 gradients reach the router weights, both biases and X through the
     logits; with K = 1 the in-group weight is the constant 1 and W_exp and
     the expert bias get no gradient.

Pins: central finite differences of the forward oracle on tiny float32
layers for every gradient (X, W_grp, W_exp, both biases, every base,
every A and B); the factored identities d/dA = dW~ B and d/dB = dW~^T A
against a scalar loop; zero residual and flat special cases.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O


def _dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _dgelu_tanh(z):
    c = np.sqrt(2.0 / np.pi)
    u = c * (z + 0.044715 * z ** 3)
    t = np.tanh(u)
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * z * z)


def softmax_backward(p, dp):
    """Gradient of the logits of p = softmax(z) given dL/dp."""
    return p * (dp - (p * dp).sum())


def factor_grads(dW, A, B):
    """Gradients of A and B in W~ = W_base + A B^T given dL/dW~."""
    return dW @ B, dW.T @ A


def expert_backward(x, Ws, act, g):
    """Gradients of sum(g * FFN(x)) for one expert with dense weights Ws:
    returns (dx, [dW_p], y)."""
    if act == O.SWIGLU:
        a, b = x @ Ws[0], x @ Ws[1]
        s = O.silu(a)
        h = s * b
        y = h @ Ws[2]
        dWd = h.T @ g
        dh = g @ Ws[2].T
        db = dh * s
        da = dh * b * _dsilu(a)
        dx = da @ Ws[0].T + db @ Ws[1].T
        return dx, [x.T @ da, x.T @ db, dWd], y
    if act == O.GELU_TANH:
        z = x @ Ws[0]
        h = O.gelu_tanh(z)
        y = h @ Ws[1]
        dW2 = h.T @ g
        dz = (g @ Ws[1].T) * _dgelu_tanh(z)
        return dz @ Ws[0].T, [x.T @ dz, dW2], y
    raise ValueError(act)


def backward(layer: dict, dY, routing: dict | None = None) -> dict:
    """All gradients of L = sum(dY * Y) (reading B1).  Returns a dict with
    dX [T, d], dbase (list over projections of [G, d_in, d_out]), dA / dB
    (lists of [E, d_in, r] / [E, d_out, r], or None when r == 0),
    dW_grp [d, G], dW_exp [G, d, K] (zeros when K == 1), d_group_bias [G],
    d_expert_bias [E], and dw [T, k] (the gradient of each gate weight)."""
    G, K, E, r = layer["G"], layer["K"], layer["G"] * layer["K"], layer["r"]
    kg, ke = layer["top_groups"], layer["top_experts"]
    X = O.as_f64(layer["X"], layer["x_dtype"])
    dY = np.asarray(dY, dtype=np.float64)
    T, d = X.shape
    rt = O.route(layer) if routing is None else routing
    idx, w = rt["idx"], rt["w"]
    P = len(layer["base"])
    dX = np.zeros_like(X)
    dbase = [np.zeros((G,) + np.asarray(b).shape[1:]) for b in layer["base"]]
    has_res = r > 0 and layer["resid"] != "none"
    dA = [np.zeros((E, np.asarray(b).shape[1], r)) for b in layer["base"]] if has_res else None
    dB = [np.zeros((E, np.asarray(b).shape[2], r)) for b in layer["base"]] if has_res else None
    dw = np.zeros_like(w)
    for i in range(E):
        rows, slots = np.nonzero(idx == i)
        if rows.size == 0:
            continue
        Ws = O.expert_weights(layer, i)
        wt = w[rows, slots][:, None]
        dx, dWs, y = expert_backward(X[rows], Ws, layer["act"], wt * dY[rows])
        dX[rows] += dx
        dw[rows, slots] = (dY[rows] * y).sum(axis=1)
        g = i // K
        for p in range(P):
            dbase[p][g] += dWs[p]
            if has_res:
                A = O.residual_factor_f64(layer["A"][p][i], layer["resid"])
                B = O.residual_factor_f64(layer["B"][p][i], layer["resid"])
                dA[p][i], dB[p][i] = factor_grads(dWs[p], A, B)

    # router: gate w = p_g q_j with softmaxes over the chosen logits (B3)
    Wg = np.asarray(layer["W_grp"], dtype=np.float64)
    dW_grp = np.zeros_like(Wg)
    dW_exp = np.zeros((G, d, K))
    dgb = np.zeros(G)
    deb = np.zeros(E)
    s = rt["group_logits"]
    gsel = rt["gidx"]
    for t in range(T):
        sc = s[t, gsel[t]]
        pg = np.exp(sc - sc.max())
        pg /= pg.sum()
        dp = np.zeros(kg)
        for a in range(kg):
            gg = gsel[t, a]
            slots = slice(a * ke, (a + 1) * ke)
            if K == 1:
                q = np.ones(1)
            else:
                el = rt["expert_logits"][t, a]
                jsel = idx[t, slots] - gg * K
                ec = el[jsel]
                q = np.exp(ec - ec.max())
                q /= q.sum()
                dq = dw[t, slots] * pg[a]
                de = softmax_backward(q, dq)
                We = np.asarray(layer["W_exp"][gg], dtype=np.float64)
                for b, j in enumerate(jsel):
                    dW_exp[gg][:, j] += X[t] * de[b]
                    deb[gg * K + j] += de[b]
                    dX[t] += de[b] * We[:, j]
            dp[a] = (dw[t, slots] * q).sum()
        ds = softmax_backward(pg, dp)
        for a in range(kg):
            gg = gsel[t, a]
            dW_grp[:, gg] += X[t] * ds[a]
            dgb[gg] += ds[a]
            dX[t] += ds[a] * Wg[:, gg]
    return dict(dX=dX, dbase=dbase, dA=dA, dB=dB, dW_grp=dW_grp, dW_exp=dW_exp,
                d_group_bias=dgb, d_expert_bias=deb, dw=dw)
