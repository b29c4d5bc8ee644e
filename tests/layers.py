"""Test helpers: build the oracle's layer description from a workload and
the seeded generator's arrays, and redraw tokens whose router scores are
closer than the parity margin."""
import dataclasses

import numpy as np

from compressed_expert_ffn_amd import synth
from compressed_expert_ffn_amd.workloads import Workload
from oracle import moe_oracle as O

MARGIN = 1e-3


def oracle_layer(w: Workload, inputs: dict) -> dict:
    fields = dict(G=w.G, K=w.K, top_groups=w.top_groups, top_experts=w.top_experts,
                  r=w.r, d=w.d, f=w.f, act=w.act, x_dtype=w.x_dtype,
                  base_dtype=w.base_dtype, resid=w.resid)
    return O.layer_from(fields, inputs)


def margin_violations(layer: dict, margin: float = MARGIN, tokens=None) -> np.ndarray:
    """Tokens whose consecutive order statistics 1..k+1 are closer than
    ``margin`` at either routing level (float64 logits of the stored X)."""
    rt = O.route(layer, tokens)
    kg, ke, K = layer["top_groups"], layer["top_experts"], layer["K"]
    bad = np.zeros(rt["group_logits"].shape[0], dtype=bool)

    def check(v, k):
        s = -np.sort(-v, axis=1)
        n = min(k + 1, v.shape[1])
        if n < 2:
            return np.zeros(v.shape[0], dtype=bool)
        gaps = s[:, :n - 1] - s[:, 1:n]
        return (gaps < margin).any(axis=1)

    bad |= check(rt["group_logits"], kg)
    if K > 1:
        for a in range(kg):
            bad |= check(rt["expert_logits"][:, a, :], ke)
    t = np.nonzero(bad)[0]
    return t if tokens is None else np.asarray(tokens)[t]


def make_parity_layer(w: Workload, T=None, seed=synth.DEFAULT_SEED, zero_residual=False,
                      max_attempts=20):
    """Seeded inputs with every token's routing margins above MARGIN."""
    inputs = synth.make_layer(w, seed=seed, T=T, zero_residual=zero_residual)
    wT = dataclasses.replace(w, T=inputs["X"].shape[0])
    layer = oracle_layer(wT, inputs)
    for attempt in range(1, max_attempts + 1):
        bad = margin_violations(layer)
        if bad.size == 0:
            break
        synth.redraw_tokens(w, inputs["X"], bad, attempt, seed)
        layer["X"] = inputs["X"]
    else:
        raise RuntimeError("could not meet routing margins")
    return wT, inputs, layer
