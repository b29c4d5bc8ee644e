"""Clustering and compression feeding the layer, end to end: dense
experts with a planted grouping are regrouped and compressed by the host
routine (include/moe_cluster.h), the result is created as an fp16-base /
INT4-residual layer, and its forward pass on the GPU is checked against
the oracle on the same compressed weights (1e-2 of max|y|), while the
compressed layer stays close to the dense experts it replaces."""
import dataclasses

import numpy as np
import pytest

from compressed_expert_ffn_amd import synth
from compressed_expert_ffn_amd.workloads import Workload
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, x_to_device, y_to_host, say
from tests.layers import make_parity_layer

pytestmark = pytest.mark.gpu


def test_recluster_compress_create_forward():
    import torch
    from compressed_expert_ffn_amd import _lib as L
    E, G, d, f, r = 16, 4, 256, 512, 16
    w = Workload("reclustered", 41, T=300, d=d, f=f, G=G, K=E // G, top_groups=1, top_experts=2, r=r,
                 act="swiglu", x_dtype="f16", base_dtype="f16", resid="int4_g32")
    dims = w.proj_dims()
    bank = synth.make_expert_bank(E, G, dims, rank=r, resid_scale=0.3, noise_scale=0.005, key=5)
    vecs = [np.concatenate([W[i].reshape(-1) for W in bank["W"]]) for i in range(E)]
    Xc, idx = synth.draw_group_tokens(bank["planted"], G, d, 2000, 2, key=5)
    cl = L.Cluster(E, G, d, vecs[0].size)
    cl.observe(Xc, idx)
    group_of, members, _, _ = cl.regroup(vecs, np.random.default_rng(3).random(G))
    cl.close()
    for g in range(G):
        assert len(set(bank["planted"][members[g]])) == 1
    base, A, B, errs = [], [], [], []
    for p in range(len(dims)):
        b, a, bb, e = L.compress_projection(bank["W"][p], members, r)
        base.append(b.astype(np.float16))
        A.append(a)
        B.append(bb)
        errs.append(e)
    say(f"[recluster] max relative Frobenius error {max(e.max() for e in errs):.4f}")
    assert max(e.max() for e in errs) <= 0.015

    wT, inputs, layer = make_parity_layer(w)
    inputs["base"], inputs["A"], inputs["B"] = base, A, B
    layer = dict(layer, base=base, A=A, B=B)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        st = lay.stats()
        assert st["stored_params"] == O.stored_params(G, E // G, r, dims)
        X = x_to_device(inputs["X"], w.x_dtype)
        Y = lay.forward(X)
        torch.cuda.synchronize()
        rt = O.route(layer)
        ref = O.forward(layer, routing=rt)
        err = rel_err(y_to_host(Y), ref)
        # the dense experts the compressed ones stand for, same routing
        Xf = inputs["X"].astype(np.float64)
        dense = np.zeros_like(ref)
        order = members.reshape(-1)            # stored index g*K + j -> original expert
        for t in range(wT.T):
            for s in range(wT.k):
                i = order[rt["idx"][t, s]]
                Ws = [bank["W"][p][i].astype(np.float64) for p in range(3)]
                dense[t] += rt["w"][t, s] * O.expert_ffn(Xf[t:t + 1], Ws, "swiglu")[0]
        dev = rel_err(ref, dense)
        say(f"[recluster] GPU vs oracle {err:.3e}; compressed vs dense experts {dev:.3e}")
        assert err <= TOL[w.x_dtype]
        # INT4 rounding of the residual factors dominates this deviation
        assert dev <= 0.1
    finally:
        lay.close()
