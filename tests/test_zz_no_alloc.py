"""moe_forward_noalloc (the entry point whose workspace is the library's
static device array) against moe_forward on the same handle, through the C
ABI: two calls in a row, the second with fewer tokens, each bit for bit
equal to moe_forward and within the oracle tolerance."""
import dataclasses

import numpy as np
import pytest

from compressed_expert_ffn_amd.workloads import WORKLOADS
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, route_to_host, say, x_to_device, y_to_host
from tests.layers import make_parity_layer
from tests.test_gpu_parity import check_routing

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wi,T_big,T_small", [(1, 2048, 700), (4, 64, 5), (3, 900, 333), (0, 64, 17)])
def test_noalloc_matches_forward(wi, T_big, T_small):
    import torch
    from compressed_expert_ffn_amd import _lib as L
    w = WORKLOADS[wi].with_T(T_big)
    say(f"[noalloc] {w.name} T={T_big} then {T_small}")
    wT, inputs, layer = make_parity_layer(w)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        X = x_to_device(inputs["X"], w.x_dtype)
        rt = O.route(layer)
        ref = O.forward(layer, routing=rt)
        for T in (T_big, T_small):
            Xt = X[:T].contiguous()
            y_ref = lay.forward(Xt)
            Y = torch.full_like(y_ref, float("nan"))
            bufs = lay.route_buffers(T)
            lay.forward_noalloc(Xt, Y, route_bufs=bufs)
            torch.cuda.synchronize()
            sub = dict(idx=rt["idx"][:T], gidx=rt["gidx"][:T], w=rt["w"][:T])
            check_routing(route_to_host(bufs), sub, dataclasses.replace(wT, T=T), T)
            assert torch.equal(Y, y_ref), "noalloc output differs from moe_forward"
            err = rel_err(y_to_host(Y), ref[:T])
            say(f"[noalloc] {w.name} T={T}: equal to moe_forward, rel err {err:.3e}")
            assert err <= TOL[w.x_dtype]
    finally:
        lay.close()


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    import torch
    from compressed_expert_ffn_amd import _lib as L
    w = WORKLOADS[3]  # 16384 tokens need far more than the static array
    lay = L.Layer(L.config_from_workload(w, T_max=w.T),
                  __import__("compressed_expert_ffn_amd.synth", fromlist=["make_layer"]).make_layer(w.with_T(8)))
    try:
        X = torch.zeros((w.T, w.d), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty_like(X)
        with pytest.raises(L.MoEError) as ei:
            lay.forward_noalloc(X, Y)
        assert ei.value.code == L.MOE_ERR_INVALID_ARG and "scratch" in str(ei.value)
    finally:
        lay.close()
