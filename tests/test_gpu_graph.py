"""The forward pass captured in a HIP graph and replayed, through the C ABI.

moe_forward is enqueue-only and clears the counters a pass needs inside its
own kernels (no memset nodes), so a captured pass can be replayed.  Each
case captures one forward pass on a side stream, replays it several times
with eager work and synchronisations in between, and checks every replay
against the eager result bit for bit (the layer is deterministic), and the
eager result against the oracle within the usual bar.
"""
import numpy as np
import pytest

from compressed_expert_ffn_amd.workloads import WORKLOADS
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, say, x_to_device, y_to_host
from tests.layers import make_parity_layer

pytestmark = pytest.mark.gpu

CASES = [(0, 64), (1, 512), (3, 700), (4, 64), (2, 96)]


@pytest.mark.parametrize("wi,T", CASES, ids=[f"w{wi}-T{T}" for wi, T in CASES])
def test_graph_replays_equal_the_eager_pass(wi, T):
    import torch
    from compressed_expert_ffn_amd import _lib as L
    w = WORKLOADS[wi].with_T(T)
    wT, inputs, layer = make_parity_layer(w)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        X = x_to_device(inputs["X"], w.x_dtype)
        Y = torch.empty((T, w.d), dtype=X.dtype, device=X.device)
        lay.forward(X, Y)
        torch.cuda.synchronize()
        eager = Y.clone()
        err = rel_err(y_to_host(eager), O.forward(layer))
        assert err <= TOL[w.x_dtype]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            lay.forward(X, Y)  # one pass on the capture stream first
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward(X, Y)
        raw = {"f32": torch.int32}.get(w.x_dtype, torch.int16)
        for rep in range(4):
            Y.zero_()
            lay.forward(X, torch.empty_like(Y))  # an eager pass between replays
            (X.float() * 2.0).sum()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y.view(raw), eager.view(raw)), f"replay {rep} differs from the eager pass"
        say(f"[graph] {w.name} T={T}: 4 replays equal the eager pass, rel err {err:.3e}")
    finally:
        lay.close()


@pytest.mark.parametrize("wi,T", [(1, 512), (4, 64), (3, 300)], ids=["w1-T512", "w4-T64", "w3-T300"])
def test_graph_replays_of_the_no_allocation_entry(wi, T):
    """moe_forward_noalloc (the entry point for callers that cannot allocate,
    such as code under graph capture) captured and replayed: every replay
    equals moe_forward's eager result bit for bit."""
    import torch
    from compressed_expert_ffn_amd import _lib as L
    w = WORKLOADS[wi].with_T(T)
    wT, inputs, layer = make_parity_layer(w)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        X = x_to_device(inputs["X"], w.x_dtype)
        eager = lay.forward(X)
        torch.cuda.synchronize()
        Y = torch.empty_like(eager)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            lay.forward_noalloc(X, Y)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward_noalloc(X, Y)
        for rep in range(4):
            Y.zero_()
            lay.forward(X)  # an eager pass on the handle's own workspace between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"
        say(f"[graph noalloc] {w.name} T={T}: 4 replays equal moe_forward")
    finally:
        lay.close()
