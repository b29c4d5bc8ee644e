"""Distinct handles are independent: two layers forwarded at the same time
on two streams (default priority) give exactly what each gives alone, so no
state is shared between handles outside the documented static scratch of
moe_forward_noalloc."""
import pytest

from compressed_expert_ffn_amd.workloads import WORKLOADS
from tests.gpu_util import say, x_to_device
from tests.layers import make_parity_layer

pytestmark = pytest.mark.gpu


def test_two_handles_on_two_streams_match_their_sequential_results():
    import torch
    from compressed_expert_ffn_amd import _lib as L
    layers, xs = [], []
    try:
        for wi, T in ((1, 700), (4, 64)):
            w = WORKLOADS[wi].with_T(T)
            wT, inputs, _ = make_parity_layer(w)
            layers.append(L.Layer(L.config_from_workload(wT), inputs))
            xs.append(x_to_device(inputs["X"], w.x_dtype))
        alone = [lay.forward(x) for lay, x in zip(layers, xs)]
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        outs = [[], []]
        for _ in range(3):
            for i, (lay, x, s) in enumerate(zip(layers, xs, streams)):
                with torch.cuda.stream(s):
                    outs[i].append(lay.forward(x, stream=s))
        torch.cuda.synchronize()
        for i in range(2):
            for y in outs[i]:
                assert torch.equal(y.view(torch.int16), alone[i].view(torch.int16)), f"layer {i} differs"
        say("[streams] two handles on two streams: every pass equals its sequential result")
    finally:
        for lay in layers:
            lay.close()
