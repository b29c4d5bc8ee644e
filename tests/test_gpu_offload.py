"""Idle-group offload (moe_offload_enable / moe_forward_offload) through
the C ABI: with groups swapped between pinned host memory and a few device
slots, every batch's output equals moe_forward's on a resident copy of the
same layer bit for bit (and the oracle within tolerance), including
batches that need more groups than slots (several GEMM passes, the copies
of the next pass overlapping the current one)."""
import numpy as np
import pytest

from compressed_expert_ffn_amd import synth
from compressed_expert_ffn_amd.workloads import WORKLOADS
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, say, x_to_device, y_to_host
from tests.layers import make_parity_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wi,T,slots", [(4, 64, 4), (4, 64, 16), (1, 300, 1), (1, 300, 2), (3, 500, 3), (0, 64, 1),
                                        (2, 96, 3)])
def test_offload_matches_resident_layer(wi, T, slots):
    import torch
    from compressed_expert_ffn_amd import _lib as L
    w = WORKLOADS[wi].with_T(T)
    if wi == 2:
        import dataclasses
        w = dataclasses.replace(w, d=512, f=1024)
    say(f"[offload] {w.name} T={T} slots={slots}")
    wT, inputs, layer = make_parity_layer(w)
    ref_lay = L.Layer(L.config_from_workload(wT), inputs)
    off = L.Layer(L.config_from_workload(wT), inputs)
    try:
        off.offload_enable(slots)
        with pytest.raises(L.MoEError) as ei:
            off.forward(x_to_device(inputs["X"], w.x_dtype))
        assert ei.value.code == L.MOE_ERR_UNSUPPORTED
        for b in range(3):
            X = inputs["X"] if b == 0 else synth.draw_x(w, T=T, seed=1000 + b)
            Xd = x_to_device(X, w.x_dtype)
            bufs = off.route_buffers(T)
            y_off = off.forward_offload(Xd, route_bufs=bufs)
            y_ref = ref_lay.forward(Xd)
            torch.cuda.synchronize()
            assert torch.equal(y_off, y_ref), f"batch {b}: offloaded output differs"
            if b == 0:
                err = rel_err(y_to_host(y_off), O.forward(layer))
                assert err <= TOL[w.x_dtype]
                gc = bufs["gcounts"].cpu().numpy()
                assert gc.sum() == T * w.top_groups
        st = off.offload_stats()
        say(f"[offload] stats {st}")
        assert st["calls"] == 3 and st["group_loads"] + st["group_hits"] >= 3
        assert st["passes"] >= 3
    finally:
        ref_lay.close()
        off.close()
