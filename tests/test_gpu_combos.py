"""Every dtype, residual and activation combination the library accepts,
on small layers, against the CPU oracle through the C ABI; plus the
boundary's secondary calls (device-pointer weights, per-handle statistics,
the INT4 read-back calls, routing outputs of an empty batch).

Bars as in the workload parity tests: routing bit-exact, gate weights to
1e-6 * max(1, sqrt(d / 1024)), outputs to 1e-5 (fp32) or 1e-2 (fp16 / bf16)
of max|y_ref|; INT4 codes, scales and dequantised values bit-exact.
"""
import numpy as np
import pytest

from compressed_expert_ffn_amd.workloads import Workload
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, route_to_host, say, x_to_device, y_to_host
from tests.layers import make_parity_layer
from tests.test_gpu_parity import check_routing

pytestmark = pytest.mark.gpu


def _lib():
    from compressed_expert_ffn_amd import _lib as L
    return L


# (act, x dtype, base dtype, residual, r, groups x experts, kg, ke, T)
COMBOS = [
    ("swiglu", "bf16", "bf16", "int4_g32", 16, (4, 4), 1, 2, 300),
    ("swiglu", "bf16", "f16", "f16", 16, (4, 4), 2, 2, 257),
    ("gelu_tanh", "f16", "f16", "f16", 16, (2, 8), 1, 3, 200),
    ("gelu_tanh", "f16", "f16", "int4_g32", 16, (4, 4), 1, 2, 190),
    ("gelu_tanh", "bf16", "bf16", "int4_g32", 8, (4, 4), 2, 1, 131),
    ("gelu_tanh", "bf16", "f16", "int4_g32", 16, (3, 4), 1, 2, 99),
    ("swiglu", "f16", "f16", "none", 0, (4, 4), 1, 2, 222),
    ("swiglu", "bf16", "f16", "none", 0, (8, 1), 2, 1, 150),
    ("gelu_tanh", "f32", "f32", "none", 0, (4, 2), 1, 2, 77),
    ("swiglu", "f32", "f32", "f32", 12, (2, 4), 1, 2, 65),
    ("gelu_tanh", "bf16", "bf16", "none", 0, (6, 1), 3, 1, 140),
]


def combo_workload(act, xd, bd, resid, r, gk, kg, ke, T, d=256, f=512):
    G, K = gk
    return Workload(f"combo_{act}_{xd}_{bd}_{resid}", 40, T=T, d=d, f=f, G=G, K=K, top_groups=kg,
                    top_experts=ke, r=r, act=act, x_dtype=xd, base_dtype=bd, resid=resid,
                    bias_scale=0.5)


@pytest.mark.parametrize("combo", COMBOS, ids=["-".join(map(str, c[:5])) for c in COMBOS])
def test_combination_matches_oracle(combo):
    import torch
    L = _lib()
    w = combo_workload(*combo)
    say(f"[combo] {w.name} r={w.r} G={w.G} K={w.K} kg={w.top_groups} ke={w.top_experts} T={w.T}")
    wT, inputs, layer = make_parity_layer(w)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        X = x_to_device(inputs["X"], w.x_dtype)
        rt = O.route(layer)
        bufs = lay.route_buffers(wT.T)
        Y = lay.forward(X, route_bufs=bufs)
        torch.cuda.synchronize()
        check_routing(route_to_host(bufs), rt, wT, wT.T)
        err = rel_err(y_to_host(Y), O.forward(layer, routing=rt))
        say(f"[combo] {w.name}: rel err {err:.3e}")
        assert err <= TOL[w.x_dtype]
        if w.resid == "int4_g32":
            # the INT4 decode of every MFMA type, bit for bit
            for p in range(w.P):
                for which, src in ((0, inputs["A"]), (1, inputs["B"])):
                    for e in (0, w.E - 1):
                        q_ref, s_ref = O.quantize_int4_g32(src[p][e])
                        q, sc = lay.debug_q(p, which, e)
                        vals = lay.debug_dequant(p, which, e)
                        assert np.array_equal(q, q_ref), (p, which, e)
                        assert np.array_equal(sc, s_ref.view(np.uint16)), (p, which, e)
                        assert np.array_equal(vals.view(np.uint32),
                                              O.dequantize_int4_g32(q_ref, s_ref).view(np.uint32))
        # the backward pass of the same combination against the backward
        # oracle (dX and every weight gradient, bars as in the backward tests)
        from compressed_expert_ffn_amd import synth
        from oracle import backward_oracle as BO
        dYs = synth.to_storage(np.random.default_rng(23).standard_normal((wT.T, w.d)).astype(np.float32),
                               w.x_dtype)
        g = lay.backward(X, x_to_device(dYs, w.x_dtype))
        torch.cuda.synchronize()
        gref = BO.backward(layer, synth.storage_to_f64(dYs, w.x_dtype))
        btol = 1e-5 if w.x_dtype == "f32" else 2e-2
        pairs = [("dX", g["dX"].float(), gref["dX"])]
        pairs += [(f"dbase{p}", g["dbase"][p], gref["dbase"][p]) for p in range(w.P)]
        if w.r:
            pairs += [(f"dA{p}", g["dA"][p], gref["dA"][p]) for p in range(w.P)]
            pairs += [(f"dB{p}", g["dB"][p], gref["dB"][p]) for p in range(w.P)]
        for name, got, ref_g in pairs:
            e = rel_err(got.cpu().numpy(), ref_g)
            assert e <= btol, (name, e)
    finally:
        lay.close()


def test_device_pointer_weights_give_the_same_layer():
    import torch
    L = _lib()
    w = combo_workload("swiglu", "f16", "f16", "int4_g32", 16, (4, 4), 1, 2, 180)
    wT, inputs, layer = make_parity_layer(w)
    a = L.Layer(L.config_from_workload(wT), inputs)
    b = L.Layer(L.config_from_workload(wT), inputs, on_device=True)
    try:
        X = x_to_device(inputs["X"], w.x_dtype)
        ya, yb = a.forward(X), b.forward(X)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        assert rel_err(y_to_host(yb), O.forward(layer)) <= TOL[w.x_dtype]
        assert a.stats() == b.stats() == L.config_stats(L.config_from_workload(wT))
        assert b.stats()["stored_params"] == O.stored_params(w.G, w.K, w.r, w.proj_dims())
    finally:
        a.close()
        b.close()


def test_forward_with_no_tokens_publishes_empty_routing():
    import torch
    L = _lib()
    w = combo_workload("swiglu", "f16", "f16", "f16", 16, (4, 4), 2, 2, 40)
    wT, inputs, _ = make_parity_layer(w)
    lay = L.Layer(L.config_from_workload(wT), inputs)
    try:
        bufs = lay.route_buffers(0)
        for key in ("counts", "offsets", "gcounts", "goffsets"):
            bufs[key].fill_(-7)
        X = x_to_device(inputs["X"][:0], w.x_dtype)
        Y = lay.forward(X, route_bufs=bufs)
        torch.cuda.synchronize()
        assert Y.shape == (0, w.d)
        got = route_to_host(bufs)
        for key in ("counts", "offsets", "gcounts", "goffsets"):
            assert (got[key] == 0).all(), key
    finally:
        lay.close()
