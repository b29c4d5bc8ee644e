"""The C ABI without a GPU: the library loads, exports every function
include/moe.h declares, and its host-side validation and bookkeeping agree
with the oracle's parameter count."""
import ctypes as C
import os
import re
import subprocess

import pytest

from compressed_expert_ffn_amd import _lib as L
from compressed_expert_ffn_amd.workloads import WORKLOADS
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    return names


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_create", "moe_route", "moe_forward", "moe_destroy"):
        assert n in names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = sorted(n for n in names if n not in exported)
    assert not missing, missing
    for n in names:
        assert hasattr(L.lib, n)


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_config_stats_match_oracle_count(w):
    st = L.config_stats(L.config_from_workload(w))
    assert st["stored_params"] == O.stored_params(w.G, w.K, w.r, w.proj_dims())
    assert st["dense_equiv_params"] == sum(w.E * di * do for di, do in w.proj_dims())
    assert st["stored_bytes"] > 0


def test_config_stats_compression_ratio_of_page_example():
    # d = 4096, K = 8, r = 16, one square projection per group: CR = 128/17
    cfg = L.make_config(1, 4096, 4096, 1, 8, 1, 2, 16, "gelu_tanh", "f16", "f16", "f16")
    st = L.config_stats(cfg)
    # two projections (d x f and f x d), both square here
    assert st["dense_equiv_params"] / st["stored_params"] == pytest.approx(128 / 17, rel=1e-12)


BAD = [
    (dict(top_groups=3, G=2), L.MOE_ERR_INVALID_ARG, "top_groups"),
    (dict(top_experts=5, K=4), L.MOE_ERR_INVALID_ARG, "top_experts"),
    (dict(r=0), L.MOE_ERR_INVALID_ARG, "r == 0"),
    (dict(d=100), L.MOE_ERR_UNSUPPORTED, "multiples of 64"),
    (dict(r=32), L.MOE_ERR_UNSUPPORTED, "r >"),
    (dict(x_dtype="f16", base_dtype="bf16", resid="int4_g32"), L.MOE_ERR_UNSUPPORTED, "dtype pair"),
    (dict(resid="f16", base_dtype="f32", x_dtype="f32"), L.MOE_ERR_UNSUPPORTED, "F16 residual"),
    (dict(T_max=-1), L.MOE_ERR_INVALID_ARG, "positive"),
]


@pytest.mark.parametrize("change,code,msg", BAD)
def test_invalid_configs_are_rejected_before_any_device_work(change, code, msg):
    base = dict(T_max=8, d=64, f=128, G=2, K=4, top_groups=1, top_experts=2, r=4,
                act="swiglu", x_dtype="f16", base_dtype="f16", resid="f16")
    base.update(change)
    cfg = L.make_config(**base)
    st = L.moe_stats()
    rc = L.lib.moe_config_stats(C.byref(cfg), C.byref(st))
    assert rc == code
    assert msg in L.lib.moe_last_error().decode()
    h = C.c_void_p()
    w = L.moe_weights()
    assert L.lib.moe_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == code
    assert not h.value


def test_null_arguments():
    assert L.lib.moe_destroy(None) == L.MOE_OK
    assert L.lib.moe_forward(None, None, 0, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert L.lib.moe_route(None, None, 0, None, None) == L.MOE_ERR_INVALID_ARG
    assert L.lib.moe_config_stats(None, None) == L.MOE_ERR_INVALID_ARG
    assert L.lib.moe_profile_begin(None, 1, -1) == L.MOE_ERR_INVALID_ARG
    cfg = L.make_config(8, 64, 128, 2, 4, 1, 2, 4, "swiglu", "f16", "f16", "f16")
    h = C.c_void_p()
    assert L.lib.moe_create(C.byref(cfg), None, None, C.byref(h)) == L.MOE_ERR_INVALID_ARG


def test_handle_calls_reject_null():
    assert L.lib.moe_stats(None, None) == L.MOE_ERR_INVALID_ARG
    assert L.lib.moe_debug_dequant(None, 0, 0, 0, None) == L.MOE_ERR_INVALID_ARG
    assert L.lib.moe_debug_q(None, 0, 0, 0, None, None) == L.MOE_ERR_INVALID_ARG


def test_weights_struct_matches_header_layout():
    # nine pointers of weights, then the on_device flag
    assert L.moe_weights.on_device.offset == 4 * 8 + 9 * 8
