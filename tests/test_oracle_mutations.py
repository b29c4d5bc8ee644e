"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that at least one pin in test_oracle.py catches each of them."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import test_oracle as P


def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _pins():
    return [
        (P.test_scalar_bruteforce_tiny, ("swiglu", 2)),
        (P.test_scalar_bruteforce_tiny, ("gelu_tanh", 1)),
        (P.test_materialized_equals_factored, ()),
        (P.test_activations_against_library_forms, ()),
        (P.test_exact_ties_go_to_lower_index, ()),
        (P.test_single_group_weight_is_softmax_over_selected_experts, ()),
        (P.test_router_matches_repeated_argmax, (4, 4, 2, 2, 1.0)),
        (P.test_zero_residual_reduces_to_group_base, (2,)),
        (P.test_flat_case_matches_independent_flat_moe, ()),
        (P.test_int4_layer_uses_dequantised_factors, ()),
        (P.test_int4_nearest_code_range_and_exact_dequant, ()),
        (P.test_int4_half_even_ties_hand_example, ()),
        (P.test_bf16_decode_hand_values, ()),
        (P.test_scalar_bruteforce_16bit_storage, ("bf16", "bf16")),
    ]


MUTATIONS = {
    "residual_dropped": ("materialize", lambda b, A, B: b + 0.0 * (A @ B.T)),
    "residual_sign": ("materialize", lambda b, A, B: b - A @ B.T),
    "residual_transposed": ("materialize", lambda b, A, B: b + (A @ B.T).T.reshape(b.shape)),
    "silu_sign": ("silu", lambda z: z / (1.0 + np.exp(z))),
    "gelu_constant": ("gelu_tanh", lambda z: 0.5 * z * (1.0 + np.tanh(np.sqrt(2 / np.pi) * (z + 0.44715 * z ** 3)))),
    "ties_to_higher_index": ("_desc_order", lambda s: (s.shape[-1] - 1) - np.argsort(-s[..., ::-1], axis=-1, kind="stable")),
    "softmax_without_max_shift_and_wrong_norm": ("_softmax", lambda v: np.exp(v) / np.exp(v).sum(axis=-1, keepdims=True) ** 0.5),
    "int4_round_half_away": ("quantize_int4_g32", None),
    "bf16_scaled": ("as_f64", None),
    "bf16_truncated_to_fp16_grid": ("as_f64", None),
}

_as_f64 = O.as_f64


def _bf16_scaled(a, dtype):
    v = _as_f64(a, dtype)
    return v * 1.01 if dtype == "bf16" else v


def _bf16_via_fp16(a, dtype):
    v = _as_f64(a, dtype)
    return v.astype(np.float16).astype(np.float64) if dtype == "bf16" else v


def _int4_half_away(M):
    M = np.asarray(M, dtype=np.float32)
    n, r = M.shape
    blocks = M.reshape(n // 32, 32, r)
    scale = (np.abs(blocks).max(axis=1) / np.float32(7.0)).astype(np.float16)
    s = scale.astype(np.float32)[:, None, :]
    safe = np.where(s > 0, s, np.float32(1.0))
    v = blocks / safe
    q = np.sign(v) * np.floor(np.abs(v) + 0.5)
    q = np.where(s > 0, np.clip(q, -8, 7), 0).astype(np.int8)
    return q.reshape(n, r), scale


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    if name == "int4_round_half_away":
        fn = _int4_half_away
    elif name == "bf16_scaled":
        fn = _bf16_scaled
    elif name == "bf16_truncated_to_fp16_grid":
        fn = _bf16_via_fp16
    monkeypatch.setattr(O, attr, fn)
    caught = [p.__name__ for p, args in _pins() if _fails(p, *args)]
    assert caught, f"no pin caught the planted mistake {name}"
