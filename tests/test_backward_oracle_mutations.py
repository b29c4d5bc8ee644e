"""Plant plausible mistakes in the backward oracle (on the CPU, via
monkeypatch) and check that a pin in test_backward_oracle.py catches each."""
import numpy as np
import pytest

from oracle import backward_oracle as BO
from tests import test_backward_oracle as P

_orig_eb = BO.expert_backward
_orig_fg = BO.factor_grads


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _pins():
    return [(P.test_every_gradient_matches_finite_differences, (c,)) for c in P.CASES] + [
        (P.test_factored_identities_by_scalar_loops, ()),
        (P.test_gate_weight_gradient_is_the_scaled_expert_output, ()),
    ]


def _dsilu_no_product_rule(z):
    return 1.0 / (1.0 + np.exp(-z))


def _dgelu_no_inner(z):
    c = np.sqrt(2.0 / np.pi)
    t = np.tanh(c * (z + 0.044715 * z ** 3))
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c


def _eb_no_up_path(x, Ws, act, g):
    dx, dWs, y = _orig_eb(x, Ws, act, g)
    if act == "swiglu":
        a, b = x @ Ws[0], x @ Ws[1]
        dh = g @ Ws[2].T
        da = dh * b * BO._dsilu(a)
        dx = da @ Ws[0].T
    return dx, dWs, y


def _softmax_bwd_no_centering(p, dp):
    return p * dp


def _factor_grads_forget_b(dW, A, B):
    dA, dB = _orig_fg(dW, A, B)
    return dA, np.zeros_like(dB)


def _factor_grads_swapped_roles(dW, A, B):
    return dW @ B * 0.5 + 0.5 * (dW @ B), (dW.T @ A) * (1.0 + 1e-3)


MUTATIONS = {
    "dsilu_without_product_rule": ("_dsilu", _dsilu_no_product_rule),
    "dgelu_without_inner_derivative": ("_dgelu_tanh", _dgelu_no_inner),
    "dx_without_up_path": ("expert_backward", _eb_no_up_path),
    "softmax_backward_not_centred": ("softmax_backward", _softmax_bwd_no_centering),
    "dB_forgotten": ("factor_grads", _factor_grads_forget_b),
    "dB_scaled": ("factor_grads", _factor_grads_swapped_roles),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(BO, attr, fn)
    caught = [p.__name__ for p, args in _pins() if _fails(p, *args)]
    assert caught, f"no pin caught the planted mistake {name}"
