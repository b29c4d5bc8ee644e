"""Helpers for the GPU parity tests: moving seeded host arrays to the device
and comparing the library's results with the oracle's."""
import sys

import numpy as np

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def x_to_device(X: np.ndarray, dt: str):
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(X)).cuda()


def y_to_host(Y) -> np.ndarray:
    return Y.float().cpu().numpy().astype(np.float64)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(y - ref).max() / (den if den > 0 else 1.0))


def route_to_host(bufs: dict) -> dict:
    return {k: v.cpu().numpy() for k, v in bufs.items()}
