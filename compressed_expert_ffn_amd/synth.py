"""Seeded synthetic inputs for one compressed-expert MoE FFN layer.

This module draws random numbers and rounds them to storage dtypes.  It holds
none of the layer's arithmetic (no routing, no projections, no quantisation):
the oracle under ``oracle/`` and the HIP library both take its output as
input, and neither side's code is used here.

Recipe (one PCG64 substream per tensor slice, keyed by
``SeedSequence(seed, spawn_key=(workload, tensor_id, slice))``):

* X ~ N(0, 1), drawn as one stream in token-major order, so the first T'
  rows of a T-row draw equal a T'-row draw.  A token that must be redrawn
  (the parity tests do this when two router scores are closer than their
  margin) takes row ``t`` from the substream ``(workload, X, t, attempt)``.
* base weights ~ N(0, 1/d_in) (variance), one slice per (projection, group).
* residual factors A_i, B_i ~ N(0, 0.05^2) (std 0.05), one slice per
  (projection, expert).  For INT4 storage the fp32 draws are handed over
  unquantised; quantising them is the library's job (and the oracle's).
* router weights ~ N(0, 1/d) (variance): W_grp [d, G] and, when K > 1,
  W_exp [G, d, K].
* an optional expert-logit prior b_i = s*log(1/(i+1)); the group logit then
  gets c_g = log(sum_{j in g} exp(b_{gK+j})), the prior that a flat router
  with per-expert prior b would put on the whole group.  With K = 1 this is
  c_g = b_g.

fp32 draws are rounded to the storage dtype with round-to-nearest-even
(fp16 through numpy's cast; bf16 by rounding the upper 16 bits).  bf16 arrays
are carried as uint16 bit patterns because numpy has no bf16 type.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import (Workload, F32, F16, BF16, RESID_NONE, RESID_F16,
                        RESID_F32, RESID_INT4)

DEFAULT_SEED = 20261203

# tensor ids of the substreams
ID_X, ID_WGRP, ID_WEXP = 0, 1, 2
ID_BASE, ID_A, ID_B = 10, 20, 30

_POOL_THREADS = 8


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


# ---------------------------------------------------------------- dtypes ----
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    # keep NaN payloads quiet (inputs are finite; this is only hygiene)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a32: np.ndarray, dt: str) -> np.ndarray:
    if dt == F32:
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dt == F16:
        return a32.astype(np.float16)
    if dt == BF16:
        return f32_to_bf16_bits(a32)
    raise ValueError(dt)


def storage_to_f64(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact value of a stored array as float64."""
    if dt == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


# -------------------------------------------------------------- drawing -----
def draw_x(w: Workload, T: int | None = None, seed: int = DEFAULT_SEED) -> np.ndarray:
    T = w.T if T is None else T
    x = _rng(seed, w.index, ID_X).standard_normal((T, w.d), dtype=np.float32)
    return to_storage(x, w.x_dtype)


def redraw_tokens(w: Workload, X: np.ndarray, tokens, attempt: int,
                  seed: int = DEFAULT_SEED) -> None:
    """Replace rows ``tokens`` of X in place with fresh N(0,1) draws from
    each token's own substream for this attempt (attempt >= 1)."""
    assert attempt >= 1
    for t in tokens:
        row = _rng(seed, w.index, ID_X, int(t), int(attempt)).standard_normal(w.d, dtype=np.float32)
        X[int(t)] = to_storage(row, w.x_dtype)


def _normal_slices(seed, keys, shape, std, dt):
    def one(key):
        a = _rng(seed, *key).standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return to_storage(a, dt)
    with ThreadPoolExecutor(_POOL_THREADS) as ex:
        parts = list(ex.map(one, keys))
    return np.stack(parts)


def log_prior(w: Workload) -> np.ndarray:
    return np.array([w.bias_scale * math.log(1.0 / (i + 1)) for i in range(w.E)], dtype=np.float64)


def make_layer(w: Workload, seed: int = DEFAULT_SEED, T: int | None = None,
               zero_residual: bool = False) -> dict:
    """All inputs of one layer.

    Returns a dict with
      X           [T, d]        x storage dtype (uint16 bits for bf16)
      W_grp       [d, G]        float32
      W_exp       [G, d, K]     float32, or None when K == 1
      group_bias  [G]           float32, or None
      expert_bias [E]           float32, or None
      base        list over projections of [G, d_in, d_out], base dtype
      A, B        list over projections of [E, d_in, r] / [E, d_out, r]:
                  float32 for f32 and INT4 residuals (INT4 is quantised
                  downstream), float16 for f16; None when r == 0.
    """
    d, G, K, E, r = w.d, w.G, w.K, w.E, w.r
    out = dict(workload=w, seed=seed)
    out["X"] = draw_x(w, T, seed)
    out["W_grp"] = (_rng(seed, w.index, ID_WGRP).standard_normal((d, G), dtype=np.float32)
                    * np.float32(1.0 / math.sqrt(d)))
    if K > 1:
        out["W_exp"] = (_rng(seed, w.index, ID_WEXP).standard_normal((G, d, K), dtype=np.float32)
                        * np.float32(1.0 / math.sqrt(d)))
    else:
        out["W_exp"] = None
    if w.bias_scale != 0.0:
        b = log_prior(w)
        c = np.array([math.log(sum(math.exp(b[g * K + j]) for j in range(K))) for g in range(G)])
        out["expert_bias"] = b.astype(np.float32) if K > 1 else None
        out["group_bias"] = c.astype(np.float32)
    else:
        out["expert_bias"] = None
        out["group_bias"] = None

    base, A, B = [], [], []
    for p, (din, dout) in enumerate(w.proj_dims()):
        base.append(_normal_slices(seed, [(w.index, ID_BASE + p, g) for g in range(G)],
                                   (din, dout), 1.0 / math.sqrt(din), w.base_dtype))
        if r == 0 or w.resid == RESID_NONE:
            A.append(None)
            B.append(None)
            continue
        rdt = {RESID_F32: F32, RESID_INT4: F32, RESID_F16: F16}[w.resid]
        if zero_residual:
            A.append(np.zeros((E, din, r), dtype=np.float16 if rdt == F16 else np.float32))
            B.append(np.zeros((E, dout, r), dtype=np.float16 if rdt == F16 else np.float32))
            continue
        A.append(_normal_slices(seed, [(w.index, ID_A + p, e) for e in range(E)], (din, r), 0.05, rdt))
        B.append(_normal_slices(seed, [(w.index, ID_B + p, e) for e in range(E)], (dout, r), 0.05, rdt))
    out["base"], out["A"], out["B"] = base, A, B
    return out


# ------------------------------------------------- dense expert banks ----
def make_expert_bank(E: int, G: int, proj_dims, rank: int, resid_scale: float = 0.3,
                     noise_scale: float = 0.005, seed: int = DEFAULT_SEED, key: int = 0) -> dict:
    """Dense experts with a planted group structure, standing in for the
    trained experts a clustering pass would see (no trained weights here).

    Expert i belongs to planted group c_i (E / G experts per group, in a
    seeded random order of the indices).  Per projection of shape
    (d_in, d_out): W_i = C_c + s_r U_c M_i V_c^T + s_n N_i, with the group
    centre C_c, the group's rank-``rank`` subspaces U_c [d_in, rank] and
    V_c [d_out, rank], the expert's mixing matrix M_i [rank, rank] and the
    noise N_i all drawn N(0, 1); C is scaled to variance 1/d_in per entry,
    the subspace part to about ``resid_scale`` and the noise to about
    ``noise_scale`` of C's Frobenius norm.

    Returns W (list over projections of float32 [E, d_in, d_out]) and
    planted (int [E]).
    """
    rng = _rng(seed, 900 + key)
    planted = rng.permutation(np.repeat(np.arange(G), E // G))
    Ws = []
    for p, (din, dout) in enumerate(proj_dims):
        r = _rng(seed, 900 + key, p)
        sd = 1.0 / math.sqrt(din)
        C = r.standard_normal((G, din, dout)) * sd
        U = r.standard_normal((G, din, rank))
        V = r.standard_normal((G, dout, rank))
        M = r.standard_normal((E, rank, rank))
        N = r.standard_normal((E, din, dout))
        s_r = resid_scale * sd / rank if rank else 0.0
        s_n = noise_scale * sd
        W = np.empty((E, din, dout))
        for i in range(E):
            c = planted[i]
            W[i] = C[c] + s_r * (U[c] @ M[i] @ V[c].T) + s_n * N[i]
        Ws.append(W.astype(np.float32))
    return dict(W=Ws, planted=planted)


def draw_group_tokens(planted, G: int, d: int, T: int, k: int, spread: float = 0.5,
                      seed: int = DEFAULT_SEED, key: int = 0):
    """Tokens and a routing that sends each token to k experts of one
    planted group: x = g_c + spread * n for a random group c (g_c a random
    direction per group, n ~ N(0, 1)).  Returns X float32 [T, d] and idx
    int32 [T, k]."""
    rng = _rng(seed, 950 + key)
    dirs = rng.standard_normal((G, d))
    c = rng.integers(0, G, size=T)
    X = dirs[c] + spread * rng.standard_normal((T, d))
    members = [np.nonzero(np.asarray(planted) == g)[0] for g in range(G)]
    idx = np.stack([rng.choice(members[ci], size=k, replace=False) for ci in c])
    return X.astype(np.float32), idx.astype(np.int32)
