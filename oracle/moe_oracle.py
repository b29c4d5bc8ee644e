"""CPU oracle for one compressed-expert MoE FFN layer, forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the library may import, call or load
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg use it.  It is deliberately slow and plain: float64 NumPy,
the definitions written out, a library matmul/sort as the only building
blocks, every expert materialised densely.

Sources (cited by page title and section):

[Trilemma]  "Breaking the MoE LLM Trilemma: Dynamic Expert Clustering with
            Structured Compression" (papernotes.org note on arXiv 2510.02345).
            Key design 2: expert i of group g is W~_i = W_base^g + A_i B_i^T,
            A_i in R^{d_in x r}, B_i in R^{d_out x r}; the compression ratio
            CR = K d_in d_out / (d_in d_out + K r (d_in + d_out)).
            Key design 3: two-level routing, a token first picks groups, then
            experts inside the chosen groups.
            Key design 4: FP16 base, INT4 residual factors.
[Routing]   "混合专家模型的路由机制与工程落地" (MoE routing mechanisms and
            engineering, jiusizaji.com).  Section 1.2: the FFN block and the
            MoE sum y = sum_i G_i(x) E_i(x), G non-zero on the top-k only.
            Section 2.2: a per-expert additive routing bias b_i.
            Section 3.1: the router is computed in FP32.
[Whitepaper] rkmt.cn "MoE whitepaper", top-2 routing snippet: take the top-k
            logits, then a softmax over just those.

Readings where the pages leave a step open (each is also listed in the
design notes):
  * row vectors: x W~ = x W_base + (x A) B^T (the page's W~ x does not
    type-check against the stated shapes of A and B);
  * gate weight of expert j of chosen group g: softmax over the chosen group
    logits times softmax over the chosen expert logits of that group; with
    one chosen group this is the softmax over the selected logits of the
    whitepaper snippet, with K = 1 it is flat top-k;
  * ordering: descending score, ties to the lower index; the decision is
    taken on the FP32 value of each logit (the router runs in FP32), the
    logit itself and the softmax are evaluated in float64;
  * no outer activation around the FFN; SwiGLU h = SiLU(x W~_gate) * (x W~_up),
    y = h W~_down; GELU in its tanh form;
  * INT4: symmetric, q in [-8, 7], one fp16 scale per 32 consecutive entries
    along the factor's first axis (d_in for A, d_out for B) and per rank
    column; scale = fp16(amax / 7) with FP32 division, q = round-half-even
    of v / scale in FP32, clamped; amax == 0 (or a scale that rounds to 0)
    gives scale 0 and q 0; the dequantised value q * scale is exact in FP32;
  * dropless: every selected (token, expert) pair is computed; the
    permutation lists, expert by expert, the tokens in ascending order.

Pins (tests under tests/ that do not need a GPU): gate weights sum to 1 per
token; exact ties resolve to the lower index; an independent repeated-argmax
router agrees; the permutation equals a stable argsort of the token-major
assignment list; counts sum to T*k; INT4 codes are the nearest integer to
v/scale (half-even on exact ties), the amax entry maps to +-7 and the
dequantised value is exact; the materialised expert equals the factored
evaluation; zero residual factors reduce the layer to the group base FFN;
G = E, K = 1, r = 0 equals an independent flat top-k MoE; a scalar-loop
brute force agrees on tiny shapes; the CR formula at the page's example
parameters is 128/17.
"""
from __future__ import annotations

import math

import numpy as np

SWIGLU, GELU_TANH = "swiglu", "gelu_tanh"


# ------------------------------------------------------------ decoding ----
def as_f64(a, dtype: str) -> np.ndarray:
    """Exact value of a stored array: 'f32', 'f16', or 'bf16' (uint16 bits)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


# ---------------------------------------------------------------- INT4 ----
def quantize_int4_g32(M) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric INT4 with one fp16 scale per 32 rows of each column.

    M: float32 [n, r], n a multiple of 32.  Returns (q int8 [n, r] in
    [-8, 7], scale float16 [n // 32, r]).  [Trilemma] key design 4 stores the
    residual factors in INT4; the block size, the symmetric range and the
    rounding are the readings stated in the module header.
    """
    M = np.asarray(M, dtype=np.float32)
    n, r = M.shape
    if n % 32:
        raise ValueError("INT4 blocks need a multiple of 32 rows")
    blocks = M.reshape(n // 32, 32, r)
    amax = np.abs(blocks).max(axis=1)                       # float32
    scale = (amax / np.float32(7.0)).astype(np.float16)     # FP32 divide, then RNE to fp16
    s = scale.astype(np.float32)[:, None, :]
    nonzero = s > 0
    safe = np.where(nonzero, s, np.float32(1.0))
    q = np.rint(blocks / safe)                              # FP32 divide, half-even
    q = np.where(nonzero, np.clip(q, -8, 7), 0).astype(np.int8)
    return q.reshape(n, r), scale


def dequantize_int4_g32(q, scale) -> np.ndarray:
    """float32 value q * scale of each entry (exact: 4-bit times 11-bit)."""
    q = np.asarray(q, dtype=np.int8)
    n, r = q.shape
    s = np.asarray(scale, dtype=np.float16).astype(np.float32)
    return (q.reshape(n // 32, 32, r).astype(np.float32) * s[:, None, :]).reshape(n, r)


def residual_factor_f64(M, resid: str) -> np.ndarray:
    """The value of one residual factor as the layer uses it."""
    if resid == "int4_g32":
        q, s = quantize_int4_g32(M)
        return dequantize_int4_g32(q, s).astype(np.float64)
    if resid in ("f32", "f16"):
        return np.asarray(M).astype(np.float64)
    raise ValueError(resid)


# ------------------------------------------------------------- routing ----
def _desc_order(scores32: np.ndarray) -> np.ndarray:
    """Indices by descending score, equal scores by ascending index."""
    return np.argsort(-scores32, axis=-1, kind="stable")


def _softmax(v: np.ndarray) -> np.ndarray:
    m = v.max(axis=-1, keepdims=True)
    e = np.exp(v - m)
    return e / e.sum(axis=-1, keepdims=True)


def route(layer: dict, tokens=None) -> dict:
    """Two-level routing of [Trilemma] key design 3.

    Level 1 scores the G groups, s_g = x . W_grp[:, g] + c_g, and keeps the
    top_groups best.  Level 2 scores, inside each chosen group g, its K
    experts, e_j = x . W_exp[g][:, j] + b_{gK+j}, and keeps the top_experts
    best.  Biases are the additive per-expert routing bias of [Routing]
    section 2.2.  Gate weight of (g, j): softmax over the chosen s times
    softmax over the chosen e of g.  With K == 1 the only expert of a
    chosen group is taken with in-group weight 1.

    Returns gidx [T, kg], idx [T, k] (global expert ids g*K + j, group rank
    major), w [T, k] float64, plus the float64 logits.
    """
    G, K = layer["G"], layer["K"]
    kg, ke = layer["top_groups"], layer["top_experts"]
    X = as_f64(layer["X"], layer["x_dtype"])
    if tokens is not None:
        X = X[np.asarray(tokens)]
    T = X.shape[0]
    s = X @ np.asarray(layer["W_grp"], dtype=np.float64)
    if layer.get("group_bias") is not None:
        s = s + np.asarray(layer["group_bias"], dtype=np.float64)
    gsel = _desc_order(s.astype(np.float32))[:, :kg]
    p = _softmax(np.take_along_axis(s, gsel, axis=1))

    k = kg * ke
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    elog = np.zeros((T, kg, K), dtype=np.float64)
    for a in range(kg):
        g = gsel[:, a]
        if K == 1:
            jsel = np.zeros((T, 1), dtype=np.int64)
            q = np.ones((T, 1))
            elog[:, a, 0] = 0.0
        else:
            e = np.zeros((T, K))
            for gg in range(G):
                rows = np.nonzero(g == gg)[0]
                if rows.size == 0:
                    continue
                e[rows] = X[rows] @ np.asarray(layer["W_exp"][gg], dtype=np.float64)
                if layer.get("expert_bias") is not None:
                    e[rows] += np.asarray(layer["expert_bias"][gg * K:(gg + 1) * K], dtype=np.float64)
            elog[:, a, :] = e
            jsel = _desc_order(e.astype(np.float32))[:, :ke]
            q = _softmax(np.take_along_axis(e, jsel, axis=1))
        idx[:, a * ke:(a + 1) * ke] = (g[:, None] * K + jsel).astype(np.int32)
        w[:, a * ke:(a + 1) * ke] = p[:, a:a + 1] * q
    return dict(gidx=gsel.astype(np.int32), idx=idx, w=w, group_logits=s, expert_logits=elog)


def permutation(assign: np.ndarray, n_bins: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Counts, offsets (exclusive scan, n_bins + 1 entries) and the token list
    grouped bin by bin, tokens ascending within a bin (dropless dispatch).

    assign: int [T, m], the bins token t goes to (distinct within a row).
    """
    assign = np.asarray(assign)
    counts = np.zeros(n_bins, dtype=np.int64)
    perm = []
    for b in range(n_bins):
        toks = np.nonzero((assign == b).any(axis=1))[0]
        counts[b] = toks.size
        perm.append(toks)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.concatenate(perm) if perm else np.zeros(0, dtype=np.int64)
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)


# ------------------------------------------------------------- experts ----
def materialize(base_g: np.ndarray, A_i: np.ndarray, B_i: np.ndarray) -> np.ndarray:
    """W~_i = W_base^g + A_i B_i^T, [d_in, d_out], float64 ([Trilemma] key design 2)."""
    return base_g + A_i @ B_i.T


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def expert_ffn(x: np.ndarray, Ws: list, act: str) -> np.ndarray:
    """One expert's FFN on row vectors x [n, d] ([Routing] section 1.2 with
    the activation of the workload; no outer activation)."""
    if act == SWIGLU:
        return (silu(x @ Ws[0]) * (x @ Ws[1])) @ Ws[2]
    if act == GELU_TANH:
        return gelu_tanh(x @ Ws[0]) @ Ws[1]
    raise ValueError(act)


def expert_weights(layer: dict, i: int) -> list:
    """Materialised float64 projections of expert i."""
    K, r = layer["K"], layer["r"]
    g = i // K
    Ws = []
    for p in range(len(layer["base"])):
        bg = as_f64(layer["base"][p][g], layer["base_dtype"])
        if r == 0 or layer["resid"] == "none":
            Ws.append(bg)
            continue
        A = residual_factor_f64(layer["A"][p][i], layer["resid"])
        B = residual_factor_f64(layer["B"][p][i], layer["resid"])
        Ws.append(materialize(bg, A, B))
    return Ws


def forward(layer: dict, tokens=None, routing: dict | None = None) -> np.ndarray:
    """y_t = sum_i G_i(x_t) E_i(x_t) over the experts i ([Routing] section 1.2),
    with E_i the FFN of the materialised compressed expert W~_i and G the
    two-level gate above.  Experts are visited in index order, so each
    token's sum runs in that order.  Returns float64 [T or len(tokens), d].
    """
    X = as_f64(layer["X"], layer["x_dtype"])
    if tokens is not None:
        X = X[np.asarray(tokens)]
    if routing is None:
        routing = route(layer, tokens)
    idx, w = routing["idx"], routing["w"]
    Y = np.zeros((X.shape[0], layer["d"]), dtype=np.float64)
    E = layer["G"] * layer["K"]
    for i in range(E):
        rows, slots = np.nonzero(idx == i)
        if rows.size == 0:
            continue
        out = expert_ffn(X[rows], expert_weights(layer, i), layer["act"])
        Y[rows] += w[rows, slots][:, None] * out
    return Y


# ---------------------------------------------------------- bookkeeping ----
def stored_params(G: int, K: int, r: int, proj_dims) -> int:
    """Parameters stored: a base per group and projection, rank-r factors per
    expert and projection ([Trilemma] key design 2)."""
    return sum(G * di * do + G * K * r * (di + do) for di, do in proj_dims)


def compression_ratio(d_in: int, d_out: int, K: int, r: int) -> float:
    """CR = K d_in d_out / (d_in d_out + K r (d_in + d_out)) ([Trilemma] key design 2)."""
    return K * d_in * d_out / (d_in * d_out + K * r * (d_in + d_out))


def layer_from(workload_fields: dict, inputs: dict) -> dict:
    """Assemble the oracle's layer description from plain fields and arrays."""
    L = dict(workload_fields)
    for key in ("X", "W_grp", "W_exp", "group_bias", "expert_bias", "base", "A", "B"):
        L[key] = inputs[key]
    return L
