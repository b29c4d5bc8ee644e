"""The five layer shapes this library is exercised on, plus their input recipe.

Each workload names the shape of one compressed-expert MoE FFN layer
(tokens T, model width d, hidden width f, E = G*K experts in G groups of K,
top_groups groups then top_experts experts per chosen group, residual rank r),
the storage dtypes, the activation, and the synthetic initialisation used in
place of trained weights.

The method is the one of "Breaking the MoE LLM Trilemma: Dynamic Expert
Clustering with Structured Compression" (papernotes.org ICML 2026 note on
arXiv 2510.02345): each expert i of group g is W_base^g + A_i B_i^T
(key design 2) and a token is routed to groups first, then to experts inside
the chosen groups (key design 3).  Base weights are stored FP16 and residual
factors FP16 or INT4 (key design 4).

Nothing here computes any part of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# storage dtype names
F32, F16, BF16 = "f32", "f16", "bf16"
RESID_NONE, RESID_F32, RESID_F16, RESID_INT4 = "none", "f32", "f16", "int4_g32"
ACT_GELU_TANH, ACT_SWIGLU = "gelu_tanh", "swiglu"


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    d: int
    f: int
    G: int
    K: int
    top_groups: int
    top_experts: int
    r: int
    act: str
    x_dtype: str
    base_dtype: str
    resid: str
    # expert-logit prior b_i = bias_scale * log(1/(i+1)); 0 disables it
    bias_scale: float = 0.0

    @property
    def E(self) -> int:
        return self.G * self.K

    @property
    def k(self) -> int:
        return self.top_groups * self.top_experts

    @property
    def P(self) -> int:
        """Projections per expert: gate, up, down (SwiGLU) or w1, w2 (GELU)."""
        return 3 if self.act == ACT_SWIGLU else 2

    @property
    def P_in(self) -> int:
        return self.P - 1

    def proj_dims(self):
        """(d_in, d_out) of each projection, in storage order."""
        if self.act == ACT_SWIGLU:
            return [(self.d, self.f), (self.d, self.f), (self.f, self.d)]
        return [(self.d, self.f), (self.f, self.d)]

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)

    # ---- algorithmic work (2 FLOP per multiply-add) -------------------------
    def algorithmic_flops(self) -> dict:
        """Work the method itself does for one forward pass.

        Base projections once per (token, chosen group); the rank-r residual
        only for the selected experts; the router scores all group logits and
        the expert logits of the chosen groups; the gate-weighted sum of the
        hidden activations is T*k*f multiply-adds.
        """
        T, d, f, r = self.T, self.d, self.f, self.r
        router = 2 * T * d * (self.G + (self.top_groups * self.K if self.K > 1 else 0))
        base = 2 * T * self.top_groups * self.P * d * f
        resid_in = 2 * T * self.k * r * self.P_in * (d + f)  # x.A and u.B^T
        resid_down = 2 * T * self.k * r * (f + d)  # h.A_down and v.B_down^T
        combine = 2 * T * self.k * f
        return dict(router=router, base=base, resid_in=resid_in,
                    resid_down=resid_down, combine=combine,
                    total=router + base + resid_in + resid_down + combine)


def _dtype_bytes(dt: str) -> int:
    return {F32: 4, F16: 2, BF16: 2}[dt]


def resid_bytes_per_factor(w: Workload, n_in: int) -> float:
    """Bytes one residual factor [n_in, r] takes in storage (INT4 with one
    fp16 scale per 32 entries along n_in, or plain floats)."""
    if w.resid == RESID_INT4:
        return n_in * w.r * 0.5 + (n_in // 32) * w.r * 2
    if w.resid == RESID_NONE:
        return 0.0
    return n_in * w.r * _dtype_bytes(w.resid)


# The five layers.  Shapes, dtypes and routing fan-out follow the workload
# list this library is measured on; layer 2 is the uncompressed flat top-2
# of 8 (the Llama-3 FFN shape d=4096, d_ff=14336 the MoE routing and
# engineering page gives in section 1.2), the degenerate case G=E, K=1, r=0.
WORKLOADS = [
    Workload("tiny_fp32_gelu", 0, T=64, d=64, f=128, G=2, K=4, top_groups=1,
             top_experts=2, r=4, act=ACT_GELU_TANH, x_dtype=F32,
             base_dtype=F32, resid=RESID_F32),
    Workload("compressed_fp16_swiglu", 1, T=2048, d=1024, f=2816, G=4, K=4,
             top_groups=1, top_experts=2, r=16, act=ACT_SWIGLU, x_dtype=F16,
             base_dtype=F16, resid=RESID_F16),
    Workload("flat_top2_of_8_bf16", 2, T=4096, d=4096, f=14336, G=8, K=1,
             top_groups=2, top_experts=1, r=0, act=ACT_SWIGLU, x_dtype=BF16,
             base_dtype=BF16, resid=RESID_NONE, bias_scale=0.5),
    Workload("fine_grained_int4", 3, T=16384, d=2048, f=1408, G=8, K=8,
             top_groups=1, top_experts=4, r=16, act=ACT_SWIGLU, x_dtype=BF16,
             base_dtype=F16, resid=RESID_INT4),
    Workload("decode_int4_zipf", 4, T=64, d=4096, f=1536, G=16, K=16,
             top_groups=2, top_experts=4, r=16, act=ACT_SWIGLU, x_dtype=F16,
             base_dtype=F16, resid=RESID_INT4, bias_scale=1.0),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]
