"""Compressed-expert MoE FFN layer (shared group base + rank-r residual,
two-level routing) for AMD Instinct MI355X (gfx950)."""
from . import workloads  # noqa: F401
