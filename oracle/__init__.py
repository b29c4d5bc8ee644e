"""CPU oracle (test infrastructure only; the library never uses it)."""
from . import moe_oracle  # noqa: F401
