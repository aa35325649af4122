"""fp64 CPU oracle (test infrastructure only; see mla_oracle.py)."""
from . import mla_oracle  # noqa: F401
