"""CPU oracle (test infrastructure only; see nvfp4_oracle's module docstring)."""
from . import nvfp4_oracle  # noqa: F401
