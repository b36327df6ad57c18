"""Float64 CPU oracle (test infrastructure only; see am_oracle's module docstring)."""
from . import am_oracle  # noqa: F401
