"""fp64 CPU oracle (test infrastructure only; see sfx_oracle's header)."""
from . import sfx_oracle  # noqa: F401
