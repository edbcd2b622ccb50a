"""fp64 CPU oracle (test infrastructure; see kd_oracle's header for the import rule)."""
from . import kd_oracle  # noqa: F401
from . import brute  # noqa: F401
