"""CSA2 oracle (test infrastructure only; never used by the GPU library).  See oracle.py."""
from . import oracle  # noqa: F401
