"""HiLS attention test oracle (test infrastructure only; see hils_oracle.py)."""
from . import hils_oracle  # noqa: F401
