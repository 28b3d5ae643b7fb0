"""CPU oracle for the MLA path (test infrastructure only; see mla_oracle)."""
from . import mla_oracle  # noqa: F401
