"""fp64 CPU oracle for the GDN layer (test infrastructure only; see gdn_oracle)."""
from . import gdn_oracle  # noqa: F401
