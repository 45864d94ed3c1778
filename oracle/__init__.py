"""fp64 CPU oracle (test infrastructure only; see paged_ref.py)."""
from . import paged_ref

__all__ = ["paged_ref"]
