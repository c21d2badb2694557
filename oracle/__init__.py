"""fp64 CPU oracle (test infrastructure only; see attention.py's header)."""
from .attention import rope_frequencies, rope, attention, decode  # noqa: F401
