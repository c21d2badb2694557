"""fp64 CPU oracle (test infrastructure only; see attention.py's header)."""
from .attention import (rope_frequencies, rope, attention, decode, round_bf16,  # noqa: F401
                        append_to_cache, attention_with_cache, decode_paged,
                        append_to_cache_paged, gather_pages,
                        RopeScaling, rope_angles)
