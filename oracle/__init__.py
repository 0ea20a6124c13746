"""Float64 CPU oracle (test infrastructure only; see ring_attention.py)."""
from .ring_attention import (  # noqa: F401
    LAYOUTS, attention, attention_backward, count_pairs, default_scale,
    layout_positions, lse_merge, merge_all, ring_backward, ring_forward,
    ring_sources, seq_ids, to_ring, visible,
)
