"""MI355X (gfx950) ring-attention per-device hot path.

The computation lives in the HIP library ``libra.so`` (C ABI: include/ra.h);
this package only loads it and marshals torch tensors into its calls.
"""
from .api import (  # noqa: F401
    LAYOUTS, CuSeqlens, KernelTimes, block_attn_bwd, block_attn_fwd, bwd_preprocess, cast_f32_to_bf16,
    gathered_bwd, gathered_fwd, gathered_workspace_bytes, kernel_timing, layout_positions, layout_posmap,
    lse_merge, noalloc_scratch_bytes, posmap, ring_bwd, ring_bwd_noalloc, ring_fwd, ring_workspace_bytes,
)
from ._lib import RAError, lib  # noqa: F401
from .functional import (  # noqa: F401
    gathered_attn_func, gathered_share_attn, llama3_attn_varlen_func, ring_attn_func, ring_attn_kvpacked_func,
    ring_attn_qkvpacked_func, ring_attn_varlen_func,
)
