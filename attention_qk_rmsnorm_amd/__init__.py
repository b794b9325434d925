"""MI355X (gfx950) sink-aware grouped-query attention, forward and backward.

Per-head RMSNorm and NeoX RoPE on Q and K, then causal or sliding-window
attention over packed variable-length documents (THD, cu_seqlens) with one
learned fp32 sink logit per query head, in hand-written HIP kernels behind the
C ABI of include/sink_attn.h.  This package is the thin Python binding.
"""
from .binding import (NOALLOC_SCRATCH_BYTES, SINK_ATTN_BF16, SINK_ATTN_F16, SINK_ATTN_F32,
                      SINK_ATTN_TILE_AUTO, SINK_ATTN_TILE_NARROW, SINK_ATTN_TILE_WIDE,
                      SINK_ATTN_TILE_WIDE_EXACT, BwdCall, Call, SinkAttnDesc, SinkAttnError,
                      bwd_workspace_bytes, header_functions, library_path, load_library,
                      make_desc, mask_to_seqlens, sink_attn_bwd, sink_attn_bwd_bshd,
                      sink_attn_bwd_workspace_bytes, sink_attn_fwd, sink_attn_fwd_bshd,
                      sink_attn_fwd_noalloc, sink_attn_prologue, sink_attn_tile_config,
                      sink_attn_workspace_bytes, status_string, tile_config, workspace_bytes)

__all__ = [
    "NOALLOC_SCRATCH_BYTES", "SINK_ATTN_BF16", "SINK_ATTN_F16", "SINK_ATTN_F32",
    "SINK_ATTN_TILE_AUTO", "SINK_ATTN_TILE_NARROW", "SINK_ATTN_TILE_WIDE",
    "SINK_ATTN_TILE_WIDE_EXACT", "BwdCall", "Call", "SinkAttnDesc", "SinkAttnError",
    "bwd_workspace_bytes", "header_functions", "library_path", "load_library", "make_desc",
    "mask_to_seqlens", "sink_attn_bwd", "sink_attn_bwd_bshd", "sink_attn_bwd_workspace_bytes",
    "sink_attn_fwd", "sink_attn_fwd_bshd", "sink_attn_fwd_noalloc", "sink_attn_prologue",
    "sink_attn_tile_config", "sink_attn_workspace_bytes", "status_string", "tile_config",
    "workspace_bytes"
]
