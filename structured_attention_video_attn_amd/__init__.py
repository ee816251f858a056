"""Monarch-factored 3D video attention (MonarchRT forward hot path) for MI355X / gfx950.

The computation lives in ``libmonarch_attn.so`` (hand-written HIP kernels behind
the C ABI of ``include/monarch_attn.h``); this package is its ctypes binding.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    MA_BF16,
    MA_F32,
    MonarchAttnError,
    dense_attn_fwd,
    load_library,
    ma_bwd_workspace_bytes,
    ma_stage_l_fwd,
    ma_stage_r_fwd,
    ma_workspace_bytes,
    monarch_attn_bwd,
    monarch_attn_causal_fwd,
    monarch_attn_chunk_fwd,
    monarch_attn_fwd,
    monarch_attn_fwd_noalloc,
    ma_noalloc_scratch_bytes,
    monarch_attn_tiled_fwd,
)
