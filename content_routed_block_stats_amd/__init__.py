"""MI355X-native hot path of Subquadratic Sparse Attention (content-routed block statistics).

The work happens in libssa_mi355x.so (hand-written gfx950 HIP kernels behind a
C ABI, include/ssa.h).  This package is its build script and a thin ctypes
binding whose functions carry the C entry points' names.
"""
from .binding import (  # noqa: F401
    SSAError,
    SSAParams,
    lib,
    make_params,
    ssa_block_stats,
    ssa_decode_step,
    ssa_decode_step_noalloc,
    ssa_group_stats,
    ssa_probe_hbm_read,
    ssa_probe_mfma_bf16,
    ssa_route_hier,
    ssa_route_hier_prefill,
    ssa_route_hier_prefill_workspace_size,
    ssa_route_tempered,
    ssa_route_tiles,
    ssa_route_topk,
    ssa_sparse_attn_bwd,
    ssa_sparse_attn_fwd,
    ssa_tile_attn_fwd,
    ssa_workspace_size,
    status_string,
)
