"""Block-sparse self-attention for video DiTs on AMD Instinct MI355X (gfx950).

Tokens of a T x H x W latent grid are grouped into 64-token tiles (static
4x4x4 or dynamic per-region shapes); every query tile keeps the top-k key tiles
by pooled score and attends exactly to them (plus an optional dense prefix).
All of it runs in the hand-written HIP kernels of ``libbsa.so`` behind the C
ABI in ``include/bsa.h``; this package is the thin Python binding.
"""
from ._lib import (EXPORTS, LIB_PATH, MASK_SPATIAL, MASK_TEMPORAL, MAX_CSR_HEADS, MAX_VIDEO_TILES, PERM_BUILD,
                   PERM_GATHER, PERM_GATHER_KF, PERM_GATHER_KF_POOL, PERM_GATHER_POOL, PERM_GATHER_VF, PERM_POOL,
                   PERM_SCATTER, PERM_TILED_TO_KF, PERM_TILED_TO_VF, TILE_DYNAMIC, TILE_STATIC, TILE_STATIC_PADDED, BsaError, Desc,
                   lib)
from .api import (DENSE_BELOW_TOKENS, BlockSparseAttention, attention, backward, backward_csr, backward_csr_workspace_size, backward_stats,
                  backward_stats_offset, backward_workspace_size,
                  csr_entries, forward, forward_csr, forward_csr_raster, forward_noalloc, forward_raster, forward_stats, forward_stats_offset, gather, gather_kf,
                  gather_kf_pool, gather_pool, gather_vf, keep_for_call, keep_tiles_for, make_desc, permute_build, plan, plan_csr, plan_structured,
                  pool, pooled_views, scatter, select, select_csr, structured_entries, tiled_to_kf, tiled_to_vf, video_slots,
                  workspace_size)

lib()  # fail at import if the HIP library was not built

__all__ = ["attention", "DENSE_BELOW_TOKENS", "keep_for_call", "keep_tiles_for", "BlockSparseAttention", "BsaError", "Desc", "EXPORTS", "LIB_PATH", "MAX_CSR_HEADS", "MAX_VIDEO_TILES",
           "backward", "backward_csr", "backward_csr_workspace_size", "backward_stats", "backward_stats_offset",
           "backward_workspace_size", "csr_entries",
           "forward", "forward_csr", "forward_csr_raster", "forward_noalloc", "forward_raster", "forward_stats", "forward_stats_offset", "plan_csr", "plan_structured",
           "structured_entries", "MASK_SPATIAL", "MASK_TEMPORAL", "gather", "gather_kf", "gather_kf_pool",
           "gather_pool", "gather_vf", "make_desc", "permute_build", "plan", "pool", "pooled_views", "scatter", "select", "select_csr",
           "tiled_to_kf", "tiled_to_vf", "workspace_size", "PERM_BUILD", "PERM_GATHER", "PERM_GATHER_KF",
           "PERM_GATHER_KF_POOL", "PERM_GATHER_POOL", "PERM_GATHER_VF", "PERM_POOL", "PERM_SCATTER", "PERM_TILED_TO_KF",
           "PERM_TILED_TO_VF", "TILE_STATIC", "TILE_DYNAMIC", "TILE_STATIC_PADDED", "video_slots"]
