"""MI355X-native hybrid mesh + 3D Gaussian tile rasterizer.

The compute path is libgm.so (hand-written HIP for gfx950, C ABI in include/gm.h).
``_lib`` is its ctypes binding (same names as the C calls); ``pipeline`` allocates
device buffers with torch and calls the entry points in order.
"""
from . import _lib
from ._lib import (GM_GRAD, GM_REC, GM_TILE, GmCamera, GmError, GmLight, GmMesh, gm_bin_triangles,
                   gm_build_mipmaps, gm_composite_hybrid_bwd, gm_composite_hybrid_fwd,
                   gm_composite_hybrid_fwd_shaded, gm_project_gaussians, gm_mesh_bwd, gm_project_gaussians_bwd,
                   gm_project_gaussians_multi, gm_raster_zbuffer, gm_shade_surface, gm_sort_depth,
                   gm_sort_tile_keys, gm_sort_tiles, gm_version)

__all__ = ["_lib", "GM_GRAD", "GM_REC", "GM_TILE", "GmCamera", "GmError", "GmLight", "GmMesh",
           "gm_bin_triangles", "gm_build_mipmaps", "gm_composite_hybrid_bwd", "gm_composite_hybrid_fwd",
           "gm_composite_hybrid_fwd_shaded", "gm_mesh_bwd", "gm_project_gaussians", "gm_project_gaussians_bwd",
           "gm_project_gaussians_multi", "gm_raster_zbuffer", "gm_shade_surface",
           "gm_sort_depth", "gm_sort_tile_keys", "gm_sort_tiles", "gm_version"]
