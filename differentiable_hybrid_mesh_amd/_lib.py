"""ctypes binding of libgm.so (include/gm.h): same names, argument marshalling only.

Every array argument is a torch tensor on the GPU (or None); the binding passes its
data pointer.  No computation happens here.  Importing this module does not touch
the GPU; ``lib()`` raises if libgm.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgm.so")

GM_TILE = 16
GM_REC = 16
GM_GRAD = 13
GM_OK, GM_ERR_ARG, GM_ERR_HIP = 0, -1, -3


class GmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gm status {status}: {msg}")
        self.status = status


class GmCamera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("R", C.c_float * 9), ("t", C.c_float * 3),
                ("near_z", C.c_float)]


class GmLight(C.Structure):
    _fields_ = [("pos", C.c_float * 3), ("ambient", C.c_float * 3), ("diffuse", C.c_float * 3),
                ("specular", C.c_float * 3), ("shininess", C.c_float)]


class GmMesh(C.Structure):
    _fields_ = [("V", C.c_int32), ("F", C.c_int32), ("Vt", C.c_int32), ("tex_size", C.c_int32),
                ("verts", C.c_void_p), ("faces", C.c_void_p), ("face_mask", C.c_void_p),
                ("vcolor", C.c_void_p), ("vnormal", C.c_void_p), ("uv", C.c_void_p),
                ("faces_uv", C.c_void_p), ("mips", C.c_void_p)]


EXPORTS = ["gm_bin_triangles_ws", "gm_bin_triangles", "gm_raster_zbuffer_ws", "gm_raster_zbuffer",
           "gm_project_gaussians",
           "gm_project_gaussians_multi",
           "gm_sort_tile_keys_ws", "gm_sort_tile_keys", "gm_sort_depth", "gm_sort_tiles", "gm_composite_hybrid_fwd",
           "gm_composite_hybrid_bwd", "gm_composite_hybrid_bwd_ws", "gm_project_gaussians_bwd", "gm_mesh_bwd", "gm_mipmaps_floats",
           "gm_build_mipmaps", "gm_last_error", "gm_version", "gm_edge_adjacency_ws", "gm_edge_adjacency",
           "gm_antialias", "gm_composite_hybrid_fwd_aa", "gm_composite_hybrid_bwd_aa", "gm_antialias_bwd_ws",
           "gm_antialias_bwd", "gm_vscreen_bwd", "gm_shade_surface", "gm_composite_hybrid_fwd_shaded"]

_lib = None


def lib():
    """Load libgm.so; raise a clear error when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python __graft_entry__.py build` "
                          "(or differentiable_hybrid_mesh_amd/build.py) first")
    L = C.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    cam, mesh, light = C.POINTER(GmCamera), C.POINTER(GmMesh), C.POINTER(GmLight)
    L.gm_bin_triangles_ws.argtypes = [I32, I32, I32, I32]
    L.gm_bin_triangles_ws.restype = SZ
    L.gm_bin_triangles.argtypes = [cam, mesh, P, P, P, I64, P, P, SZ, P]
    L.gm_raster_zbuffer_ws.argtypes = [I32, I32]
    L.gm_raster_zbuffer_ws.restype = SZ
    L.gm_raster_zbuffer.argtypes = [cam, mesh, P, P, P, P, P, P, P, SZ, P]
    L.gm_project_gaussians.argtypes = [cam, I32, P, P, P, P, P, I32, P, P]
    L.gm_project_gaussians_multi.argtypes = [cam, I32, I32, P, P, P, P, P, I32, P, P]
    L.gm_sort_tile_keys_ws.argtypes = [I32, I64, I32, I32]
    L.gm_sort_tile_keys_ws.restype = SZ
    L.gm_sort_tile_keys.argtypes = [cam, I32, P, P, F32, P, P, I64, P, P, SZ, P]
    L.gm_sort_depth.argtypes = [cam, I32, P, I64, P, SZ, P]
    L.gm_sort_tiles.argtypes = [cam, I32, P, P, F32, P, P, I64, P, P, SZ, P]
    L.gm_composite_hybrid_fwd.argtypes = [cam, P, P, P, P, P, mesh, P, light, P, F32, P, P, P, P, P, P, P]
    L.gm_shade_surface.argtypes = [cam, P, mesh, P, light, P, P, P]
    L.gm_composite_hybrid_fwd_shaded.argtypes = [cam, P, P, P, P, P, F32, P, P, P, P, P, P, P]
    L.gm_composite_hybrid_bwd.argtypes = [cam, I32, P, P, P, P, P, F32, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.gm_composite_hybrid_bwd_ws.argtypes = [I32, I32]
    L.gm_composite_hybrid_bwd_ws.restype = SZ
    L.gm_project_gaussians_bwd.argtypes = [cam, I32, P, P, P, P, P, I32, P, P, P, P, P, P, P, P, P, P]
    L.gm_mesh_bwd.argtypes = [cam, mesh, light, P, P, P, P, P, P, P, P, P, P]
    L.gm_edge_adjacency_ws.argtypes = [I32]
    L.gm_edge_adjacency_ws.restype = SZ
    L.gm_edge_adjacency.argtypes = [mesh, P, P, SZ, P]
    L.gm_antialias.argtypes = [cam, mesh, P, P, light, P, P, P, P, P, P, P]
    L.gm_composite_hybrid_fwd_aa.argtypes = [cam, P, P, P, P, P, F32, P, P, P, P, P]
    L.gm_composite_hybrid_bwd_aa.argtypes = [cam, I32, P, P, P, P, P, F32, P, P, P, P, P, P, P, SZ, P]
    L.gm_antialias_bwd_ws.argtypes = [I32, I32]
    L.gm_antialias_bwd_ws.restype = SZ
    L.gm_antialias_bwd.argtypes = [cam, mesh, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.gm_vscreen_bwd.argtypes = [cam, mesh, P, P, P]
    L.gm_mipmaps_floats.argtypes = [I32]
    L.gm_mipmaps_floats.restype = SZ
    L.gm_build_mipmaps.argtypes = [P, I32, P, P]
    L.gm_last_error.argtypes = []
    L.gm_last_error.restype = C.c_char_p
    L.gm_version.argtypes = []
    L.gm_version.restype = I32
    for name in EXPORTS:
        if not hasattr(L, name):
            raise ImportError(f"{LIB_PATH} does not export {name}")
    for name in ("gm_bin_triangles", "gm_raster_zbuffer", "gm_project_gaussians", "gm_project_gaussians_multi",
                 "gm_sort_tile_keys", "gm_sort_depth", "gm_sort_tiles",
                 "gm_composite_hybrid_fwd", "gm_composite_hybrid_bwd", "gm_project_gaussians_bwd",
                 "gm_mesh_bwd", "gm_build_mipmaps", "gm_edge_adjacency", "gm_antialias", "gm_composite_hybrid_fwd_aa",
                 "gm_composite_hybrid_bwd_aa", "gm_antialias_bwd", "gm_vscreen_bwd", "gm_shade_surface",
                 "gm_composite_hybrid_fwd_shaded"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def check(status: int):
    if status != GM_OK:
        raise GmError(status, lib().gm_last_error().decode(errors="replace"))
    return status


# ---------------------------------------------------------------------------
# the six calls and the auxiliary ones, same names as the C ABI
# ---------------------------------------------------------------------------

def gm_bin_triangles_ws(V, F, width, height) -> int:
    return lib().gm_bin_triangles_ws(V, F, width, height)


def gm_bin_triangles(cam, mesh, vscreen, tile_offsets, tile_tris, cap, n_pairs, ws, stream):
    """n_pairs: device int64 tensor that receives the pair count (asynchronously)."""
    check(lib().gm_bin_triangles(C.byref(cam), C.byref(mesh), ptr(vscreen), ptr(tile_offsets),
                                 ptr(tile_tris), int(cap), ptr(n_pairs), ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_raster_zbuffer_ws(width, height) -> int:
    return lib().gm_raster_zbuffer_ws(int(width), int(height))


def gm_raster_zbuffer(cam, mesh, vscreen, tile_offsets, tile_tris, face_id, depth, tile_dmax, ws, stream):
    check(lib().gm_raster_zbuffer(C.byref(cam), C.byref(mesh), ptr(vscreen), ptr(tile_offsets),
                                  ptr(tile_tris), ptr(face_id), ptr(depth), ptr(tile_dmax), ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_project_gaussians(cam, N, means, quats, scales, opacity, sh, sh_degree, rec, stream):
    check(lib().gm_project_gaussians(C.byref(cam), int(N), ptr(means), ptr(quats), ptr(scales),
                                     ptr(opacity), ptr(sh), int(sh_degree), ptr(rec), stream))


def gm_project_gaussians_multi(cams, N, means, quats, scales, opacity, sh, sh_degree, rec, stream):
    """cams: sequence of GmCamera; rec holds len(cams) * N records."""
    arr = (GmCamera * max(len(cams), 1))(*cams)
    check(lib().gm_project_gaussians_multi(arr, len(cams), int(N), ptr(means), ptr(quats), ptr(scales),
                                           ptr(opacity), ptr(sh), int(sh_degree), ptr(rec), stream))


def gm_sort_tile_keys_ws(N, cap, width, height) -> int:
    return lib().gm_sort_tile_keys_ws(int(N), int(cap), width, height)


def gm_sort_tile_keys(cam, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap, n_keys, ws, stream):
    """n_keys: device int64 tensor that receives the key count (asynchronously)."""
    check(lib().gm_sort_tile_keys(C.byref(cam), int(N), ptr(rec), ptr(tile_dmax), float(softness),
                                  ptr(tile_ranges), ptr(sorted_ids), int(cap), ptr(n_keys), ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_sort_depth(cam, N, rec, cap, ws, stream):
    """First half of gm_sort_tile_keys: the depth order, kept in ws for gm_sort_tiles."""
    check(lib().gm_sort_depth(C.byref(cam), int(N), ptr(rec), int(cap), ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_sort_tiles(cam, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap, n_keys, ws, stream):
    """Second half of gm_sort_tile_keys, ordered after gm_sort_depth on the same ws."""
    check(lib().gm_sort_tiles(C.byref(cam), int(N), ptr(rec), ptr(tile_dmax), float(softness),
                              ptr(tile_ranges), ptr(sorted_ids), int(cap), ptr(n_keys), ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), stream))


def _light_ref(light):
    return None if light is None else C.byref(light)


def gm_composite_hybrid_fwd(cam, rec, tile_ranges, sorted_ids, face_id, depth, mesh, vscreen, light, bg,
                            softness, out_rgb, out_depth, out_alpha, state_T, state_last, state_cm, stream):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    check(lib().gm_composite_hybrid_fwd(C.byref(cam), ptr(rec), ptr(tile_ranges), ptr(sorted_ids),
                                        ptr(face_id), ptr(depth), C.byref(mesh), ptr(vscreen),
                                        _light_ref(light), C.cast(bgv, C.c_void_p), float(softness),
                                        ptr(out_rgb), ptr(out_depth), ptr(out_alpha), ptr(state_T),
                                        ptr(state_last), ptr(state_cm), stream))


def gm_shade_surface(cam, face_id, mesh, vscreen, light, bg, state_cm, stream):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    check(lib().gm_shade_surface(C.byref(cam), ptr(face_id), C.byref(mesh), ptr(vscreen), _light_ref(light),
                                 C.cast(bgv, C.c_void_p), ptr(state_cm), stream))


def gm_composite_hybrid_fwd_shaded(cam, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_cm, out_rgb,
                                   out_depth, out_alpha, state_T, state_last, stream):
    check(lib().gm_composite_hybrid_fwd_shaded(C.byref(cam), ptr(rec), ptr(tile_ranges), ptr(sorted_ids),
                                               ptr(face_id), ptr(depth), float(softness), ptr(state_cm),
                                               ptr(out_rgb), ptr(out_depth), ptr(out_alpha), ptr(state_T),
                                               ptr(state_last), stream))


def gm_composite_hybrid_bwd_ws(width, height) -> int:
    return lib().gm_composite_hybrid_bwd_ws(int(width), int(height))


def gm_composite_hybrid_bwd(cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T, state_last,
                            state_cm, g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth, ws, stream):
    """ws: device scratch of gm_composite_hybrid_bwd_ws(width, height) bytes."""
    check(lib().gm_composite_hybrid_bwd(C.byref(cam), int(N), ptr(rec), ptr(tile_ranges), ptr(sorted_ids),
                                        ptr(face_id), ptr(depth), float(softness), ptr(state_T),
                                        ptr(state_last), ptr(state_cm), ptr(g_rgb), ptr(g_depth),
                                        ptr(g_alpha), ptr(g_rec), ptr(g_mesh_rgb), ptr(g_mesh_depth), ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_project_gaussians_bwd(cam, N, means, quats, scales, opacity, sh, sh_degree, rec, g_rec, g_means, g_quats,
                             g_scales, g_opacity, g_sh, g_log_scales, g_logit_opacity, stream):
    check(lib().gm_project_gaussians_bwd(C.byref(cam), int(N), ptr(means), ptr(quats), ptr(scales), ptr(opacity),
                                         ptr(sh), int(sh_degree), ptr(rec), ptr(g_rec), ptr(g_means), ptr(g_quats),
                                         ptr(g_scales), ptr(g_opacity), ptr(g_sh), ptr(g_log_scales),
                                         ptr(g_logit_opacity), stream))


def gm_mesh_bwd(cam, mesh, light, face_id, g_mesh_rgb, g_mesh_depth, g_verts, g_vcolor, g_vnormal, g_uv, g_mips,
                g_light, stream):
    check(lib().gm_mesh_bwd(C.byref(cam), C.byref(mesh), _light_ref(light), ptr(face_id), ptr(g_mesh_rgb),
                            ptr(g_mesh_depth), ptr(g_verts), ptr(g_vcolor), ptr(g_vnormal), ptr(g_uv), ptr(g_mips),
                            ptr(g_light), stream))


def gm_mipmaps_floats(S) -> int:
    return lib().gm_mipmaps_floats(int(S))


def gm_build_mipmaps(tex, S, mips, stream):
    check(lib().gm_build_mipmaps(ptr(tex), int(S), ptr(mips), stream))


def gm_version() -> int:
    return lib().gm_version()


# analytic edge antialiasing

def gm_edge_adjacency_ws(F) -> int:
    return lib().gm_edge_adjacency_ws(int(F))


def gm_edge_adjacency(mesh, adj, ws, stream):
    check(lib().gm_edge_adjacency(C.byref(mesh), ptr(adj), ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  stream))


def gm_antialias(cam, mesh, vscreen, adj, light, face_id, depth, colour, layer, pairs, tile_dmax, stream):
    check(lib().gm_antialias(C.byref(cam), C.byref(mesh), ptr(vscreen), ptr(adj), _light_ref(light), ptr(face_id),
                             ptr(depth), ptr(colour), ptr(layer), ptr(pairs), ptr(tile_dmax), stream))


def gm_composite_hybrid_fwd_aa(cam, rec, tile_ranges, sorted_ids, layer, bg, softness, out_rgb, out_depth, out_alpha,
                               state, stream):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])  # host array, alive for the call
    check(lib().gm_composite_hybrid_fwd_aa(C.byref(cam), ptr(rec), ptr(tile_ranges), ptr(sorted_ids), ptr(layer),
                                           C.cast(bgv, C.c_void_p), float(softness), ptr(out_rgb), ptr(out_depth),
                                           ptr(out_alpha), ptr(state), stream))


def gm_composite_hybrid_bwd_aa(cam, N, rec, tile_ranges, sorted_ids, layer, bg, softness, state, g_rgb, g_depth,
                               g_alpha, g_rec, g_layer, ws, stream):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    check(lib().gm_composite_hybrid_bwd_aa(C.byref(cam), int(N), ptr(rec), ptr(tile_ranges), ptr(sorted_ids),
                                           ptr(layer), C.cast(bgv, C.c_void_p), float(softness), ptr(state), ptr(g_rgb),
                                           ptr(g_depth), ptr(g_alpha), ptr(g_rec), ptr(g_layer), ptr(ws),
                                           0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_antialias_bwd_ws(width, height) -> int:
    return lib().gm_antialias_bwd_ws(int(width), int(height))


def gm_antialias_bwd(cam, mesh, vscreen, pairs, face_id, depth, colour, g_layer, g_mesh_rgb, g_mesh_depth, g_vscreen,
                     ws, stream):
    check(lib().gm_antialias_bwd(C.byref(cam), C.byref(mesh), ptr(vscreen), ptr(pairs), ptr(face_id), ptr(depth),
                                 ptr(colour), ptr(g_layer), ptr(g_mesh_rgb), ptr(g_mesh_depth), ptr(g_vscreen), ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), stream))


def gm_vscreen_bwd(cam, mesh, g_vscreen, g_verts, stream):
    check(lib().gm_vscreen_bwd(C.byref(cam), C.byref(mesh), ptr(g_vscreen), ptr(g_verts), stream))
