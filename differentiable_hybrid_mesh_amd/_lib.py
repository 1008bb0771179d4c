"""ctypes binding of libgm.so (include/gm.h): same names, argument marshalling only.

Every array argument is a torch tensor on the GPU (or None where the C call takes
NULL); the binding checks that each one is a contiguous tensor of the expected dtype
on the current GPU holding at least the elements the call reads or writes (exactly
that many for per-pixel images), raises ValueError before anything is launched
otherwise, and passes its data pointer.  No computation happens here.  Importing
this module does not touch the GPU; ``lib()`` raises if libgm.so has not been built.
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
           "gm_sort_tile_keys_ws", "gm_sort_tile_keys", "gm_sort_depth", "gm_sort_tiles", "gm_project_sort_depth",
           "gm_composite_hybrid_fwd",
           "gm_composite_hybrid_bwd", "gm_composite_hybrid_bwd_ws", "gm_project_gaussians_bwd", "gm_mesh_bwd", "gm_mipmaps_floats",
           "gm_build_mipmaps", "gm_last_error", "gm_version", "gm_edge_adjacency_ws", "gm_edge_adjacency",
           "gm_antialias", "gm_composite_hybrid_fwd_aa", "gm_composite_hybrid_bwd_aa", "gm_antialias_bwd_ws",
           "gm_antialias_bwd", "gm_vscreen_bwd", "gm_shade_surface", "gm_composite_hybrid_fwd_shaded",
           "gm_composite_hybrid_bwd_noalloc", "gm_composite_hybrid_fwd_stats"]

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
    L.gm_project_sort_depth.argtypes = [cam, I32, P, P, P, P, P, I32, P, I64, P, SZ, P]
    L.gm_sort_tiles.argtypes = [cam, I32, P, P, F32, P, P, I64, P, P, SZ, P]
    L.gm_composite_hybrid_fwd.argtypes = [cam, P, P, P, P, P, mesh, P, light, P, F32, P, P, P, P, P, P, P]
    L.gm_shade_surface.argtypes = [cam, P, mesh, P, light, P, P, P]
    L.gm_composite_hybrid_fwd_shaded.argtypes = [cam, P, P, P, P, P, F32, P, P, P, P, P, P, P]
    L.gm_composite_hybrid_fwd_stats.argtypes = [cam, P, P, P, P, P, F32, P, P, P, P, P, P, P, P]
    L.gm_composite_hybrid_bwd.argtypes = [cam, I32, P, P, P, P, P, F32, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.gm_composite_hybrid_bwd_noalloc.argtypes = [cam, I32, P, P, P, P, P, F32, P, P, P, P, P, P, P, P, P, P]
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
                 "gm_sort_tile_keys", "gm_sort_depth", "gm_sort_tiles", "gm_project_sort_depth",
                 "gm_composite_hybrid_fwd", "gm_composite_hybrid_bwd", "gm_project_gaussians_bwd",
                 "gm_mesh_bwd", "gm_build_mipmaps", "gm_edge_adjacency", "gm_antialias", "gm_composite_hybrid_fwd_aa",
                 "gm_composite_hybrid_bwd_aa", "gm_antialias_bwd", "gm_vscreen_bwd", "gm_shade_surface",
                 "gm_composite_hybrid_fwd_shaded", "gm_composite_hybrid_bwd_noalloc", "gm_composite_hybrid_fwd_stats"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


F32, I32, I64, U8 = "float32", "int32", "int64", "uint8"


def dev(t, name: str, dtype: str, n: int, exact: bool = False, optional: bool = False) -> Optional[int]:
    """Data pointer of tensor ``t`` after checking it: a contiguous torch tensor of
    ``dtype`` on the current GPU with at least ``n`` elements (exactly ``n`` when
    ``exact``); None passes NULL when ``optional``.  Raises ValueError otherwise, so a
    host tensor, a wrongly typed or permuted one, or one too small never reaches a
    kernel."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name}: a tensor is required")
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor is on {t.device}, a GPU tensor is required")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: tensor is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype is not getattr(torch, dtype):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor is not contiguous (shape {tuple(t.shape)}, strides {t.stride()})")
    if exact and t.numel() != n:
        raise ValueError(f"{name}: {t.numel()} elements, expected exactly {n} (shape {tuple(t.shape)})")
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, at least {n} needed")
    return t.data_ptr()


def _ws(t, need: int, name: str = "ws"):
    """Pointer and byte size of a workspace tensor of at least ``need`` bytes."""
    p = dev(t, name, U8, need)
    return p, t.numel()


def _tiles(cam) -> int:
    return ((cam.width + GM_TILE - 1) // GM_TILE) * ((cam.height + GM_TILE - 1) // GM_TILE)


def _hw(cam) -> int:
    return cam.width * cam.height


def _sh_planes(sh_degree: int) -> int:
    return 1 if sh_degree < 0 else (sh_degree + 1) ** 2


def img(t, name: str, cam, k: int, dtype: str = F32, optional: bool = False) -> Optional[int]:
    """dev() for a per-pixel image of ``k`` values per pixel: exactly H*W*k elements
    and, when it has more than one dimension, shape (H, W) (k = 1) or (H, W, k)."""
    if t is not None and getattr(t, "dim", None) is not None and t.dim() > 1:
        want = (cam.height, cam.width) if k == 1 else (cam.height, cam.width, k)
        if tuple(t.shape) != want:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    return dev(t, name, dtype, cam.width * cam.height * k, exact=True, optional=optional)


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
    wp, wb = _ws(ws, gm_bin_triangles_ws(mesh.V, mesh.F, cam.width, cam.height))
    check(lib().gm_bin_triangles(C.byref(cam), C.byref(mesh), dev(vscreen, "vscreen", F32, 3 * mesh.V),
                                 dev(tile_offsets, "tile_offsets", I32, _tiles(cam) + 1),
                                 dev(tile_tris, "tile_tris", I32, int(cap), optional=int(cap) == 0), int(cap),
                                 dev(n_pairs, "n_pairs", I64, 1), wp, wb, stream))


def gm_raster_zbuffer_ws(width, height) -> int:
    return lib().gm_raster_zbuffer_ws(int(width), int(height))


def gm_raster_zbuffer(cam, mesh, vscreen, tile_offsets, tile_tris, face_id, depth, tile_dmax, ws, stream):
    wp, wb = _ws(ws, gm_raster_zbuffer_ws(cam.width, cam.height))
    check(lib().gm_raster_zbuffer(C.byref(cam), C.byref(mesh), dev(vscreen, "vscreen", F32, 3 * mesh.V),
                                  dev(tile_offsets, "tile_offsets", I32, _tiles(cam) + 1),
                                  dev(tile_tris, "tile_tris", I32, 0, optional=True),
                                  img(face_id, "face_id", cam, 1, I32), img(depth, "depth", cam, 1),
                                  dev(tile_dmax, "tile_dmax", F32, _tiles(cam)), wp, wb, stream))


def _gauss_in(N, means, quats, scales, opacity, sh, sh_degree):
    n = int(N)
    return (dev(means, "means", F32, 3 * n), dev(quats, "quats", F32, 4 * n), dev(scales, "scales", F32, 3 * n),
            dev(opacity, "opacity", F32, n), dev(sh, "sh", F32, 3 * _sh_planes(int(sh_degree)) * n))


def gm_project_gaussians(cam, N, means, quats, scales, opacity, sh, sh_degree, rec, stream):
    check(lib().gm_project_gaussians(C.byref(cam), int(N), *_gauss_in(N, means, quats, scales, opacity, sh, sh_degree),
                                     int(sh_degree), dev(rec, "rec", F32, GM_REC * int(N)), stream))


def gm_project_gaussians_multi(cams, N, means, quats, scales, opacity, sh, sh_degree, rec, stream):
    """cams: sequence of GmCamera; rec holds len(cams) * N records."""
    arr = (GmCamera * max(len(cams), 1))(*cams)
    check(lib().gm_project_gaussians_multi(arr, len(cams), int(N),
                                           *_gauss_in(N, means, quats, scales, opacity, sh, sh_degree),
                                           int(sh_degree), dev(rec, "rec", F32, GM_REC * int(N) * len(cams)),
                                           stream))


def gm_sort_tile_keys_ws(N, cap, width, height) -> int:
    return lib().gm_sort_tile_keys_ws(int(N), int(cap), width, height)


def _sort_common(cam, N, rec, cap, ws):
    wp, wb = _ws(ws, gm_sort_tile_keys_ws(N, cap, cam.width, cam.height))
    return dev(rec, "rec", F32, GM_REC * int(N), optional=int(N) == 0), wp, wb


def gm_sort_tile_keys(cam, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap, n_keys, ws, stream):
    """n_keys: device int64 tensor that receives the key count (asynchronously)."""
    rp, wp, wb = _sort_common(cam, N, rec, cap, ws)
    check(lib().gm_sort_tile_keys(C.byref(cam), int(N), rp,
                                  dev(tile_dmax, "tile_dmax", F32, _tiles(cam), optional=True), float(softness),
                                  dev(tile_ranges, "tile_ranges", I32, 2 * _tiles(cam)),
                                  dev(sorted_ids, "sorted_ids", I32, int(cap), optional=int(cap) == 0), int(cap),
                                  dev(n_keys, "n_keys", I64, 1), wp, wb, stream))


def gm_sort_depth(cam, N, rec, cap, ws, stream):
    """First half of gm_sort_tile_keys: the depth order, kept in ws for gm_sort_tiles."""
    rp, wp, wb = _sort_common(cam, N, rec, cap, ws)
    check(lib().gm_sort_depth(C.byref(cam), int(N), rp, int(cap), wp, wb, stream))


def gm_project_sort_depth(cam, N, means, quats, scales, opacity, sh, sh_degree, rec, cap, ws, stream):
    """gm_project_gaussians then gm_sort_depth in one call (the projection also writes the
    depth sort's keys into ws)."""
    gin = _gauss_in(N, means, quats, scales, opacity, sh, sh_degree)
    rp, wp, wb = _sort_common(cam, N, rec, cap, ws)
    check(lib().gm_project_sort_depth(C.byref(cam), int(N), *gin, int(sh_degree), rp, int(cap), wp, wb, stream))


def gm_sort_tiles(cam, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap, n_keys, ws, stream):
    """Second half of gm_sort_tile_keys, ordered after gm_sort_depth on the same ws."""
    rp, wp, wb = _sort_common(cam, N, rec, cap, ws)
    check(lib().gm_sort_tiles(C.byref(cam), int(N), rp, dev(tile_dmax, "tile_dmax", F32, _tiles(cam), optional=True),
                              float(softness), dev(tile_ranges, "tile_ranges", I32, 2 * _tiles(cam)),
                              dev(sorted_ids, "sorted_ids", I32, int(cap), optional=int(cap) == 0), int(cap),
                              dev(n_keys, "n_keys", I64, 1), wp, wb, stream))


def _light_ref(light):
    return None if light is None else C.byref(light)


def _bg(bg):
    vals = [float(x) for x in bg]
    if len(vals) != 3:
        raise ValueError(f"bg: 3 values expected, got {len(vals)}")
    return (C.c_float * 3)(*vals)


def _lists(cam, rec, tile_ranges, sorted_ids):
    # rec and sorted_ids: the kernels read the entries the tile ranges name, which
    # were written by the sort for these buffers; only their type and place are checked
    return (dev(rec, "rec", F32, 0), dev(tile_ranges, "tile_ranges", I32, 2 * _tiles(cam)),
            dev(sorted_ids, "sorted_ids", I32, 0))


def _fwd_out(cam, out_rgb, out_depth, out_alpha, state_T, state_last):
    return (img(out_rgb, "out_rgb", cam, 3), img(out_depth, "out_depth", cam, 1),
            img(out_alpha, "out_alpha", cam, 1), img(state_T, "state_T", cam, 1),
            img(state_last, "state_last", cam, 1, I32))


def gm_composite_hybrid_fwd(cam, rec, tile_ranges, sorted_ids, face_id, depth, mesh, vscreen, light, bg,
                            softness, out_rgb, out_depth, out_alpha, state_T, state_last, state_cm, stream):
    bgv = _bg(bg)
    check(lib().gm_composite_hybrid_fwd(C.byref(cam), *_lists(cam, rec, tile_ranges, sorted_ids),
                                        img(face_id, "face_id", cam, 1, I32), img(depth, "depth", cam, 1),
                                        C.byref(mesh), dev(vscreen, "vscreen", F32, 3 * mesh.V, optional=mesh.F == 0),
                                        _light_ref(light), C.cast(bgv, C.c_void_p), float(softness),
                                        *_fwd_out(cam, out_rgb, out_depth, out_alpha, state_T, state_last),
                                        img(state_cm, "state_cm", cam, 3), stream))


def gm_shade_surface(cam, face_id, mesh, vscreen, light, bg, state_cm, stream):
    bgv = _bg(bg)
    check(lib().gm_shade_surface(C.byref(cam), img(face_id, "face_id", cam, 1, I32), C.byref(mesh),
                                 dev(vscreen, "vscreen", F32, 3 * mesh.V, optional=mesh.F == 0), _light_ref(light),
                                 C.cast(bgv, C.c_void_p), img(state_cm, "state_cm", cam, 3), stream))


def gm_composite_hybrid_fwd_shaded(cam, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_cm, out_rgb,
                                   out_depth, out_alpha, state_T, state_last, stream):
    check(lib().gm_composite_hybrid_fwd_shaded(C.byref(cam), *_lists(cam, rec, tile_ranges, sorted_ids),
                                               img(face_id, "face_id", cam, 1, I32), img(depth, "depth", cam, 1),
                                               float(softness), img(state_cm, "state_cm", cam, 3),
                                               *_fwd_out(cam, out_rgb, out_depth, out_alpha, state_T, state_last),
                                               stream))


def gm_composite_hybrid_fwd_stats(cam, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_cm, out_rgb,
                                  out_depth, out_alpha, state_T, state_last, stats, stream):
    """gm_composite_hybrid_fwd_shaded with counters added to stats (device int64 [3])."""
    check(lib().gm_composite_hybrid_fwd_stats(C.byref(cam), *_lists(cam, rec, tile_ranges, sorted_ids),
                                              img(face_id, "face_id", cam, 1, I32), img(depth, "depth", cam, 1),
                                              float(softness), img(state_cm, "state_cm", cam, 3),
                                              *_fwd_out(cam, out_rgb, out_depth, out_alpha, state_T, state_last),
                                              dev(stats, "stats", I64, 3), stream))


def gm_composite_hybrid_bwd_ws(width, height) -> int:
    return lib().gm_composite_hybrid_bwd_ws(int(width), int(height))


def _bwd_args(cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T, state_last, state_cm, g_rgb,
              g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth):
    return (C.byref(cam), int(N), *_lists(cam, rec, tile_ranges, sorted_ids), img(face_id, "face_id", cam, 1, I32),
            img(depth, "depth", cam, 1), float(softness), img(state_T, "state_T", cam, 1),
            img(state_last, "state_last", cam, 1, I32), img(state_cm, "state_cm", cam, 3), img(g_rgb, "g_rgb", cam, 3),
            img(g_depth, "g_depth", cam, 1, optional=True), img(g_alpha, "g_alpha", cam, 1, optional=True),
            dev(g_rec, "g_rec", F32, GM_GRAD * int(N), optional=int(N) == 0),
            img(g_mesh_rgb, "g_mesh_rgb", cam, 3, optional=True), img(g_mesh_depth, "g_mesh_depth", cam, 1, optional=True))


def gm_composite_hybrid_bwd(cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T, state_last,
                            state_cm, g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth, ws, stream):
    """ws: device scratch of gm_composite_hybrid_bwd_ws(width, height) bytes."""
    wp, wb = _ws(ws, gm_composite_hybrid_bwd_ws(cam.width, cam.height))
    check(lib().gm_composite_hybrid_bwd(*_bwd_args(cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness,
                                                   state_T, state_last, state_cm, g_rgb, g_depth, g_alpha, g_rec,
                                                   g_mesh_rgb, g_mesh_depth), wp, wb, stream))


def gm_composite_hybrid_bwd_noalloc(cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T,
                                    state_last, state_cm, g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth,
                                    stream):
    """gm_composite_hybrid_bwd with the library's fixed scratch instead of ws."""
    check(lib().gm_composite_hybrid_bwd_noalloc(*_bwd_args(cam, N, rec, tile_ranges, sorted_ids, face_id, depth,
                                                           softness, state_T, state_last, state_cm, g_rgb, g_depth,
                                                           g_alpha, g_rec, g_mesh_rgb, g_mesh_depth), stream))


def gm_project_gaussians_bwd(cam, N, means, quats, scales, opacity, sh, sh_degree, rec, g_rec, g_means, g_quats,
                             g_scales, g_opacity, g_sh, g_log_scales, g_logit_opacity, stream):
    n, K = int(N), _sh_planes(int(sh_degree))
    check(lib().gm_project_gaussians_bwd(C.byref(cam), n, *_gauss_in(N, means, quats, scales, opacity, sh, sh_degree),
                                         int(sh_degree), dev(rec, "rec", F32, GM_REC * n),
                                         dev(g_rec, "g_rec", F32, GM_GRAD * n), dev(g_means, "g_means", F32, 3 * n),
                                         dev(g_quats, "g_quats", F32, 4 * n), dev(g_scales, "g_scales", F32, 3 * n),
                                         dev(g_opacity, "g_opacity", F32, n), dev(g_sh, "g_sh", F32, 3 * K * n),
                                         dev(g_log_scales, "g_log_scales", F32, 3 * n, optional=True),
                                         dev(g_logit_opacity, "g_logit_opacity", F32, n, optional=True), stream))


def gm_mesh_bwd(cam, mesh, light, face_id, g_mesh_rgb, g_mesh_depth, g_verts, g_vcolor, g_vnormal, g_uv, g_mips,
                g_light, stream):
    V = mesh.V
    check(lib().gm_mesh_bwd(C.byref(cam), C.byref(mesh), _light_ref(light), img(face_id, "face_id", cam, 1, I32),
                            img(g_mesh_rgb, "g_mesh_rgb", cam, 3, optional=True),
                            img(g_mesh_depth, "g_mesh_depth", cam, 1, optional=True),
                            dev(g_verts, "g_verts", F32, 3 * V, optional=True),
                            dev(g_vcolor, "g_vcolor", F32, 3 * V, optional=True),
                            dev(g_vnormal, "g_vnormal", F32, 3 * V, optional=True),
                            dev(g_uv, "g_uv", F32, 2 * mesh.Vt, optional=True),
                            dev(g_mips, "g_mips", F32, gm_mipmaps_floats(mesh.tex_size) if mesh.tex_size else 0,
                                optional=True),
                            dev(g_light, "g_light", F32, 13, optional=True), stream))


def gm_mipmaps_floats(S) -> int:
    return lib().gm_mipmaps_floats(int(S))


def gm_build_mipmaps(tex, S, mips, stream):
    check(lib().gm_build_mipmaps(dev(tex, "tex", F32, int(S) * int(S) * 3), int(S),
                                 dev(mips, "mips", F32, gm_mipmaps_floats(S)), stream))


def gm_version() -> int:
    return lib().gm_version()


# analytic edge antialiasing

def gm_edge_adjacency_ws(F) -> int:
    return lib().gm_edge_adjacency_ws(int(F))


def gm_edge_adjacency(mesh, adj, ws, stream):
    wp, wb = _ws(ws, gm_edge_adjacency_ws(mesh.F))
    check(lib().gm_edge_adjacency(C.byref(mesh), dev(adj, "adj", I32, 3 * mesh.F), wp, wb, stream))


def gm_antialias(cam, mesh, vscreen, adj, light, face_id, depth, colour, layer, pairs, tile_dmax, stream):
    check(lib().gm_antialias(C.byref(cam), C.byref(mesh), dev(vscreen, "vscreen", F32, 3 * mesh.V),
                             dev(adj, "adj", I32, 3 * mesh.F), _light_ref(light), img(face_id, "face_id", cam, 1, I32),
                             img(depth, "depth", cam, 1), img(colour, "colour", cam, 3), img(layer, "layer", cam, 8),
                             img(pairs, "pairs", cam, 12, optional=True),
                             dev(tile_dmax, "tile_dmax", F32, _tiles(cam), optional=True), stream))


def gm_composite_hybrid_fwd_aa(cam, rec, tile_ranges, sorted_ids, layer, bg, softness, out_rgb, out_depth, out_alpha,
                               state, stream):
    bgv = _bg(bg)  # host array, alive for the call
    check(lib().gm_composite_hybrid_fwd_aa(C.byref(cam), *_lists(cam, rec, tile_ranges, sorted_ids),
                                           img(layer, "layer", cam, 8), C.cast(bgv, C.c_void_p), float(softness),
                                           img(out_rgb, "out_rgb", cam, 3), img(out_depth, "out_depth", cam, 1),
                                           img(out_alpha, "out_alpha", cam, 1), img(state, "state", cam, 8), stream))


def gm_composite_hybrid_bwd_aa(cam, N, rec, tile_ranges, sorted_ids, layer, bg, softness, state, g_rgb, g_depth,
                               g_alpha, g_rec, g_layer, ws, stream):
    bgv = _bg(bg)
    wp, wb = _ws(ws, gm_composite_hybrid_bwd_ws(cam.width, cam.height))
    check(lib().gm_composite_hybrid_bwd_aa(C.byref(cam), int(N), *_lists(cam, rec, tile_ranges, sorted_ids),
                                           img(layer, "layer", cam, 8), C.cast(bgv, C.c_void_p), float(softness),
                                           img(state, "state", cam, 8), img(g_rgb, "g_rgb", cam, 3),
                                           img(g_depth, "g_depth", cam, 1, optional=True),
                                           img(g_alpha, "g_alpha", cam, 1, optional=True),
                                           dev(g_rec, "g_rec", F32, GM_GRAD * int(N), optional=int(N) == 0),
                                           img(g_layer, "g_layer", cam, 8), wp, wb, stream))


def gm_antialias_bwd_ws(width, height) -> int:
    return lib().gm_antialias_bwd_ws(int(width), int(height))


def gm_antialias_bwd(cam, mesh, vscreen, pairs, face_id, depth, colour, g_layer, g_mesh_rgb, g_mesh_depth, g_vscreen,
                     ws, stream):
    wp, wb = _ws(ws, gm_antialias_bwd_ws(cam.width, cam.height))
    check(lib().gm_antialias_bwd(C.byref(cam), C.byref(mesh), dev(vscreen, "vscreen", F32, 3 * mesh.V),
                                 img(pairs, "pairs", cam, 12), img(face_id, "face_id", cam, 1, I32),
                                 img(depth, "depth", cam, 1), img(colour, "colour", cam, 3),
                                 img(g_layer, "g_layer", cam, 8), img(g_mesh_rgb, "g_mesh_rgb", cam, 3, optional=True),
                                 img(g_mesh_depth, "g_mesh_depth", cam, 1, optional=True),
                                 dev(g_vscreen, "g_vscreen", F32, 2 * mesh.V), wp, wb, stream))


def gm_vscreen_bwd(cam, mesh, g_vscreen, g_verts, stream):
    check(lib().gm_vscreen_bwd(C.byref(cam), C.byref(mesh), dev(g_vscreen, "g_vscreen", F32, 2 * mesh.V),
                               dev(g_verts, "g_verts", F32, 3 * mesh.V), stream))
