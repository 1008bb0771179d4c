"""CPU oracle for the hybrid mesh + Gaussian tile rasterizer (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``liboracle.so`` built from
``gm_oracle.c``, ``project_bwd.c``, ``mesh_bwd.c`` and ``antialias.c`` with gcc (``-O2 -fopenmp
-ffp-contract=off``) and shares no code with the HIP library; the two meet only at
the seeded inputs of ``scenes``.

The functions below marshal numpy arrays into the C oracle and return plain numpy
arrays.  ``render_view`` runs the whole definition for one view on a set of tiles
(all tiles by default).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "gm_oracle.c"), os.path.join(_HERE, "project_bwd.c"),
         os.path.join(_HERE, "mesh_bwd.c"), os.path.join(_HERE, "antialias.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
NREC = 13

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no -ffast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in _SRCS):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, *_SRCS, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Camera(C.Structure):
    _fields_ = [("width", C.c_int), ("height", C.c_int),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("R", C.c_float * 9), ("t", C.c_float * 3), ("near_z", C.c_float)]


class Light(C.Structure):
    _fields_ = [("pos", C.c_float * 3), ("ambient", C.c_float * 3), ("diffuse", C.c_float * 3),
                ("specular", C.c_float * 3), ("shininess", C.c_float)]


class Mesh(C.Structure):
    _fields_ = [("cam", C.POINTER(Camera)), ("V", C.c_int), ("F", C.c_int),
                ("vscreen", C.c_void_p), ("faces", C.c_void_p), ("vcolor", C.c_void_p),
                ("vnormal", C.c_void_p), ("verts", C.c_void_p), ("uv", C.c_void_p),
                ("faces_uv", C.c_void_p), ("Vt", C.c_int), ("mips", C.c_void_p),
                ("tex_size", C.c_int), ("light", C.POINTER(Light))]


class Comp(C.Structure):
    _fields_ = [("cam", C.POINTER(Camera)), ("mesh", C.POINTER(Mesh)), ("N", C.c_int),
                ("rec", C.c_void_p), ("ntiles", C.c_int), ("tiles", C.c_void_p),
                ("offsets", C.c_void_p), ("ids", C.c_void_p), ("face_id", C.c_void_p),
                ("depth", C.c_void_p), ("bg", C.c_double * 3), ("softness", C.c_double),
                ("g_rgb", C.c_void_p), ("g_depth", C.c_void_p), ("g_alpha", C.c_void_p),
                ("rgb", C.c_void_p), ("out_depth", C.c_void_p), ("alpha", C.c_void_p),
                ("rgb2", C.c_void_p), ("depth2", C.c_void_p), ("alpha2", C.c_void_p),
                ("T_final", C.c_void_p), ("n_last", C.c_void_p), ("n_incl", C.c_void_p),
                ("margin", C.c_void_p), ("clamp_margin", C.c_void_p), ("grad", C.c_void_p),
                ("g_mesh_rgb", C.c_void_p), ("g_mesh_depth", C.c_void_p),
                ("pairs_evaluated", C.c_void_p), ("layer", C.c_void_p), ("g_layer", C.c_void_p),
                ("T_back", C.c_void_p), ("n_last_back", C.c_void_p)]


_lib = None


class MeshB(C.Structure):
    """mb_mesh of mesh_bwd.c: fp64 mesh attributes for the mesh-side backward."""
    _fields_ = [("V", C.c_int), ("F", C.c_int), ("Vt", C.c_int), ("S", C.c_int),
                ("verts", C.c_void_p), ("faces", C.c_void_p), ("vcolor", C.c_void_p),
                ("vnormal", C.c_void_p), ("uv", C.c_void_p), ("faces_uv", C.c_void_p),
                ("tex", C.c_void_p), ("light", C.c_void_p)]


def lib():
    """The loaded oracle library.  ``GM_ORACLE_LIB`` names another build of the same
    sources to load instead (the mutation tests load copies with a planted mistake
    this way, in a child process)."""
    global _lib
    if _lib is None:
        _lib = C.CDLL(os.environ.get("GM_ORACLE_LIB") or build())
        P, I, D = C.c_void_p, C.c_int, C.c_double
        cam = C.POINTER(Camera)
        _lib.oc_project_vertices.argtypes = [cam, I, P, P]
        _lib.oc_tile_bins.argtypes = [cam, I, I, P, P, P, P, P, P]
        _lib.oc_zbuffer.argtypes = [cam, I, I, P, P, P, I, P, I, P, P, P, P, P]
        _lib.oc_project_gaussians.argtypes = [cam, I, P, P, P, P, P, I, P, P, P, P]
        _lib.oc_depth_order.argtypes = [I, P, P, P]
        _lib.oc_depth_order.restype = I
        _lib.oc_tile_counts.argtypes = [cam, P, P, I, I, P, P]
        _lib.oc_tile_lists.argtypes = [cam, P, P, P, I, P, D, I, P, P, P, P]
        _lib.oc_build_mips.argtypes = [P, I, P]
        _lib.oc_shade_pixels.argtypes = [C.POINTER(Mesh), I, P, P, P, P]
        _lib.oc_composite.argtypes = [C.POINTER(Comp)]
        _lib.oc_Phi.argtypes = [D]
        _lib.oc_Phi.restype = D
        _lib.oc_sh_basis.argtypes = [D, D, D, P]
        _lib.oc_num_threads.argtypes = []
        _lib.oc_num_threads.restype = I
        _lib.oc_project_f64.argtypes = [cam, I, P, P, P, P, P, I, P]
        _lib.oc_project_bwd.argtypes = [cam, I, P, P, P, P, I, P, P, P, P, P, P, P]
        _lib.oc_mesh_fwd64.argtypes = [cam, C.POINTER(MeshB), I, P, P, P, P]
        _lib.oc_mesh_bwd.argtypes = [cam, C.POINTER(MeshB), I, P, P, P, P, P, P, P, P, P, P]
        _lib.oc_vscreen_bwd.argtypes = [cam, C.POINTER(MeshB), P, P]
        _lib.oc_edge_adjacency.argtypes = [I, P, P]
        _lib.oc_antialias.argtypes = [cam, I, I, P, P, P, P, P, P, P, P, P]
        _lib.oc_antialias_bwd.argtypes = [cam, I, I, P, P, P, P, P, P, P, P, P, P, P]
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def camera(scene, view_index: int = 0) -> Camera:
    v = scene.views[view_index]
    cam = Camera()
    cam.width, cam.height = scene.width, scene.height
    cam.fx, cam.fy, cam.cx, cam.cy = scene.fx, scene.fy, scene.cx, scene.cy
    for i in range(9):
        cam.R[i] = float(v.R[i])
    for i in range(3):
        cam.t[i] = float(v.t[i])
    cam.near_z = scene.near_z
    return cam


def make_camera(width, height, fx, fy, cx, cy, R=None, t=None, near_z=0.01) -> Camera:
    cam = Camera()
    cam.width, cam.height, cam.fx, cam.fy, cam.cx, cam.cy = width, height, fx, fy, cx, cy
    R = np.eye(3, dtype=np.float32).reshape(-1) if R is None else np.asarray(R, np.float32).reshape(-1)
    t = np.zeros(3, np.float32) if t is None else np.asarray(t, np.float32)
    for i in range(9):
        cam.R[i] = float(R[i])
    for i in range(3):
        cam.t[i] = float(t[i])
    cam.near_z = near_z
    return cam


def n_tiles(cam: Camera):
    tx, ty = (cam.width + 15) // 16, (cam.height + 15) // 16
    return tx, ty, tx * ty


# ---------------------------------------------------------------------------
# stages
# ---------------------------------------------------------------------------

def project_vertices(cam: Camera, verts: np.ndarray) -> np.ndarray:
    verts = _c(verts, np.float32)
    V = verts.shape[1]
    out = np.empty((3, V), np.float32)
    lib().oc_project_vertices(C.byref(cam), V, _p(verts), _p(out))
    return out


def tile_bins(cam: Camera, vscreen, faces, mask=None):
    """Bins by pixel-centre bounding box: (offsets [T+1], ids)."""
    faces = _c(faces, np.int32)
    mask = _c(mask, np.uint8)
    V, F = vscreen.shape[1], faces.shape[1]
    T = n_tiles(cam)[2]
    counts = np.zeros(T, np.int32)
    lib().oc_tile_bins(C.byref(cam), V, F, _p(vscreen), _p(faces), _p(mask), _p(counts), None, None)
    offsets = np.zeros(T + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    ids = np.zeros(max(int(offsets[-1]), 1), np.int32)
    lib().oc_tile_bins(C.byref(cam), V, F, _p(vscreen), _p(faces), _p(mask), _p(counts),
                       _p(offsets), _p(ids))
    return offsets, ids[: offsets[-1]]


def zbuffer(cam: Camera, vscreen, faces, mask=None, tiles=None, prefilter=False):
    faces = _c(faces, np.int32)
    mask = _c(mask, np.uint8)
    V, F = vscreen.shape[1], faces.shape[1]
    W, H = cam.width, cam.height
    T = n_tiles(cam)[2]
    tiles = np.arange(T, dtype=np.int32) if tiles is None else _c(tiles, np.int32)
    face_id = np.full((H, W), -1, np.int32)
    depth = np.full((H, W), np.inf, np.float32)
    z1 = np.full((H, W), np.inf)
    z2 = np.full((H, W), np.inf)
    dmax = np.full(T, np.nan, np.float32)
    lib().oc_zbuffer(C.byref(cam), V, F, _p(vscreen), _p(faces), _p(mask), len(tiles), _p(tiles),
                     1 if prefilter else 0, _p(face_id), _p(depth), _p(z1), _p(z2), _p(dmax))
    return {"face_id": face_id, "depth": depth, "z1": z1, "z2": z2, "tile_dmax": dmax}


def project_gaussians(cam: Camera, means, quats, scales, opacity, sh, sh_degree):
    means, quats, scales = _c(means, np.float32), _c(quats, np.float32), _c(scales, np.float32)
    opacity, sh = _c(opacity, np.float32), _c(sh, np.float32)
    N = means.shape[1]
    rec = np.zeros((N, NREC), np.float32)
    rect = np.zeros((N, 4), np.int32)
    valid = np.zeros(N, np.int32)
    rgb = np.zeros((N, 3), np.float64)
    lib().oc_project_gaussians(C.byref(cam), N, _p(means), _p(quats), _p(scales), _p(opacity),
                               _p(sh), int(sh_degree), _p(rec), _p(rect), _p(valid), _p(rgb))
    return {"rec": rec, "rect": rect, "valid": valid, "rgb64": rgb}


def depth_order(rec, valid):
    N = rec.shape[0]
    order = np.zeros(max(N, 1), np.int32)
    n = lib().oc_depth_order(N, _p(rec), _p(valid), _p(order))
    return order[:n].copy()


def tile_lists(cam: Camera, rec, rect, order, tiles, tile_dmax=None, softness=1.0):
    """Per-tile lists (pre-cull) with the cull ratio of every entry.
    Returns (offsets [len(tiles)+1] int64, ids, cullq)."""
    tiles = _c(tiles, np.int32)
    counts = np.zeros(len(tiles), np.int32)
    lib().oc_tile_counts(C.byref(cam), _p(rect), _p(order), len(order), len(tiles), _p(tiles),
                         _p(counts))
    offsets = np.zeros(len(tiles) + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    K = int(offsets[-1])
    ids = np.zeros(max(K, 1), np.int32)
    cullq = np.zeros(max(K, 1), np.float64)
    dm = _c(tile_dmax, np.float32)
    lib().oc_tile_lists(C.byref(cam), _p(rec), _p(rect), _p(order), len(order), _p(dm),
                        float(softness), len(tiles), _p(tiles), _p(offsets), _p(ids), _p(cullq))
    return offsets, ids[:K], cullq[:K]


def apply_cull(offsets, ids, cullq):
    """Drop entries with cull ratio < 1; returns new (offsets, ids)."""
    keep = cullq >= 1.0
    nseg = len(offsets) - 1
    seg = np.repeat(np.arange(nseg), np.diff(offsets))
    cnt = np.bincount(seg[keep], minlength=nseg)
    noff = np.zeros_like(offsets)
    noff[1:] = np.cumsum(cnt)
    return noff, ids[keep]


def build_mips(texture: np.ndarray) -> np.ndarray:
    tex = _c(texture, np.float32)
    S = tex.shape[0]
    total, s = 0, S
    while s >= 1:
        total += s * s * 3
        s //= 2
    out = np.zeros(total, np.float64)
    lib().oc_build_mips(_p(tex), S, _p(out))
    return out


class MeshRef:
    """Keeps the numpy arrays alive while the C struct points at them."""

    def __init__(self, cam: Camera, scene, vscreen, mips=None, light=None):
        self.keep = []
        m = Mesh()
        m.cam = C.pointer(cam)
        m.V, m.F = scene.V, scene.F

        def ptr(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=dt)
            self.keep.append(a)
            return a.ctypes.data

        m.vscreen = ptr(vscreen, np.float32)
        m.faces = ptr(scene.faces, np.int32)
        m.vcolor = ptr(scene.vcolor, np.float32)
        m.vnormal = ptr(scene.vnormal, np.float32)
        m.verts = ptr(scene.verts, np.float32)
        m.uv = ptr(scene.uv, np.float32)
        m.faces_uv = ptr(scene.faces_uv, np.int32)
        m.Vt = 0 if scene.uv is None else scene.uv.shape[1]
        m.mips = ptr(mips, np.float64)
        m.tex_size = 0 if scene.texture is None else scene.texture.shape[0]
        lt = light if light is not None else scene.light
        if lt is not None:
            L = Light()
            for i in range(3):
                L.pos[i] = float(lt["pos"][i])
                L.ambient[i] = float(lt["ambient"][i])
                L.diffuse[i] = float(lt["diffuse"][i])
                L.specular[i] = float(lt["specular"][i])
            L.shininess = float(lt["shininess"])
            self.light = L
            m.light = C.pointer(L)
        self.cam = cam
        self.struct = m


def shade_pixels(meshref: MeshRef, pix, face_id):
    pix = _c(pix, np.int32)
    face_id = _c(face_id, np.int32)
    n = len(pix)
    cm = np.zeros((n, 3))
    lod = np.zeros(n)
    lib().oc_shade_pixels(C.byref(meshref.struct), n, _p(pix), _p(face_id), _p(cm), _p(lod))
    return cm, lod


def composite(cam: Camera, meshref: Optional[MeshRef], rec64, tiles, offsets, ids, face_id, depth,
              bg=(1.0, 1.0, 1.0), softness=1.0, grads=None, layer=None):
    """Forward (both layer forms) and, when ``grads`` is given, the reverse mode.
    With ``layer`` ([H][W][6] antialiased mesh layer from ``antialias``) the mesh
    enters through it and the general two-layer form is computed, forward and
    reverse (``g_layer``, ``T_back``, ``n_last_back`` are returned as well)."""
    H, W = cam.height, cam.width
    N = rec64.shape[0]
    rec64 = _c(rec64, np.float64)
    tiles = _c(tiles, np.int32)
    offsets = _c(offsets, np.int64)
    ids = _c(ids if len(ids) else np.zeros(1, np.int32), np.int32)
    face_id = _c(face_id, np.int32)
    depth64 = _c(depth, np.float64)
    out = {
        "rgb": np.full((H, W, 3), np.nan), "depth": np.full((H, W), np.nan),
        "alpha": np.full((H, W), np.nan), "rgb2": np.full((H, W, 3), np.nan),
        "depth2": np.full((H, W), np.nan), "alpha2": np.full((H, W), np.nan),
        "T_final": np.full((H, W), np.nan), "n_last": np.full((H, W), -1, np.int32),
        "n_incl": np.full((H, W), -1, np.int32), "margin": np.full((H, W), np.inf),
        "clamp_margin": np.full((H, W), np.inf),
        "grad": np.zeros((N, NREC)), "g_mesh_rgb": np.zeros((H, W, 3)),
        "g_mesh_depth": np.zeros((H, W)), "pairs": np.zeros(1, np.int64),
    }
    a = Comp()
    a.cam = C.pointer(cam)
    a.mesh = C.pointer(meshref.struct) if meshref is not None else None
    a.N = N
    a.rec = _p(rec64)
    a.ntiles = len(tiles)
    a.tiles = _p(tiles)
    a.offsets = _p(offsets)
    a.ids = _p(ids)
    a.face_id = _p(face_id)
    a.depth = _p(depth64)
    for i in range(3):
        a.bg[i] = float(bg[i])
    a.softness = float(softness)
    keep = []
    if grads is not None:
        g_rgb = _c(grads["rgb"], np.float32)
        g_d = _c(grads.get("depth"), np.float32)
        g_a = _c(grads.get("alpha"), np.float32)
        keep += [g_rgb, g_d, g_a]
        a.g_rgb, a.g_depth, a.g_alpha = _p(g_rgb), _p(g_d), _p(g_a)
    for k in ("rgb", "alpha", "rgb2", "depth2", "alpha2", "T_final", "n_last", "n_incl", "margin",
              "clamp_margin", "grad", "g_mesh_rgb", "g_mesh_depth"):
        setattr(a, k, _p(out[k]))
    a.out_depth = _p(out["depth"])
    a.pairs_evaluated = _p(out["pairs"])
    if layer is not None:
        layer = _c(layer, np.float64)
        keep.append(layer)
        out["g_layer"] = np.zeros((H, W, 6))
        out["T_back"] = np.full((H, W), np.nan)
        out["n_last_back"] = np.full((H, W), -1, np.int32)
        a.layer, a.g_layer = _p(layer), _p(out["g_layer"])
        a.T_back, a.n_last_back = _p(out["T_back"]), _p(out["n_last_back"])
    lib().oc_composite(C.byref(a))
    out["pairs"] = int(out["pairs"][0])
    return out


def num_threads() -> int:
    return int(lib().oc_num_threads())


def Phi(s: float) -> float:
    return lib().oc_Phi(float(s))


def sh_basis(x, y, z) -> np.ndarray:
    Y = np.zeros(16)
    lib().oc_sh_basis(float(x), float(y), float(z), _p(Y))
    return Y


def tiles_of_pixels(cam: Camera, pix: Sequence[int]) -> np.ndarray:
    TX = (cam.width + 15) // 16
    pix = np.asarray(pix)
    return np.unique((pix // cam.width) // 16 * TX + (pix % cam.width) // 16).astype(np.int32)


# ---------------------------------------------------------------------------
# whole view
# ---------------------------------------------------------------------------

def _with_neighbour_tiles(cam: Camera, tiles) -> np.ndarray:
    TX, TY, _ = n_tiles(cam)
    t = np.asarray(tiles, np.int64)
    tx, ty = t % TX, t // TX
    out = set()
    for dy in (-1, 0, 1):
        for dx in (-1, 0, 1):
            x, y = tx + dx, ty + dy
            ok = (x >= 0) & (x < TX) & (y >= 0) & (y < TY)
            out.update((y[ok] * TX + x[ok]).tolist())
    return np.array(sorted(out), np.int32)


def render_view(scene, view_index: int = 0, tiles=None, cull: bool = True, backward: bool = True,
                prefilter: Optional[bool] = None, grads=None, mips=None, antialias: bool = False):
    """The whole definition for one view on ``tiles`` (all tiles when None).

    Returns a dict with the z-buffer, records, per-tile lists (pre- and post-cull),
    the composite outputs and, with ``backward``, the gradients of the 13 record
    fields and of the mesh colour / depth, for the upstream gradients ``grads``
    (the scene's own when None).  With ``antialias`` the mesh enters through the
    antialiased layer (``layer``, with ``adj`` and ``colour``); the z-buffer then
    also covers the neighbouring tiles, whose border pixels the pairs reach, and the
    composite's reverse mode returns ``g_layer``."""
    cam = camera(scene, view_index)
    TX, TY, T = n_tiles(cam)
    tiles = np.arange(T, dtype=np.int32) if tiles is None else np.asarray(tiles, np.int32)
    if prefilter is None:
        prefilter = scene.F * scene.width * scene.height > 1e9
    res = {"cam": cam, "tiles": tiles}
    if scene.F > 0:
        vs = project_vertices(cam, scene.verts)
        zt = _with_neighbour_tiles(cam, tiles) if antialias else tiles
        zb = zbuffer(cam, vs, scene.faces, scene.face_mask, tiles=zt, prefilter=prefilter)
    else:
        vs = np.zeros((3, 0), np.float32)
        zb = {"face_id": np.full((scene.height, scene.width), -1, np.int32),
              "depth": np.full((scene.height, scene.width), np.inf, np.float32),
              "z1": np.full((scene.height, scene.width), np.inf),
              "z2": np.full((scene.height, scene.width), np.inf),
              "tile_dmax": np.full(T, np.inf, np.float32)}
    res["vscreen"] = vs
    res.update(zb)
    pg = project_gaussians(cam, scene.means, scene.quats, scene.scales, scene.opacity, scene.sh,
                           scene.sh_degree)
    res.update(pg)
    order = depth_order(pg["rec"], pg["valid"])
    res["order"] = order
    dm = np.where(np.isnan(zb["tile_dmax"]), np.inf, zb["tile_dmax"]).astype(np.float32)
    if scene.texture is not None and mips is None:
        mips = build_mips(scene.texture)
    mref = MeshRef(cam, scene, vs, mips=mips) if scene.F > 0 else None
    layer = None
    if antialias:
        if scene.F > 0:
            adj = edge_adjacency(scene.faces)
            colour = surface_colours(mref, zb["face_id"])
            layer = aa_layer(cam, vs.astype(np.float64), scene.faces, scene.face_mask, adj, zb["face_id"],
                             zb["depth"], colour)
            res.update(adj=adj, colour=colour)
        else:
            layer = np.zeros((scene.height, scene.width, 6))
            layer[..., 5] = np.inf
        res["layer"] = layer
        dm = aa_tile_dmax(cam, dm, layer)
        res["tile_dmax_aa"] = dm
    off, ids, cq = tile_lists(cam, pg["rec"], pg["rect"], order, tiles,
                              tile_dmax=dm if cull else None, softness=scene.softness)
    res["lists_pre"] = (off, ids, cq)
    if cull:
        off2, ids2 = apply_cull(off, ids, cq)
    else:
        off2, ids2 = off, ids
    res["lists"] = (off2, ids2)
    rec64 = pg["rec"].astype(np.float64)
    g = None
    if backward:
        g = grads if grads is not None else scene.grads[view_index]
    comp = composite(cam, mref, rec64, tiles, off2, ids2, zb["face_id"], zb["depth"],
                     bg=scene.bg, softness=scene.softness, grads=g, layer=layer)
    res["comp"] = comp
    return res


# ---------------------------------------------------------------------------
# analytic edge antialiasing (antialias.c)
# ---------------------------------------------------------------------------

def edge_adjacency(faces) -> np.ndarray:
    """[3][F] int32: for edge k of face f (corner k+1 -> k+2) the one other face with
    the same two vertex indices, -1 if none, -2 if several."""
    faces = _c(faces, np.int32)
    F = faces.shape[1]
    adj = np.zeros((3, max(F, 1)), np.int32)
    lib().oc_edge_adjacency(F, _p(faces), _p(adj))
    return adj[:, :F]


def _aa_args(cam, vs, faces, mask, adj, face_id, depth, colour):
    vs = _c(vs, np.float64)
    faces = _c(faces, np.int32)
    mask = _c(mask, np.uint8)
    adj = _c(adj, np.int32)
    face_id = _c(face_id, np.int32)
    depth = _c(depth, np.float32)
    colour = _c(colour, np.float64)
    return vs, faces, mask, adj, face_id, depth, colour


def antialias(cam: Camera, vs, faces, mask, adj, face_id, depth, colour, raw: bool = False):
    """Antialiased mesh layer [H][W][6] = (M_rgb, M_D premultiplied, a_m, D_split) from
    the z-buffer (face_id, fp32 depth), the surface colour at covered pixels
    (colour [H][W][3]) and the screen vertices vs [3][V] (fp64; the fp32 buffer
    upcast).  raw=True also returns [H][W][6] (w_self, w_left, w_right, w_up,
    w_down, raw coverage)."""
    H, W = cam.height, cam.width
    args = _aa_args(cam, vs, faces, mask, adj, face_id, depth, colour)
    vs, faces = args[0], args[1]
    layer = np.zeros((H, W, 6))
    rw = np.zeros((H, W, 6)) if raw else None
    lib().oc_antialias(C.byref(cam), vs.shape[1], faces.shape[1], *(_p(x) for x in args), _p(layer), _p(rw))
    return (layer, rw) if raw else layer


aa_layer = antialias  # the name render_view's flag shadows


def antialias_bwd(cam: Camera, vs, faces, mask, adj, face_id, depth, colour, g_layer) -> dict:
    """Reverse mode of ``antialias``: dL/d(colour) [H][W][3], dL/dD [H][W] (at covered
    pixels' own centres) and dL/d(u, v) of the screen vertices [2][V]."""
    H, W = cam.height, cam.width
    args = _aa_args(cam, vs, faces, mask, adj, face_id, depth, colour)
    vs, faces = args[0], args[1]
    V = vs.shape[1]
    out = {"colour": np.zeros((H, W, 3)), "depth": np.zeros((H, W)), "vs": np.zeros((2, max(V, 1)))}
    g_layer = _c(g_layer, np.float64)
    lib().oc_antialias_bwd(C.byref(cam), V, faces.shape[1], *(_p(x) for x in args), _p(g_layer),
                           _p(out["colour"]), _p(out["depth"]), _p(out["vs"]))
    out["vs"] = out["vs"][:, :V]
    return out


def surface_colours(meshref: "MeshRef", face_id) -> np.ndarray:
    """[H][W][3] surface colour c at covered pixels (0 elsewhere)."""
    fid = np.asarray(face_id).reshape(-1)
    H, W = face_id.shape
    pix = np.nonzero(fid >= 0)[0].astype(np.int32)
    col = np.zeros((H * W, 3))
    if len(pix):
        cm, _ = shade_pixels(meshref, pix, fid[pix])
        col[pix] = cm
    return col.reshape(H, W, 3)


def aa_tile_dmax(cam: Camera, tile_dmax, layer) -> np.ndarray:
    """The cull bound with antialiasing: +inf on every tile that holds a pixel with
    coverage below 1 (there the back layer is visible)."""
    TX, TY, T = n_tiles(cam)
    H, W = cam.height, cam.width
    dm = np.array(tile_dmax, np.float32).copy()
    low = np.zeros((TY * 16, TX * 16), bool)
    low[:H, :W] = layer[..., 4] < 1.0
    part = low.reshape(TY, 16, TX, 16).any(axis=(1, 3)).reshape(-1)
    dm[part] = np.inf
    return dm


def vscreen_bwd(cam: Camera, mesh: "MeshB64", g_vs) -> np.ndarray:
    """dL/d(world vertex) [3][V] from dL/d(u, v) [2][V] through the fp64 projection."""
    g_vs = _c(g_vs, np.float64)
    out = np.zeros((3, mesh.struct.V))
    lib().oc_vscreen_bwd(C.byref(cam), C.byref(mesh.struct), _p(g_vs), _p(out))
    return out


# ---------------------------------------------------------------------------
# projection backward (project_bwd.c)
# ---------------------------------------------------------------------------

def _sh_planes(sh_degree: int) -> int:
    return 1 if sh_degree < 0 else (sh_degree + 1) ** 2


def project_f64(cam: Camera, means, quats, scales, opacity, sh, sh_degree) -> np.ndarray:
    """fp64 records [N][13] from fp64 inputs (same formulas as project_gaussians)."""
    means, quats, scales = _c(means, np.float64), _c(quats, np.float64), _c(scales, np.float64)
    opacity, sh = _c(opacity, np.float64), _c(sh, np.float64)
    N = means.shape[1]
    out = np.zeros((N, NREC), np.float64)
    lib().oc_project_f64(C.byref(cam), N, _p(means), _p(quats), _p(scales), _p(opacity), _p(sh),
                         int(sh_degree), _p(out))
    return out


def project_bwd(cam: Camera, means, quats, scales, sh, sh_degree, listed, g_rec) -> dict:
    """Gradients of sum(g_rec * records) with respect to the projection inputs (fp64).
    Returns means [3][N], quats [4][N], scales [3][N], opacity [N], sh [K][3][N]."""
    means, quats, scales = _c(means, np.float64), _c(quats, np.float64), _c(scales, np.float64)
    sh = _c(sh, np.float64)
    listed = _c(listed, np.int32)
    g_rec = _c(g_rec, np.float64)
    N = means.shape[1]
    K = _sh_planes(sh_degree)
    out = {"means": np.zeros((3, N)), "quats": np.zeros((4, N)), "scales": np.zeros((3, N)),
           "opacity": np.zeros(N), "sh": np.zeros((K, 3, N))}
    lib().oc_project_bwd(C.byref(cam), N, _p(means), _p(quats), _p(scales), _p(sh), int(sh_degree), _p(listed),
                         _p(g_rec), _p(out["means"]), _p(out["quats"]), _p(out["scales"]), _p(out["opacity"]),
                         _p(out["sh"]))
    return out


# ---------------------------------------------------------------------------
# mesh-side backward (mesh_bwd.c)
# ---------------------------------------------------------------------------

def light_vector(light) -> Optional[np.ndarray]:
    """pos, ambient, diffuse, specular, shininess as 13 fp64 values (None: unlit)."""
    if light is None:
        return None
    return np.concatenate([np.asarray(light[k], np.float64).reshape(-1)
                           for k in ("pos", "ambient", "diffuse", "specular", "shininess")])


class MeshB64:
    """fp64 copies of a mesh's arrays (overridable for finite differences)."""

    def __init__(self, scene, verts=None, vcolor=None, vnormal=None, uv=None, tex=None, light=None):
        def f64(a):
            return None if a is None else np.ascontiguousarray(a, np.float64)
        self.verts = f64(scene.verts if verts is None else verts)
        self.faces = np.ascontiguousarray(scene.faces, np.int32)
        self.vcolor = f64(scene.vcolor if vcolor is None else vcolor)
        self.vnormal = f64(scene.vnormal if vnormal is None else vnormal)
        self.uv = f64(scene.uv if uv is None else uv)
        self.faces_uv = None if scene.faces_uv is None else np.ascontiguousarray(scene.faces_uv, np.int32)
        self.tex = f64(scene.texture if tex is None else tex)
        self.light = light_vector(scene.light) if light is None else f64(light)
        if self.vnormal is None:
            self.light = None
        m = MeshB()
        m.V, m.F = self.verts.shape[1], self.faces.shape[1]
        m.Vt = 0 if self.uv is None else self.uv.shape[1]
        m.S = 0 if self.tex is None else self.tex.shape[0]
        m.verts, m.faces = _p(self.verts), _p(self.faces)
        m.vcolor, m.vnormal, m.uv = _p(self.vcolor), _p(self.vnormal), _p(self.uv)
        m.faces_uv, m.tex, m.light = _p(self.faces_uv), _p(self.tex), _p(self.light)
        self.struct = m


def mesh_fwd64(cam: Camera, mesh: MeshB64, pix, face):
    """c_m [n][3] and D [n] at the given pixels, each covered by the given face."""
    pix, face = _c(pix, np.int32), _c(face, np.int32)
    n = len(pix)
    cm, D = np.zeros((n, 3)), np.zeros(n)
    lib().oc_mesh_fwd64(C.byref(cam), C.byref(mesh.struct), n, _p(pix), _p(face), _p(cm), _p(D))
    return cm, D


def mesh_bwd(cam: Camera, mesh: MeshB64, pix, face, g_cm=None, g_D=None) -> dict:
    """Gradients of sum(g_cm * c_m) + sum(g_D * D) with respect to the mesh inputs."""
    pix, face = _c(pix, np.int32), _c(face, np.int32)
    n = len(pix)
    m = mesh.struct
    out = {"verts": np.zeros((3, m.V)), "vcolor": np.zeros((3, m.V)), "vnormal": np.zeros((3, m.V)),
           "uv": np.zeros((2, max(m.Vt, 1))), "tex": np.zeros((max(m.S, 1), max(m.S, 1), 3)),
           "light": np.zeros(13)}
    lib().oc_mesh_bwd(C.byref(cam), C.byref(m), n, _p(pix), _p(face), _p(_c(g_cm, np.float64)),
                      _p(_c(g_D, np.float64)), _p(out["verts"]), _p(out["vcolor"]), _p(out["vnormal"]),
                      _p(out["uv"]), _p(out["tex"]), _p(out["light"]))
    return out
