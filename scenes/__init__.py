"""Seeded synthetic inputs for the hybrid mesh + Gaussian tile rasterizer.

This module only *draws inputs*: camera poses, meshes, Gaussians, textures and
upstream gradients.  It holds none of the rendering arithmetic (no projection,
rasterization, compositing or shading), so both the CPU oracle and the HIP path
can consume the same arrays without sharing any of the method's code.

Every array is returned in the layout the library boundary takes: structure of
arrays, ``[k][N]`` = ``k`` contiguous planes of ``N`` values, C-contiguous,
float32 / int32 / uint8.

Workloads (gmesh README "Design Details" and "Benchmark"; DiffSoup abstract):

* ``c1``  64x64, 200 random triangles, 500 Gaussians (RGB colours).
* ``c2``  512x512, subdivision-4 icosphere (5120 faces), 100k Gaussians in a shell.
* ``c3``  1920x1080, 200k-face displaced geodesic sphere with normals and a Phong
  point light, 1M Gaussians with degree-3 SH.
* ``c4``  800x800, 4096-triangle soup with stochastic binary masks and a
  1024^2 mip-mapped texture, 16 views, no Gaussians.
* ``c5``  1920x1080, four displaced spheres (499,280 faces), 3M Gaussians with
  degree-3 SH, 4 views.

All draws use ``numpy.random.default_rng(seed)`` (PCG64) in fp64, in the order
written below, and are cast to fp32 at the end.  Opacity is drawn as a logit and
passed through a sigmoid, scales as log-scales passed through exp: the boundary
takes activated opacity and linear scales.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = ["Scene", "View", "make_scene", "CONFIGS", "icosphere", "geodesic_sphere",
           "look_at_y", "upstream_grads"]

CONFIGS = ("c1", "c2", "c3", "c4", "c5")


@dataclass
class View:
    """World->camera pose: x_c = R x_w + t (row-major R), OpenCV axes."""
    R: np.ndarray  # (9,) float32 row-major
    t: np.ndarray  # (3,) float32


@dataclass
class Scene:
    name: str
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    views: List[View]
    near_z: float = 0.01
    # mesh (SoA planes)
    verts: Optional[np.ndarray] = None      # [3][V] f32
    faces: Optional[np.ndarray] = None      # [3][F] i32
    vcolor: Optional[np.ndarray] = None     # [3][V] f32
    vnormal: Optional[np.ndarray] = None    # [3][V] f32
    uv: Optional[np.ndarray] = None         # [2][Vt] f32
    faces_uv: Optional[np.ndarray] = None   # [3][F] i32
    texture: Optional[np.ndarray] = None    # [S][S][3] f32 (HWC)
    face_mask: Optional[np.ndarray] = None  # [F] u8
    light: Optional[Dict[str, np.ndarray]] = None  # pos, ambient, diffuse, specular, shininess
    # Gaussians (SoA planes)
    means: np.ndarray = field(default_factory=lambda: np.zeros((3, 0), np.float32))
    quats: np.ndarray = field(default_factory=lambda: np.zeros((4, 0), np.float32))
    scales: np.ndarray = field(default_factory=lambda: np.zeros((3, 0), np.float32))
    opacity: np.ndarray = field(default_factory=lambda: np.zeros((0,), np.float32))
    sh: np.ndarray = field(default_factory=lambda: np.zeros((1, 3, 0), np.float32))
    sh_degree: int = -1        # -1: ``sh`` holds plain RGB in [1][3][N]
    bg: tuple = (1.0, 1.0, 1.0)
    softness: float = 1.0
    # upstream gradients, one dict per view (filled lazily by upstream_grads)
    grads: List[Dict[str, np.ndarray]] = field(default_factory=list)

    @property
    def V(self) -> int:
        return 0 if self.verts is None else int(self.verts.shape[1])

    @property
    def F(self) -> int:
        return 0 if self.faces is None else int(self.faces.shape[1])

    @property
    def N(self) -> int:
        return int(self.means.shape[1])

    @property
    def tiles_x(self) -> int:
        return (self.width + 15) // 16

    @property
    def tiles_y(self) -> int:
        return (self.height + 15) // 16


# ----------------------------------------------------------------------------
# geometry helpers (input construction only)
# ----------------------------------------------------------------------------

def _icosahedron():
    p = (1.0 + math.sqrt(5.0)) / 2.0
    v = np.array([[-1, p, 0], [1, p, 0], [-1, -p, 0], [1, -p, 0],
                  [0, -1, p], [0, 1, p], [0, -1, -p], [0, 1, -p],
                  [p, 0, -1], [p, 0, 1], [-p, 0, -1], [-p, 0, 1]], dtype=np.float64)
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    f = np.array([[0, 11, 5], [0, 5, 1], [0, 1, 7], [0, 7, 10], [0, 10, 11],
                  [1, 5, 9], [5, 11, 4], [11, 10, 2], [10, 7, 6], [7, 1, 8],
                  [3, 9, 4], [3, 4, 2], [3, 2, 6], [3, 6, 8], [3, 8, 9],
                  [4, 9, 5], [2, 4, 11], [6, 2, 10], [8, 6, 7], [9, 8, 1]], dtype=np.int64)
    return v, f


def _orient_outward(v: np.ndarray, f: np.ndarray) -> np.ndarray:
    """Swap two corners of every face whose normal points to the sphere centre."""
    c = v.mean(axis=0)
    a, b, d = v[f[:, 0]], v[f[:, 1]], v[f[:, 2]]
    n = np.cross(b - a, d - a)
    flip = np.einsum("ij,ij->i", n, (a + b + d) / 3.0 - c) < 0
    f = f.copy()
    f[flip, 1], f[flip, 2] = f[flip, 2].copy(), f[flip, 1].copy()
    return f


def icosphere(subdiv: int):
    """Icosahedron with ``subdiv`` rounds of midpoint subdivision, re-projected to the
    unit sphere after every round.  subdiv=4 -> 2562 vertices, 5120 faces."""
    v, f = _icosahedron()
    verts = [tuple(x) for x in v]
    faces = f.tolist()
    for _ in range(subdiv):
        cache = {}
        vlist = verts

        def mid(a, b):
            key = (a, b) if a < b else (b, a)
            if key in cache:
                return cache[key]
            m = np.array(vlist[a]) + np.array(vlist[b])
            m /= np.linalg.norm(m)
            vlist.append(tuple(m))
            cache[key] = len(vlist) - 1
            return cache[key]

        nf = []
        for a, b, c in faces:
            ab, bc, ca = mid(a, b), mid(b, c), mid(c, a)
            nf += [[a, ab, ca], [b, bc, ab], [c, ca, bc], [ab, bc, ca]]
        faces = nf
    v = np.array(verts, dtype=np.float64)
    f = np.array(faces, dtype=np.int64)
    return v, _orient_outward(v, f)


def geodesic_sphere(freq: int):
    """Class-I geodesic sphere: every icosahedron face split into freq^2 triangles
    on a barycentric grid, grid points pushed to the unit sphere.
    V = 10 freq^2 + 2, F = 20 freq^2."""
    iv, ifa = _icosahedron()
    index: Dict[tuple, int] = {}
    pts: List[np.ndarray] = []

    def point(face, i, j, k):
        # canonical key: the (corner, weight) pairs with non-zero weight, sorted
        key = tuple(sorted((c, w) for c, w in zip(face, (i, j, k)) if w > 0))
        got = index.get(key)
        if got is not None:
            return got
        p = np.zeros(3)
        for c, w in key:
            p = p + iv[c] * (w / freq)
        p /= np.linalg.norm(p)
        index[key] = len(pts)
        pts.append(p)
        return index[key]

    faces = []
    for face in ifa.tolist():
        a, b, c = face
        grid = {}
        for i in range(freq + 1):
            for j in range(freq + 1 - i):
                k = freq - i - j
                grid[(i, j)] = point((a, b, c), i, j, k)
        for i in range(freq):
            for j in range(freq - i):
                faces.append([grid[(i, j)], grid[(i + 1, j)], grid[(i, j + 1)]])
                if i + j + 1 < freq:
                    faces.append([grid[(i + 1, j)], grid[(i + 1, j + 1)], grid[(i, j + 1)]])
    v = np.array(pts, dtype=np.float64)
    f = np.array(faces, dtype=np.int64)
    return v, _orient_outward(v, f)


def _vertex_normals(v: np.ndarray, f: np.ndarray) -> np.ndarray:
    """Normalized area-weighted sum of incident face normals (input attribute)."""
    a, b, c = v[f[:, 0]], v[f[:, 1]], v[f[:, 2]]
    fn = np.cross(b - a, c - a)
    n = np.zeros_like(v)
    for k in range(3):
        np.add.at(n, f[:, k], fn)
    n /= np.maximum(np.linalg.norm(n, axis=1, keepdims=True), 1e-30)
    return n


def _rot_y(phi: float) -> np.ndarray:
    c, s = math.cos(phi), math.sin(phi)
    return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])


def look_at_y(theta: float, radius: float, zc: float) -> View:
    """Camera on a circle of ``radius`` in the xz plane around (0, 0, zc), looking at
    (0, 0, zc); camera-to-world rotation R_y(-theta); theta = 0 is the identity pose."""
    center = np.array([radius * math.sin(theta), 0.0, zc - radius * math.cos(theta)])
    r_cw = _rot_y(-theta)
    r_wc = r_cw.T
    t = -r_wc @ center
    return View(R=r_wc.reshape(-1).astype(np.float32), t=t.astype(np.float32))


def _identity_view() -> View:
    return View(R=np.eye(3, dtype=np.float32).reshape(-1), t=np.zeros(3, np.float32))


def _unit_quats(rng, n):
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _planes(a: np.ndarray, dtype) -> np.ndarray:
    """[N][k] -> [k][N] contiguous planes."""
    return np.ascontiguousarray(np.asarray(a).T, dtype=dtype)


def _shell_points(rng, n, center, r0, r1):
    d = rng.normal(size=(n, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    r = rng.uniform(r0 ** 3, r1 ** 3, size=n) ** (1.0 / 3.0)
    return center[None, :] + d * r[:, None]


def upstream_grads(scene: Scene, view_index: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """N(0,1) upstream gradients for rgb [H][W][3], depth [H][W] and alpha [H][W]."""
    rng = np.random.default_rng([seed, 1000 + view_index])
    H, W = scene.height, scene.width
    return {
        "rgb": rng.normal(size=(H, W, 3)).astype(np.float32),
        "depth": rng.normal(size=(H, W)).astype(np.float32),
        "alpha": rng.normal(size=(H, W)).astype(np.float32),
    }


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def _c1(seed):
    rng = np.random.default_rng(seed)
    W = H = 64
    u = rng.uniform(size=(200, 3, 3))
    tri = np.empty_like(u)
    tri[..., 0] = -1.0 + 2.0 * u[..., 0]
    tri[..., 1] = -1.0 + 2.0 * u[..., 1]
    tri[..., 2] = 2.0 + 4.0 * u[..., 2]
    vcol = rng.uniform(size=(200, 3, 3))
    um = rng.uniform(size=(500, 3))
    means = np.stack([-1 + 2 * um[:, 0], -1 + 2 * um[:, 1], 2 + 4 * um[:, 2]], axis=1)
    logs = rng.normal(-3.0, 0.5, size=(500, 3))
    quats = _unit_quats(rng, 500)
    logits = rng.normal(size=500)
    rgb = rng.uniform(size=(500, 3))
    verts = tri.reshape(-1, 3)
    faces = np.arange(600, dtype=np.int64).reshape(200, 3)
    return Scene(
        name="c1", width=W, height=H, fx=64.0, fy=64.0, cx=32.0, cy=32.0,
        views=[_identity_view()],
        verts=_planes(verts, np.float32), faces=_planes(faces, np.int32),
        vcolor=_planes(vcol.reshape(-1, 3), np.float32),
        means=_planes(means, np.float32), quats=_planes(quats, np.float32),
        scales=_planes(np.exp(logs), np.float32),
        opacity=_sigmoid(logits).astype(np.float32),
        sh=np.ascontiguousarray(rgb.T[None], dtype=np.float32), sh_degree=-1)


def _c2(seed):
    rng = np.random.default_rng(seed)
    v, f = icosphere(4)
    center = np.array([0.0, 0.0, 4.0])
    verts = v * 1.0 + center
    vcol = rng.uniform(size=(v.shape[0], 3))
    n = 100_000
    means = _shell_points(rng, n, center, 0.8, 1.3)
    logs = rng.normal(-4.0, 0.5, size=(n, 3))
    quats = _unit_quats(rng, n)
    logits = rng.normal(size=n)
    rgb = rng.uniform(size=(n, 3))
    return Scene(
        name="c2", width=512, height=512, fx=512.0, fy=512.0, cx=256.0, cy=256.0,
        views=[_identity_view()],
        verts=_planes(verts, np.float32), faces=_planes(f, np.int32),
        vcolor=_planes(vcol, np.float32),
        means=_planes(means, np.float32), quats=_planes(quats, np.float32),
        scales=_planes(np.exp(logs), np.float32),
        opacity=_sigmoid(logits).astype(np.float32),
        sh=np.ascontiguousarray(rgb.T[None], dtype=np.float32), sh_degree=-1)


def _phong_light():
    return {"pos": np.array([2.0, -2.0, 0.0], np.float32),
            "ambient": np.full(3, 0.1, np.float32),
            "diffuse": np.full(3, 0.8, np.float32),
            "specular": np.full(3, 0.3, np.float32),
            "shininess": np.float32(32.0)}


def _displaced_sphere(rng, freq, radius, center):
    v, f = geodesic_sphere(freq)
    disp = rng.normal(0.0, 0.02, size=v.shape[0])
    verts = center[None, :] + v * (radius + disp)[:, None]
    normals = _vertex_normals(verts, f)
    return verts, f, normals


def _sh3(rng, n):
    # [16][3][N] planes, coefficient-major
    return rng.normal(0.0, 0.2, size=(16, 3, n))


def _c3(seed):
    rng = np.random.default_rng(seed)
    center = np.array([0.0, 0.0, 4.0])
    verts, f, normals = _displaced_sphere(rng, 100, 1.0, center)
    vcol = rng.uniform(size=(verts.shape[0], 3))
    n = 1_000_000
    means = _shell_points(rng, n, center, 0.8, 1.3)
    logs = rng.normal(-4.0, 0.5, size=(n, 3))
    quats = _unit_quats(rng, n)
    logits = rng.normal(size=n)
    sh = _sh3(rng, n)
    return Scene(
        name="c3", width=1920, height=1080, fx=1920.0, fy=1920.0, cx=960.0, cy=540.0,
        views=[_identity_view()],
        verts=_planes(verts, np.float32), faces=_planes(f, np.int32),
        vcolor=_planes(vcol, np.float32), vnormal=_planes(normals, np.float32),
        light=_phong_light(),
        means=_planes(means, np.float32), quats=_planes(quats, np.float32),
        scales=_planes(np.exp(logs), np.float32),
        opacity=_sigmoid(logits).astype(np.float32),
        sh=sh.astype(np.float32), sh_degree=3)


def _equilateral_soup(rng, n, edge):
    cen = np.empty((n, 3))
    u = rng.uniform(size=(n, 3))
    cen[:, 0] = -0.5 + u[:, 0]
    cen[:, 1] = -0.5 + u[:, 1]
    cen[:, 2] = 2.5 + u[:, 2]
    q = _unit_quats(rng, n)
    w, x, y, z = q[:, 0], q[:, 1], q[:, 2], q[:, 3]
    rot = np.stack([
        np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
        np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
        np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], 1)
    rad = edge / math.sqrt(3.0)
    ang = np.array([math.pi / 2, math.pi / 2 + 2 * math.pi / 3, math.pi / 2 + 4 * math.pi / 3])
    local = np.stack([rad * np.cos(ang), rad * np.sin(ang), np.zeros(3)], axis=1)  # (3,3)
    tri = cen[:, None, :] + np.einsum("nij,kj->nki", rot, local)
    return tri


def _c4(seed):
    rng = np.random.default_rng(seed)
    n = 4096
    tri = _equilateral_soup(rng, n, 0.05)
    uvs = rng.uniform(size=(n, 3, 2))
    tex = rng.uniform(size=(1024, 1024, 3))
    logits = rng.normal(size=n)
    mask = (rng.uniform(size=n) < _sigmoid(logits)).astype(np.uint8)
    faces = np.arange(3 * n, dtype=np.int64).reshape(n, 3)
    views = [look_at_y(2.0 * math.pi * k / 16.0, 3.0, 3.0) for k in range(16)]
    return Scene(
        name="c4", width=800, height=800, fx=800.0, fy=800.0, cx=400.0, cy=400.0,
        views=views,
        verts=_planes(tri.reshape(-1, 3), np.float32), faces=_planes(faces, np.int32),
        uv=_planes(uvs.reshape(-1, 2), np.float32), faces_uv=_planes(faces, np.int32),
        texture=np.ascontiguousarray(tex, dtype=np.float32), face_mask=mask)


def _c5(seed):
    rng = np.random.default_rng(seed)
    centers = [np.array([sx * 0.55, sy * 0.55, 4.0]) for sx in (-1, 1) for sy in (-1, 1)]
    vs, fs, ns = [], [], []
    off = 0
    for c in centers:
        v, f, nrm = _displaced_sphere(rng, 79, 0.5, c)
        vs.append(v)
        fs.append(f + off)
        ns.append(nrm)
        off += v.shape[0]
    verts = np.concatenate(vs)
    faces = np.concatenate(fs)
    normals = np.concatenate(ns)
    vcol = rng.uniform(size=(verts.shape[0], 3))
    n = 3_000_000
    n_surf = (n * 6) // 10
    n_box = n - n_surf
    which = rng.integers(0, 4, size=n_surf)
    d = rng.normal(size=(n_surf, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    r = 0.5 + rng.uniform(-0.05, 0.05, size=n_surf)
    surf = np.stack(centers)[which] + d * r[:, None]
    lo, hi = verts.min(axis=0), verts.max(axis=0)
    box = lo[None, :] + rng.uniform(size=(n_box, 3)) * (hi - lo)[None, :]
    means = np.concatenate([surf, box])
    logs = rng.normal(-4.5, 0.7, size=(n, 3))
    quats = _unit_quats(rng, n)
    logits = rng.normal(0.0, 1.5, size=n)
    sh = _sh3(rng, n)
    views = [look_at_y(th, 4.0, 4.0) for th in (0.0, math.pi / 2, math.pi, 3 * math.pi / 2)]
    return Scene(
        name="c5", width=1920, height=1080, fx=1920.0, fy=1920.0, cx=960.0, cy=540.0,
        views=views,
        verts=_planes(verts, np.float32), faces=_planes(faces, np.int32),
        vcolor=_planes(vcol, np.float32), vnormal=_planes(normals, np.float32),
        light=_phong_light(),
        means=_planes(means, np.float32), quats=_planes(quats, np.float32),
        scales=_planes(np.exp(logs), np.float32),
        opacity=_sigmoid(logits).astype(np.float32),
        sh=sh.astype(np.float32), sh_degree=3)


_MAKERS = {"c1": _c1, "c2": _c2, "c3": _c3, "c4": _c4, "c5": _c5}


def make_scene(name: str, seed: int = 0) -> Scene:
    """Build workload ``name`` (one of CONFIGS) with PCG64 seed ``seed``."""
    s = _MAKERS[name](seed)
    s.grads = [upstream_grads(s, k, seed) for k in range(len(s.views))]
    return s
