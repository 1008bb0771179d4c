"""Small hand-built scenes for pins and parity (inputs only, no method arithmetic)."""
import math

import numpy as np

import scenes


def identity_view():
    return scenes.View(R=np.eye(3, dtype=np.float32).reshape(-1), t=np.zeros(3, np.float32))


def empty_scene(width, height, fx, fy, cx, cy, views=None, name="tiny"):
    return scenes.Scene(name=name, width=width, height=height, fx=fx, fy=fy, cx=cx, cy=cy,
                        views=views or [identity_view()])


def set_mesh(s, verts, faces, vcolor=None, vnormal=None, mask=None):
    s.verts = np.ascontiguousarray(np.asarray(verts, np.float64).T, np.float32)
    s.faces = np.ascontiguousarray(np.asarray(faces, np.int64).T, np.int32)
    if vcolor is not None:
        s.vcolor = np.ascontiguousarray(np.asarray(vcolor, np.float64).T, np.float32)
    if vnormal is not None:
        s.vnormal = np.ascontiguousarray(np.asarray(vnormal, np.float64).T, np.float32)
    if mask is not None:
        s.face_mask = np.asarray(mask, np.uint8)
    return s


def set_gaussians(s, means, quats, scales, opacity, rgb=None, sh=None, sh_degree=-1):
    n = len(means)
    s.means = np.ascontiguousarray(np.asarray(means, np.float64).T, np.float32)
    s.quats = np.ascontiguousarray(np.asarray(quats, np.float64).T, np.float32)
    s.scales = np.ascontiguousarray(np.asarray(scales, np.float64).T, np.float32)
    s.opacity = np.asarray(opacity, np.float32).reshape(n)
    if sh is not None:
        s.sh = np.ascontiguousarray(sh, np.float32)
        s.sh_degree = sh_degree
    else:
        s.sh = np.ascontiguousarray(np.asarray(rgb, np.float64).T[None], np.float32)
        s.sh_degree = -1
    return s


def random_tiny(seed, n_tri=6, n_gauss=12, size=32, soup=True):
    """Random tiny hybrid scene: triangles and Gaussians in front of an identity camera."""
    rng = np.random.default_rng(seed)
    s = empty_scene(size, size, float(size), float(size), size / 2, size / 2, name="rand%d" % seed)
    tri = np.empty((n_tri, 3, 3))
    tri[..., :2] = rng.uniform(-0.8, 0.8, size=(n_tri, 3, 2))
    tri[..., 2] = rng.uniform(2.0, 4.0, size=(n_tri, 3))
    set_mesh(s, tri.reshape(-1, 3), np.arange(3 * n_tri).reshape(n_tri, 3),
             vcolor=rng.uniform(size=(3 * n_tri, 3)))
    means = np.stack([rng.uniform(-0.6, 0.6, n_gauss), rng.uniform(-0.6, 0.6, n_gauss),
                      rng.uniform(2.0, 4.0, n_gauss)], 1)
    q = rng.normal(size=(n_gauss, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    sc = np.exp(rng.normal(-2.0, 0.4, size=(n_gauss, 3)))
    op = 1.0 / (1.0 + np.exp(-rng.normal(size=n_gauss)))
    set_gaussians(s, means, q, sc, op, rgb=rng.uniform(size=(n_gauss, 3)))
    s.grads = [scenes.upstream_grads(s, 0, seed)]
    return s
