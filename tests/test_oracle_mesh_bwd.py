"""Pins of the oracle's mesh-side backward (oracle/mesh_bwd.c).

Checked against: the shading forward of the main oracle (the fp64 re-evaluation of
c_m and D agrees with it), central finite differences of that fp64 forward for
every input, and closed forms: constant-texture and vertex-colour gradient sums,
the ambient-light gradient, and the invariance of the perspective-correct
barycentrics under a common scaling of the scene about the camera centre.
"""
import numpy as np
import pytest

import oracle
import scenes
import tiny


def _covered(scene, cam):
    vs = oracle.project_vertices(cam, scene.verts)
    zb = oracle.zbuffer(cam, vs, scene.faces, scene.face_mask)
    fid = zb["face_id"].reshape(-1)
    pix = np.nonzero(fid >= 0)[0].astype(np.int32)
    return pix, fid[pix].astype(np.int32), zb, vs


def _lit_scene(seed, n_tri=10, size=48):
    s = tiny.random_tiny(seed, n_tri=n_tri, n_gauss=0, size=size)
    rng = np.random.default_rng(seed)
    nrm = rng.normal(size=(3, s.V))
    nrm[2] = -np.abs(nrm[2]) - 0.5  # facing the camera (which looks down +z)
    s.vnormal = (nrm / np.linalg.norm(nrm, axis=0)).astype(np.float32)
    s.light = {"pos": [0.3, -0.4, 0.5], "ambient": [0.1, 0.15, 0.2], "diffuse": [0.8, 0.7, 0.6],
               "specular": [0.3, 0.25, 0.2], "shininess": 8.0}
    return s


def _textured_scene(seed, S=64, linear=False, size=48):
    s = tiny.random_tiny(seed, n_tri=8, n_gauss=0, size=size)
    rng = np.random.default_rng(seed)
    nc = 3 * 8
    s.uv = np.concatenate([rng.uniform(0.3, 0.7, size=(2, nc))], 0).astype(np.float32)
    # small uv footprints keep the level of detail near the finest levels
    for f in range(8):
        c = rng.uniform(0.3, 0.7, size=2)
        s.uv[:, 3 * f:3 * f + 3] = (c[:, None] + rng.uniform(-0.05, 0.05, size=(2, 3))).astype(np.float32)
    s.faces_uv = s.faces.copy()
    if linear:  # a linear ramp per channel: every pyramid level samples the same function
        x = (np.arange(S) + 0.5) / S
        U, V = np.meshgrid(x, x)  # U varies along columns (u), V along rows (v)
        s.texture = np.stack([0.2 + 0.5 * U, 0.7 - 0.3 * V, 0.1 + 0.2 * U + 0.4 * V], -1).astype(np.float32)
    else:
        s.texture = rng.uniform(size=(S, S, 3)).astype(np.float32)
    s.vcolor = None
    return s


def test_fwd64_matches_main_oracle_shading():
    for s in (_lit_scene(3), _textured_scene(4)):
        cam = oracle.camera(s, 0)
        pix, face, zb, vs = _covered(s, cam)
        mips = oracle.build_mips(s.texture) if s.texture is not None else None
        ref, _ = oracle.shade_pixels(oracle.MeshRef(cam, s, vs, mips=mips), pix, face)
        cm, D = oracle.mesh_fwd64(cam, oracle.MeshB64(s), pix, face)
        np.testing.assert_allclose(cm, ref, atol=2e-4)
        np.testing.assert_allclose(D, zb["depth"].reshape(-1)[pix], rtol=1e-5)


def _fd(cam, s, pix, face, g_cm, g_D, name, arr, idxs, h_rel=1e-6, **over):
    out = []
    for i in idxs:
        a = arr.copy().reshape(-1)
        h = h_rel * max(abs(a[i]), 1.0)
        a[i] += h
        cp, Dp = oracle.mesh_fwd64(cam, oracle.MeshB64(s, **{name: a.reshape(arr.shape)}, **over), pix, face)
        a[i] -= 2 * h
        cm_, Dm = oracle.mesh_fwd64(cam, oracle.MeshB64(s, **{name: a.reshape(arr.shape)}, **over), pix, face)
        out.append((np.sum((cp - cm_) * g_cm) + np.sum((Dp - Dm) * g_D)) / (2 * h))
    return np.array(out)


def _check(fd, an, scale):
    assert np.all(np.abs(fd - an) <= 1e-5 * (np.abs(an) + scale)), np.max(np.abs(fd - an) / (np.abs(an) + scale))


@pytest.mark.parametrize("seed", [11, 12])
def test_fd_lit_vertex_colours(seed):
    s = _lit_scene(seed)
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    rng = np.random.default_rng(seed)
    g_cm, g_D = rng.normal(size=(len(pix), 3)), rng.normal(size=len(pix))
    m = oracle.MeshB64(s)
    g = oracle.mesh_bwd(cam, m, pix, face, g_cm, g_D)
    for name, arr in (("verts", m.verts), ("vcolor", m.vcolor), ("vnormal", m.vnormal), ("light", m.light)):
        an = g[name].reshape(-1)
        idx = np.arange(an.size) if an.size <= 40 else rng.choice(an.size, 40, replace=False)
        fd = _fd(cam, s, pix, face, g_cm, g_D, name, arr, idx)
        _check(fd, an[idx], np.sqrt(np.mean(an ** 2)) + 1e-12)


def test_fd_texture_texels_and_uv():
    s = _textured_scene(21)
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    rng = np.random.default_rng(21)
    g_cm, g_D = rng.normal(size=(len(pix), 3)), np.zeros(len(pix))
    m = oracle.MeshB64(s)
    g = oracle.mesh_bwd(cam, m, pix, face, g_cm, g_D)
    an = g["tex"].reshape(-1)
    nz = np.nonzero(an)[0]
    idx = np.concatenate([rng.choice(nz, 30, replace=False), rng.choice(an.size, 10, replace=False)])
    fd = _fd(cam, s, pix, face, g_cm, g_D, "tex", m.tex, idx)
    _check(fd, an[idx], np.sqrt(np.mean(an[nz] ** 2)))
    # uv and vertex positions on a linear ramp texture (the level of detail, held
    # fixed by the backward, then has no effect on the colour)
    s = _textured_scene(22, linear=True)
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    g_D = rng.normal(size=len(pix))
    g_cm = rng.normal(size=(len(pix), 3))
    m = oracle.MeshB64(s)
    g = oracle.mesh_bwd(cam, m, pix, face, g_cm, g_D)
    for name, arr in (("uv", m.uv), ("verts", m.verts)):
        an = g[name].reshape(-1)
        fd = _fd(cam, s, pix, face, g_cm, g_D, name, arr, np.arange(an.size))
        _check(fd, an, np.sqrt(np.mean(an ** 2)))


def test_constant_texture_and_vertex_colour_sums():
    # constant texture: the pyramid adjoint and the bilinear/trilinear weights keep
    # sums, so the texel gradients add up to the pixel gradients
    s = _textured_scene(31)
    s.texture[:] = 0.4
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    g_cm = np.random.default_rng(1).normal(size=(len(pix), 3))
    g = oracle.mesh_bwd(cam, oracle.MeshB64(s), pix, face, g_cm, None)
    np.testing.assert_allclose(g["tex"].sum((0, 1)), g_cm.sum(0), rtol=1e-10)
    assert np.all(g["uv"] == 0.0)  # a constant texture has no spatial gradient
    # vertex colours, unlit: the barycentrics sum to one
    s = tiny.random_tiny(32, n_tri=10, n_gauss=0, size=48)
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    g_cm = np.random.default_rng(2).normal(size=(len(pix), 3))
    g = oracle.mesh_bwd(cam, oracle.MeshB64(s), pix, face, g_cm, None)
    np.testing.assert_allclose(g["vcolor"].sum(1), g_cm.sum(0), rtol=1e-10)


def test_ambient_light_closed_form():
    # white vertex colours: c = ambient + diffuse max(0, n.l) + specular spec, so
    # dL/d ambient_c = sum over pixels of dL/dc_c
    s = _lit_scene(41)
    s.vcolor = np.ones_like(s.vcolor)
    cam = oracle.camera(s, 0)
    pix, face, _, _ = _covered(s, cam)
    g_cm = np.random.default_rng(3).normal(size=(len(pix), 3))
    g = oracle.mesh_bwd(cam, oracle.MeshB64(s), pix, face, g_cm, None)
    np.testing.assert_allclose(g["light"][3:6], g_cm.sum(0), rtol=1e-10)


def test_scaling_about_the_camera():
    # scaling every vertex by k about the camera centre leaves u, v and the
    # perspective-correct barycentrics unchanged and scales D by k, so for an unlit
    # vertex-coloured mesh sum_v X_v . dL/dX_v = sum_p dL/dD_p D_p
    s = tiny.random_tiny(51, n_tri=10, n_gauss=0, size=48)
    cam = oracle.camera(s, 0)  # identity camera: centre at the origin
    pix, face, _, _ = _covered(s, cam)
    rng = np.random.default_rng(4)
    g_cm, g_D = rng.normal(size=(len(pix), 3)), rng.normal(size=len(pix))
    m = oracle.MeshB64(s)
    g = oracle.mesh_bwd(cam, m, pix, face, g_cm, g_D)
    _, D = oracle.mesh_fwd64(cam, m, pix, face)
    lhs = float(np.sum(m.verts * g["verts"]))
    rhs = float(np.sum(g_D * D))
    assert abs(lhs - rhs) <= 1e-9 * (abs(rhs) + np.abs(m.verts * g["verts"]).sum())
