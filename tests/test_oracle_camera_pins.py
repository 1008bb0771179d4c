"""Pins of the oracle under rotated and translated cameras, and of its Phong shading
off the optical axis.

The gmesh README (Design Details > Mesh rasterizer) puts meshes and Gaussians
through one pinhole camera; the 3DGS projection carries a Gaussian's covariance
into the camera frame with the world-to-camera rotation W (Sigma_c = W Sigma W^T)
and evaluates its colour at the direction from the camera centre C = -W^T t.  The
v1.1 notes of the README shade the mesh with a point light and a specular highlight
that follows the camera.  Each pin below checks the oracle against something other
than itself:

* an fp64 projection built on scipy's quaternion rotation, at the four views of the
  four-sphere workload and at a random camera;
* equivariance: projecting under (W, t) equals projecting Gaussians moved by
  (W, t) beforehand under the identity camera (whose projection the closed forms of
  test_oracle_pins fix);
* the colour at the direction from the camera centre known from the pose's
  construction (not from W and t), with the real spherical harmonics of scipy;
* per-pixel Phong on a quad facing a rotated, translated camera, lit off axis: the
  reflection of the light vector in a fronto-parallel plane is its mirror image in
  that plane, so r.e is written out by hand; Blinn-Phong's value and the value with
  the light left in world coordinates differ from it by far more than the tolerance.
"""
import math

import numpy as np
import pytest

import oracle
import scenes
import tiny

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _rot(ax, ay, az):
    from scipy.spatial.transform import Rotation
    return Rotation.from_euler("xyz", [ax, ay, az]).as_matrix()


def _camera_at(R, centre):
    """World-to-camera (R, t) of a camera at ``centre`` (fp32, as the scenes store them)."""
    R = np.asarray(R, np.float64)
    t = -R @ np.asarray(centre, np.float64)
    return scenes.View(R=R.reshape(-1).astype(np.float32), t=t.astype(np.float32))


def _random_camera(seed, target, dist):
    """A camera with a random orientation looking at ``target`` from ``dist`` away."""
    from scipy.spatial.transform import Rotation
    R = Rotation.random(random_state=seed).as_matrix()
    forward = R.T @ np.array([0.0, 0.0, 1.0])  # the camera's +z axis in world space
    centre = np.asarray(target) - dist * forward
    return _camera_at(R, centre), centre


def _proj_fp64(s, i, view):
    """fp64 projection of Gaussian i from scipy's rotation of its quaternion."""
    from scipy.spatial.transform import Rotation
    q = s.quats[:, i].astype(np.float64)
    Rq = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
    Sig = Rq @ np.diag(s.scales[:, i].astype(np.float64) ** 2) @ Rq.T
    W = view.R.astype(np.float64).reshape(3, 3)
    mc = W @ s.means[:, i].astype(np.float64) + view.t.astype(np.float64)
    Sc = W @ Sig @ W.T
    x, y, z = mc
    J = np.array([[s.fx / z, 0, -s.fx * x / z ** 2], [0, s.fy / z, -s.fy * y / z ** 2], [0, 0, 1.0]])
    Suvz = J @ Sc @ J.T
    Q = np.linalg.inv(Suvz[:2, :2] + 0.3 * np.eye(2))
    k = Suvz[:2, 2]
    g = Q @ k
    return dict(u=s.fx * x / z + s.cx, v=s.fy * y / z + s.cy, Q=Q, z=z, g=g,
                sigma=math.sqrt(max(Suvz[2, 2] - k @ g, 1e-12)))


def _check_fp64(s, view, idx, rec, valid):
    n = 0
    for i in idx:
        if not valid[i]:
            continue
        r = _proj_fp64(s, i, view)
        assert abs(rec[i, 0] - r["u"]) < 2e-4 and abs(rec[i, 1] - r["v"]) < 2e-4, i
        Qs = np.array([[rec[i, 2], rec[i, 3]], [rec[i, 3], rec[i, 4]]])
        assert np.allclose(Qs, r["Q"], rtol=2e-4, atol=1e-6 * np.abs(r["Q"]).max()), i
        assert abs(rec[i, 9] - r["z"]) <= 1e-6 * r["z"], i
        gs = np.abs(r["g"]).max() + 1e-9
        assert np.allclose(rec[i, 10:12], r["g"], rtol=0, atol=2e-3 * gs), i
        assert abs(rec[i, 12] - r["sigma"]) <= 2e-3 * r["sigma"] + 1e-6, i
        assert rec[i, 5] == s.opacity[i]
        n += 1
    return n


@pytest.fixture(scope="module")
def c5():
    return scenes.make_scene("c5")


@pytest.mark.parametrize("view", [1, 2, 3])
def test_projection_fp64_four_sphere_views(c5, view):
    """The rotated and translated views of the four-sphere workload (quarter turns
    around the scene's centre)."""
    s = c5
    idx = np.random.default_rng(view).choice(s.N, 4000, replace=False)
    sub = _subset(s, idx)
    pg = oracle.project_gaussians(oracle.camera(sub, view), sub.means, sub.quats, sub.scales, sub.opacity,
                                  sub.sh, sub.sh_degree)
    assert _check_fp64(sub, sub.views[view], range(sub.N), pg["rec"].astype(np.float64), pg["valid"]) > 1000


def _subset(s, idx):
    """The scene with only Gaussians ``idx`` (inputs only)."""
    return scenes.Scene(**{**s.__dict__, "means": np.ascontiguousarray(s.means[:, idx]),
                           "quats": np.ascontiguousarray(s.quats[:, idx]),
                           "scales": np.ascontiguousarray(s.scales[:, idx]),
                           "opacity": np.ascontiguousarray(s.opacity[idx]),
                           "sh": np.ascontiguousarray(s.sh[..., idx])})


def _random_view_scene(seed):
    """The 512x512 workload's Gaussians seen by a randomly oriented camera 3 units
    from their centre."""
    s = scenes.make_scene("c2")
    v, centre = _random_camera(seed, [0.0, 0.0, 4.0], 3.0)
    return scenes.Scene(**{**s.__dict__, "views": [v]}), centre


@pytest.mark.parametrize("seed", [11, 12])
def test_projection_fp64_random_camera(seed):
    s, _ = _random_view_scene(seed)
    assert abs(np.linalg.det(s.views[0].R.reshape(3, 3).astype(np.float64)) - 1) < 1e-6
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    idx = np.random.default_rng(seed).choice(s.N, 3000, replace=False)
    assert _check_fp64(s, s.views[0], idx, pg["rec"].astype(np.float64), pg["valid"]) > 1000


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_projection_equivariance(seed):
    """Projecting under (W, t) equals projecting the Gaussians moved into the camera
    frame beforehand (mean W mu + t, rotation W R(q)) under the identity camera, up
    to the rounding of the moved inputs to fp32."""
    from scipy.spatial.transform import Rotation
    s, _ = _random_view_scene(seed)
    idx = np.random.default_rng(seed).choice(s.N, 5000, replace=False)
    s = _subset(s, idx)
    W = s.views[0].R.astype(np.float64).reshape(3, 3)
    t = s.views[0].t.astype(np.float64)
    a = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    moved = W @ s.means.astype(np.float64) + t[:, None]
    q = s.quats.astype(np.float64)
    rq = Rotation.from_matrix(W) * Rotation.from_quat(np.stack([q[1], q[2], q[3], q[0]], 1))
    xyzw = rq.as_quat()
    quats = np.stack([xyzw[:, 3], xyzw[:, 0], xyzw[:, 1], xyzw[:, 2]])
    ident = tiny.empty_scene(s.width, s.height, s.fx, s.fy, s.cx, s.cy)
    b = oracle.project_gaussians(oracle.camera(ident), np.ascontiguousarray(moved, np.float32),
                                 np.ascontiguousarray(quats, np.float32), s.scales, s.opacity, s.sh, s.sh_degree)
    ok = a["valid"].astype(bool) & b["valid"].astype(bool)
    assert ok.sum() > 2000 and (a["valid"] != b["valid"]).sum() <= 2
    ra, rb = a["rec"][ok].astype(np.float64), b["rec"][ok].astype(np.float64)
    assert np.abs(ra[:, 0:2] - rb[:, 0:2]).max() < 2e-3  # pixels
    assert np.abs(ra[:, 9] - rb[:, 9]).max() <= 2e-6 * ra[:, 9].max()
    qscale = np.abs(ra[:, 2:5]).max(1)
    assert (np.abs(ra[:, 2:5] - rb[:, 2:5]).max(1) <= 2e-3 * qscale).all()
    gscale = np.abs(ra[:, 10:12]).max(1) + 1e-9
    assert (np.abs(ra[:, 10:12] - rb[:, 10:12]).max(1) <= 2e-2 * gscale).mean() > 0.999
    assert (np.abs(ra[:, 12] - rb[:, 12]) <= 2e-2 * ra[:, 12] + 1e-6).mean() > 0.999


def _real_sh(d, signs):
    """Real spherical harmonics l <= 3 at unit direction d from scipy's complex ones;
    ``signs`` fixes each function's sign (the splatting convention)."""
    from scipy.special import sph_harm_y
    th, ph = math.acos(max(-1.0, min(1.0, d[2]))), math.atan2(d[1], d[0])
    Y = np.zeros(16)
    for l in range(4):
        for m in range(-l, l + 1):
            if m == 0:
                v = sph_harm_y(l, 0, th, ph).real
            elif m > 0:
                v = math.sqrt(2) * sph_harm_y(l, m, th, ph).real
            else:
                v = math.sqrt(2) * sph_harm_y(l, -m, th, ph).imag
            Y[l * l + l + m] = signs[l * l + l + m] * v
    return Y


def _sh_signs():
    """Sign of each oracle basis function relative to scipy's real form, read at one
    generic direction (the sign convention itself is pinned in test_oracle_pins)."""
    d = np.array([0.3, -0.5, 0.81])
    d /= np.linalg.norm(d)
    Y = oracle.sh_basis(*d)
    ref = _real_sh(d, np.ones(16))
    return np.sign(Y / ref)


def _check_colour(s, view_index, centre, idx):
    signs = _sh_signs()
    pg = oracle.project_gaussians(oracle.camera(s, view_index), s.means, s.quats, s.scales, s.opacity, s.sh,
                                  s.sh_degree)
    worst = 0.0
    for i in idx:
        d = s.means[:, i].astype(np.float64) - np.asarray(centre, np.float64)
        d /= np.linalg.norm(d)
        Y = _real_sh(d, signs)
        want = np.maximum(Y @ s.sh[:, :, i].astype(np.float64) + 0.5, 0.0)
        worst = max(worst, float(np.abs(pg["rgb64"][i] - want).max()))
    assert worst < 1e-5, worst
    return worst


@pytest.mark.parametrize("view", [1, 3])
def test_sh_colour_direction_four_sphere_views(c5, view):
    """Colour at the direction from the camera centre of the pose's construction:
    (4 sin theta, 0, 4 - 4 cos theta), theta = view * pi / 2."""
    th = view * math.pi / 2
    centre = [4 * math.sin(th), 0.0, 4 - 4 * math.cos(th)]
    sub = _subset(c5, np.random.default_rng(view).choice(c5.N, 300, replace=False))
    _check_colour(sub, view, centre, range(sub.N))


@pytest.mark.parametrize("seed", [11, 12])
def test_sh_colour_direction_random_camera(seed):
    s, centre = _random_view_scene(seed)
    rng = np.random.default_rng(seed)
    s = _subset(s, rng.choice(s.N, 300, replace=False))
    s.sh = rng.normal(0.0, 0.3, size=(16, 3, s.N)).astype(np.float32)
    s.sh_degree = 3
    _check_colour(s, 0, centre, range(s.N))


# ---------------------------------------------------------------------------
# Phong off the optical axis, rotated and translated camera
# ---------------------------------------------------------------------------

def _phong_scene(light_cam, base, z0=2.0, size=48, f=48.0):
    """A quad at camera depth z0 facing the camera (normal (0, 0, -1) in camera
    space), seen by a rotated, translated camera; the light is placed at camera-space
    position ``light_cam``.  Returns the scene and the camera's (W, t)."""
    W = _rot(0.2, -0.45, 0.1)
    centre = np.array([0.7, -0.3, 0.5])
    view = _camera_at(W, centre)
    Wf = view.R.astype(np.float64).reshape(3, 3)
    tf = view.t.astype(np.float64)
    s = tiny.empty_scene(size, size, f, f, size / 2, size / 2, views=[view])
    h = 5.0
    cam_pts = np.array([[-h, -h, z0], [h, -h, z0], [h, h, z0], [-h, h, z0]])
    world = (Wf.T @ (cam_pts.T - tf[:, None])).T
    nw = Wf.T @ np.array([0.0, 0.0, -1.0])
    tiny.set_mesh(s, world, [[0, 1, 2], [0, 2, 3]], vcolor=[base] * 4, vnormal=[nw] * 4)
    Lw = Wf.T @ (np.asarray(light_cam, np.float64) - tf)
    s.light = {"pos": Lw.astype(np.float32), "ambient": np.full(3, 0.1, np.float32),
               "diffuse": np.full(3, 0.8, np.float32), "specular": np.full(3, 0.3, np.float32),
               "shininess": np.float32(32.0)}
    return s, Wf, tf


def test_phong_off_axis_rotated_camera():
    base = np.array([0.6, 0.3, 0.2])
    light_cam = np.array([0.9, -0.6, 0.4])
    s, Wf, tf = _phong_scene(light_cam, base)
    r = oracle.render_view(s, 0, backward=False)
    rgb = r["comp"]["rgb"]
    fid = r["face_id"]
    L = Wf @ s.light["pos"].astype(np.float64) + tf  # the light in camera space, as stored (fp32)
    ka, kd, ks = (float(np.float32(x)) for x in (0.1, 0.8, 0.3))
    b = base.astype(np.float32).astype(np.float64)
    n_checked, d_blinn, d_world = 0, 0.0, 0.0
    for (i, j) in [(5, 7), (30, 12), (24, 24), (40, 40), (10, 35), (33, 20)]:
        assert fid[j, i] >= 0
        z = float(r["depth"][j, i])
        x = np.array([(i + 0.5 - s.cx) / s.fx * z, (j + 0.5 - s.cy) / s.fy * z, z])
        l = (L - x) / np.linalg.norm(L - x)
        e = -x / np.linalg.norm(x)
        ndl = -l[2]  # n = (0, 0, -1)
        rde = -l[0] * e[0] - l[1] * e[1] + l[2] * e[2]  # the mirror image of l in the plane, dotted with e
        spec = ks * max(rde, 0.0) ** 32 if ndl > 0 else 0.0
        want = b * (ka + kd * max(ndl, 0.0)) + spec
        assert np.allclose(rgb[j, i], want, atol=2e-6), (i, j, rgb[j, i], want)
        # the alternatives this pin rules out
        h = (l + e) / np.linalg.norm(l + e)
        blinn = b * (ka + kd * max(ndl, 0.0)) + (ks * max(-h[2], 0.0) ** 32 if ndl > 0 else 0.0)
        d_blinn = max(d_blinn, float(np.abs(blinn - want).max()))
        lw = s.light["pos"].astype(np.float64)
        lw = (lw - x) / np.linalg.norm(lw - x)
        ndl_w = -lw[2]
        rde_w = -lw[0] * e[0] - lw[1] * e[1] + lw[2] * e[2]
        world = b * (ka + kd * max(ndl_w, 0.0)) + (ks * max(rde_w, 0.0) ** 32 if ndl_w > 0 else 0.0)
        d_world = max(d_world, float(np.abs(world - want).max()))
        n_checked += 1
    assert n_checked == 6
    assert d_blinn > 1e-3 and d_world > 1e-2, (d_blinn, d_world)
    # the highlight is lit: some checked pixel has a visible specular term
    assert rgb[:, :, 0].max() > b[0] * (ka + kd) + 0.01 * ks
