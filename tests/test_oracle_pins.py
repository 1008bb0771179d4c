"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself: exact
rational arithmetic, closed forms, library routines (scipy rotations, scipy
spherical harmonics, scipy's normal CDF), invariants and central finite
differences.  None of these needs a GPU.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import scenes
import tiny

pytestmark = pytest.mark.usefixtures("oracle_lib")


# ---------------------------------------------------------------------------
# mesh visibility
# ---------------------------------------------------------------------------

def _exact_cover(us, vs, px, py):
    """Inclusive coverage of pixel centre (px+1/2, py+1/2) in exact rationals."""
    U = [Fraction(float(x)) for x in us]
    Vv = [Fraction(float(x)) for x in vs]
    pu, pv = Fraction(2 * px + 1, 2), Fraction(2 * py + 1, 2)

    def e(a, b):
        return (U[b] - U[a]) * (pv - Vv[a]) - (Vv[b] - Vv[a]) * (pu - U[a])

    A = (U[1] - U[0]) * (Vv[2] - Vv[0]) - (Vv[1] - Vv[0]) * (U[2] - U[0])
    if A == 0:
        return False
    E = [e(1, 2), e(2, 0), e(0, 1)]
    return all(x * (1 if A > 0 else -1) >= 0 for x in E)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("size", [16, 64])
def test_single_triangle_coverage_exact(seed, size):
    """The covered pixel set of one triangle equals the exact rational edge test.
    With fx = fy = 1, cx = cy = 0 and z = 1 the projection is the identity, so the
    screen vertices are the drawn ones; half the cases put vertices on pixel centres
    so that pixel centres fall exactly on edges (inclusive rule)."""
    rng = np.random.default_rng(seed)
    if seed % 2 == 0:
        xy = rng.uniform(-2, size + 2, size=(3, 2))
    else:
        xy = rng.integers(0, size, size=(3, 2)) + 0.5
    verts = np.concatenate([xy, np.ones((3, 1))], 1)
    s = tiny.set_mesh(tiny.empty_scene(size, size, 1.0, 1.0, 0.0, 0.0), verts, [[0, 1, 2]])
    cam = oracle.camera(s)
    vs = oracle.project_vertices(cam, s.verts)
    assert np.array_equal(vs[:2].T.astype(np.float64), xy.astype(np.float32).astype(np.float64))
    zb = oracle.zbuffer(cam, vs, s.faces)
    got = zb["face_id"] >= 0
    want = np.zeros_like(got)
    for py in range(size):
        for px in range(size):
            want[py, px] = _exact_cover(vs[0], vs[1], px, py)
    assert np.array_equal(got, want)
    # the winding does not matter
    s2 = tiny.set_mesh(tiny.empty_scene(size, size, 1.0, 1.0, 0.0, 0.0), verts, [[0, 2, 1]])
    zb2 = oracle.zbuffer(cam, oracle.project_vertices(cam, s2.verts), s2.faces)
    assert np.array_equal(zb2["face_id"] >= 0, want)


def _ray_plane_depth(P, px, py, fx, fy, cx, cy):
    n = np.cross(P[1] - P[0], P[2] - P[0])
    r = np.array([(px + 0.5 - cx) / fx, (py + 0.5 - cy) / fy, 1.0])
    return n.dot(P[0]) / n.dot(r)


@pytest.mark.parametrize("seed", range(4))
def test_mesh_depth_is_ray_plane(seed):
    """Perspective-correct depth equals the ray-plane intersection depth."""
    rng = np.random.default_rng(100 + seed)
    while True:  # redraw slivers that cover almost nothing
        P = np.stack([rng.uniform(-1, 1, 3), rng.uniform(-1, 1, 3), rng.uniform(2, 5, 3)], 1)
        s = tiny.set_mesh(tiny.empty_scene(48, 40, 40.0, 44.0, 24.0, 19.0), P, [[0, 1, 2]])
        cam = oracle.camera(s)
        vs = oracle.project_vertices(cam, s.verts)
        zb = oracle.zbuffer(cam, vs, s.faces)
        ys, xs = np.nonzero(zb["face_id"] >= 0)
        if len(xs) > 10:
            break
    Pc = s.verts.T.astype(np.float64)
    for x, y in zip(xs, ys):
        z = _ray_plane_depth(Pc, x, y, s.fx, s.fy, s.cx, s.cy)
        assert abs(zb["z1"][y, x] - z) <= 2e-6 * z


def test_perspective_correct_attributes():
    """An attribute affine in camera-space position is reproduced at the ray-plane
    point (perspective-correct barycentrics)."""
    rng = np.random.default_rng(7)
    P = np.stack([rng.uniform(-1, 1, 3), rng.uniform(-1, 1, 3), rng.uniform(2, 6, 3)], 1)
    M = rng.normal(size=(3, 3))
    b = rng.normal(size=3)
    col = P @ M.T + b
    s = tiny.set_mesh(tiny.empty_scene(40, 40, 40.0, 40.0, 20.0, 20.0), P, [[0, 1, 2]], vcolor=col)
    cam = oracle.camera(s)
    vs = oracle.project_vertices(cam, s.verts)
    zb = oracle.zbuffer(cam, vs, s.faces)
    pix = np.flatnonzero(zb["face_id"].ravel() >= 0)
    mref = oracle.MeshRef(cam, s, vs)
    cm, _ = oracle.shade_pixels(mref, pix, zb["face_id"].ravel()[pix])
    Pc = s.verts.T.astype(np.float64)
    colf = s.vcolor.T.astype(np.float64)
    # the affine map realised by the fp32 vertex colours
    Mf = np.linalg.lstsq(np.c_[Pc, np.ones(3)], colf, rcond=None)[0]  # exact on the plane
    for k, p in enumerate(pix):
        x, y = p % 40, p // 40
        z = _ray_plane_depth(Pc, x, y, 40.0, 40.0, 20.0, 20.0)
        X = np.array([(x + 0.5 - 20.0) / 40.0 * z, (y + 0.5 - 20.0) / 40.0 * z, z])
        want = np.r_[X, 1.0] @ Mf
        assert np.allclose(cm[k], want, rtol=0, atol=2e-5 * (1 + np.abs(want).max()))


def test_nearest_triangle_wins_and_ties_to_smaller_id():
    big = [[-1.0, -1.0], [1.0, -1.0], [0.0, 1.0]]
    for order in ([2.0, 3.0], [3.0, 2.0]):
        verts = [[x * z, y * z, z] for z in order for x, y in big]
        s = tiny.set_mesh(tiny.empty_scene(32, 32, 16.0, 16.0, 16.0, 16.0), verts, [[0, 1, 2], [3, 4, 5]])
        cam = oracle.camera(s)
        zb = oracle.zbuffer(cam, oracle.project_vertices(cam, s.verts), s.faces)
        near = 0 if order[0] == 2.0 else 1
        assert zb["face_id"][16, 16] == near
        assert abs(zb["depth"][16, 16] - 2.0) < 1e-6
        assert abs(zb["z2"][16, 16] - 3.0) < 1e-6
    # identical triangles: exact tie -> smaller id
    verts = [[x * 2, y * 2, 2.0] for x, y in big] * 2
    s = tiny.set_mesh(tiny.empty_scene(32, 32, 16.0, 16.0, 16.0, 16.0), verts, [[3, 4, 5], [0, 1, 2]])
    cam = oracle.camera(s)
    zb = oracle.zbuffer(cam, oracle.project_vertices(cam, s.verts), s.faces)
    assert zb["face_id"][16, 16] == 0


def test_near_plane_and_mask_skip_triangles():
    verts = [[-1, -1, 2], [1, -1, 2], [0, 1, 2], [-1, -1, 0.005], [1, -1, 2], [0, 1, 2]]
    s = tiny.set_mesh(tiny.empty_scene(32, 32, 16.0, 16.0, 16.0, 16.0), verts, [[0, 1, 2], [3, 4, 5]],
                      mask=[0, 1])
    cam = oracle.camera(s)
    zb = oracle.zbuffer(cam, oracle.project_vertices(cam, s.verts), s.faces, s.face_mask)
    assert (zb["face_id"] == -1).all()
    assert np.isinf(zb["depth"]).all()


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_prefilter_equals_literal_and_bins_hold_coverage(name):
    """The bbox-prefiltered z-buffer (used for 1080p samples) equals the literal
    all-triangle loop; every covering (tile, face) pair is in the tile's bin."""
    s = scenes.make_scene(name)
    for vi in range(min(2, len(s.views))):
        cam = oracle.camera(s, vi)
        vs = oracle.project_vertices(cam, s.verts)
        a = oracle.zbuffer(cam, vs, s.faces, s.face_mask, prefilter=False)
        b = oracle.zbuffer(cam, vs, s.faces, s.face_mask, prefilter=True)
        for k in ("face_id", "depth", "z1", "z2", "tile_dmax"):
            assert np.array_equal(a[k], b[k]), k
        off, ids = oracle.tile_bins(cam, vs, s.faces, s.face_mask)
        TX = s.tiles_x
        fid = a["face_id"]
        ys, xs = np.nonzero(fid >= 0)
        tiles = (ys // 16) * TX + xs // 16
        for t, f in set(zip(tiles.tolist(), fid[ys, xs].tolist())):
            assert f in set(ids[off[t]:off[t + 1]].tolist())
        # tile_dmax: max depth of a fully covered tile, +inf otherwise
        for t in range(0, len(a["tile_dmax"]), 7):
            ty, tx = divmod(t, TX)
            blk = a["depth"][ty * 16:(ty + 1) * 16, tx * 16:(tx + 1) * 16]
            want = blk.max() if np.isfinite(blk).all() else np.inf
            assert a["tile_dmax"][t] == want


def test_vertex_projection_matches_fp64():
    s = scenes.make_scene("c4")
    for vi in (0, 5):
        cam = oracle.camera(s, vi)
        vs = oracle.project_vertices(cam, s.verts)
        R = s.views[vi].R.astype(np.float64).reshape(3, 3)
        Xc = R @ s.verts.astype(np.float64) + s.views[vi].t.astype(np.float64)[:, None]
        u = s.fx * Xc[0] / Xc[2] + s.cx
        v = s.fy * Xc[1] / Xc[2] + s.cy
        assert np.allclose(vs[0], u, rtol=1e-6, atol=1e-4)
        assert np.allclose(vs[1], v, rtol=1e-6, atol=1e-4)
        assert np.allclose(vs[2], Xc[2], rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# Gaussian projection and the conditional depth model
# ---------------------------------------------------------------------------

def _proj_fp64(scene, i, view=0):
    """Independent fp64 projection built from scipy's quaternion rotation."""
    from scipy.spatial.transform import Rotation
    q = scene.quats[:, i].astype(np.float64)
    Rq = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
    S = np.diag(scene.scales[:, i].astype(np.float64) ** 2)
    Sig = Rq @ S @ Rq.T
    W = scene.views[view].R.astype(np.float64).reshape(3, 3)
    t = scene.views[view].t.astype(np.float64)
    mc = W @ scene.means[:, i].astype(np.float64) + t
    Sc = W @ Sig @ W.T
    x, y, z = mc
    J = np.array([[scene.fx / z, 0, -scene.fx * x / z ** 2], [0, scene.fy / z, -scene.fy * y / z ** 2],
                  [0, 0, 1.0]])
    Suvz = J @ Sc @ J.T
    Suv = Suvz[:2, :2] + 0.3 * np.eye(2)
    k = Suvz[:2, 2]
    Q = np.linalg.inv(Suv)
    g = Q @ k
    var = Suvz[2, 2] - k @ g
    u = scene.fx * x / z + scene.cx
    v = scene.fy * y / z + scene.cy
    return dict(u=u, v=v, Q=Q, z=z, g=g, sigma=math.sqrt(max(var, 1e-12)))


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_projection_matches_independent_fp64(name):
    s = scenes.make_scene(name)
    cam = oracle.camera(s)
    pg = oracle.project_gaussians(cam, s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    rec = pg["rec"].astype(np.float64)
    for i in np.linspace(0, s.N - 1, 60).astype(int):
        r = _proj_fp64(s, i)
        assert abs(rec[i, 0] - r["u"]) < 1e-4 and abs(rec[i, 1] - r["v"]) < 1e-4
        Qs = np.array([[rec[i, 2], rec[i, 3]], [rec[i, 3], rec[i, 4]]])
        assert np.allclose(Qs, r["Q"], rtol=2e-4, atol=1e-6 * np.abs(r["Q"]).max())
        assert abs(rec[i, 9] - r["z"]) <= 1e-6 * r["z"]
        gs = np.abs(r["g"]).max() + 1e-9
        assert np.allclose(rec[i, 10:12], r["g"], rtol=0, atol=2e-3 * gs)
        assert abs(rec[i, 12] - r["sigma"]) <= 2e-3 * r["sigma"] + 1e-6


def test_axis_aligned_conic_closed_form():
    fx, fy = 300.0, 200.0
    s = tiny.empty_scene(64, 64, fx, fy, 32.0, 32.0)
    z, sx, sy, sz = 3.0, 0.05, 0.02, 0.07
    tiny.set_gaussians(s, [[0, 0, z]], [[1, 0, 0, 0]], [[sx, sy, sz]], [0.5], rgb=[[1, 0, 0]])
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, -1)
    r = pg["rec"][0].astype(np.float64)
    a = fx ** 2 * sx ** 2 / z ** 2 + 0.3
    c = fy ** 2 * sy ** 2 / z ** 2 + 0.3
    assert abs(r[2] - 1 / a) <= 1e-6 / a and abs(r[4] - 1 / c) <= 1e-6 / c and r[3] == 0
    # isotropic / axis-aligned on the optical axis: g = 0, sigma = s_z
    assert r[10] == 0 and r[11] == 0
    assert abs(r[12] - sz) <= 1e-6
    assert r[0] == 32.0 and r[1] == 32.0


def test_flat_gaussian_on_tilted_plane_tilts():
    """A flat Gaussian lying in the plane z = z0 + a x has g0 -> a z0 / fx (the plane's
    screen-depth slope) and sigma -> 0 when its footprint dwarfs the 0.3 px^2 dilation."""
    fx = 512.0
    z0, a = 4.0, 0.6
    ang = math.atan(a)
    # rotation about y by -ang maps the local x axis onto (cos, 0, sin) direction
    qw, qy = math.cos(-ang / 2), math.sin(-ang / 2)
    s = tiny.empty_scene(64, 64, fx, fx, 32.0, 32.0)
    tiny.set_gaussians(s, [[0, 0, z0]], [[qw, 0, qy, 0]], [[0.2, 0.2, 1e-6]], [0.5], rgb=[[1, 1, 1]])
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, -1)
    r = pg["rec"][0].astype(np.float64)
    from scipy.spatial.transform import Rotation
    Rm = Rotation.from_quat([0, qy, 0, qw]).as_matrix()
    slope = Rm[2, 0] / Rm[0, 0]
    assert abs(slope - a) < 1e-6
    assert abs(r[10] - a * z0 / fx) <= 2e-3 * abs(a * z0 / fx)
    assert abs(r[11]) < 1e-7
    # sigma -> 0 as eps / Sigma_uu -> 0: for a rank-one footprint in the x-z plane the
    # Schur complement reduces to Sigma_zz eps / (Sigma_uu + eps)
    ext = 0.2 * math.sin(ang)
    suu = (fx / z0 * 0.2 * math.cos(ang)) ** 2
    assert abs(r[12] - math.sqrt(ext ** 2 * 0.3 / (suu + 0.3))) <= 1e-3 * r[12]
    assert r[12] < 0.03 * ext


def test_phi_matches_library():
    from scipy.stats import norm
    for x in [-6.0, -2.5, -1.0, -0.1, 0.0, 0.3, 1.7, 5.0]:
        assert abs(oracle.Phi(x) - norm.cdf(x)) <= 1e-15 + 1e-13 * norm.cdf(x)
    assert oracle.Phi(0.0) == 0.5


# ---------------------------------------------------------------------------
# spherical harmonics
# ---------------------------------------------------------------------------

def test_sh_degree0_matches_splat_constant():
    """Band 0: rgb = 0.2820948 f_dc + 0.5 (the .splat conversion constant)."""
    rng = np.random.default_rng(3)
    n = 50
    s = tiny.empty_scene(64, 64, 64.0, 64.0, 32.0, 32.0)
    means = np.c_[rng.uniform(-1, 1, (n, 2)), rng.uniform(2, 4, n)]
    dc = rng.normal(0, 1, (1, 3, n))
    tiny.set_gaussians(s, means, np.tile([1, 0, 0, 0], (n, 1)), np.full((n, 3), 0.05), np.full(n, 0.5),
                       sh=dc, sh_degree=0)
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, 0)
    want = np.maximum(0.2820948 * s.sh[0].astype(np.float64).T + 0.5, 0)
    assert np.allclose(pg["rgb64"], want, atol=2e-7 * (1 + np.abs(want)))


def test_sh_basis_orthonormal_and_matches_scipy():
    from scipy.special import sph_harm_y
    # Gauss-Legendre in cos(theta) x uniform phi: exact for products of degree <= 3
    xs, ws = np.polynomial.legendre.leggauss(10)
    nphi = 20
    G = np.zeros((16, 16))
    for ct, w in zip(xs, ws):
        st = math.sqrt(1 - ct * ct)
        for j in range(nphi):
            ph = 2 * math.pi * j / nphi
            Y = oracle.sh_basis(st * math.cos(ph), st * math.sin(ph), ct)
            G += np.outer(Y, Y) * w * (2 * math.pi / nphi)
    assert np.allclose(G, np.eye(16), atol=1e-12)
    # each basis function equals +-1 x the real SH built from scipy's complex ones
    rng = np.random.default_rng(0)
    dirs = rng.normal(size=(40, 3))
    dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
    sign = {}
    for d in dirs:
        th, ph = math.acos(d[2]), math.atan2(d[1], d[0])
        Y = oracle.sh_basis(*d)
        for l in range(4):
            for m in range(-l, l + 1):
                if m == 0:
                    ref = sph_harm_y(l, 0, th, ph).real
                elif m > 0:
                    ref = math.sqrt(2) * sph_harm_y(l, m, th, ph).real
                else:
                    ref = math.sqrt(2) * sph_harm_y(l, -m, th, ph).imag
                k = l * l + l + m
                if abs(ref) > 1e-3:
                    sg = np.sign(Y[k] / ref)
                    sign.setdefault(k, sg)
                    assert sign[k] == sg
                    assert abs(abs(Y[k]) - abs(ref)) < 1e-12
    assert len(sign) == 16
    # band-1 order and signs of the splatting convention: (-y, z, -x)
    Y = oracle.sh_basis(0.0, 1.0, 0.0)
    assert Y[1] < 0 and abs(Y[2]) < 1e-15 and abs(Y[3]) < 1e-15


# ---------------------------------------------------------------------------
# compositing closed forms
# ---------------------------------------------------------------------------

def _one_view(s, cull=True, grads=None, backward=False):
    return oracle.render_view(s, 0, cull=cull, backward=backward, grads=grads)


def test_peak_alpha_equals_opacity_no_mesh():
    for o in (0.05, 0.3, 0.8, 0.98):
        s = tiny.empty_scene(33, 33, 33.0, 33.0, 16.5, 16.5)
        tiny.set_gaussians(s, [[0, 0, 3.0]], [[1, 0, 0, 0]], [[0.05, 0.05, 0.05]], [o], rgb=[[0.2, 0.6, 0.9]])
        r = _one_view(s)["comp"]
        o = float(np.float32(o))  # opacity is an fp32 input
        assert abs(r["alpha"][16, 16] - o) < 1e-12
        want = o * np.array([0.2, 0.6, 0.9], np.float32) + (1 - o) * 1.0
        assert np.allclose(r["rgb"][16, 16], want, atol=1e-12)
        assert abs(r["depth"][16, 16] - o * 3.0) < 1e-12


def test_alpha_clamped_at_099():
    s = tiny.empty_scene(33, 33, 33.0, 33.0, 16.5, 16.5)
    tiny.set_gaussians(s, [[0, 0, 3.0]], [[1, 0, 0, 0]], [[0.05, 0.05, 0.05]], [0.999], rgb=[[0, 0, 0]])
    r = _one_view(s)["comp"]
    assert abs(r["alpha"][16, 16] - 0.99) < 1e-15


def test_transmittance_is_product():
    ops = [0.5, 0.3, 0.7, 0.2, 0.6]
    cols = np.random.default_rng(1).uniform(size=(5, 3))
    s = tiny.empty_scene(33, 33, 33.0, 33.0, 16.5, 16.5)
    zs = [2.0, 2.5, 3.0, 3.5, 4.0]
    tiny.set_gaussians(s, [[0, 0, z] for z in zs][::-1], [[1, 0, 0, 0]] * 5, [[0.05] * 3] * 5, ops[::-1],
                       rgb=cols[::-1])
    r = _one_view(s)["comp"]
    T = 1.0
    C = np.zeros(3)
    for o, c in zip(np.float32(ops).astype(np.float64), cols.astype(np.float32)):
        C += o * T * c
        T *= 1 - o
    assert abs(r["T_final"][16, 16] - T) < 1e-14
    assert np.allclose(r["rgb"][16, 16], C + T, atol=1e-12)
    assert abs(r["alpha"][16, 16] - (1 - T)) < 1e-14


def test_stop_rule_and_skip_rule():
    # opacities 0.9 ... T after 4 = 1e-4 -> the 4th entry would bring T below 1e-4: stop before it
    ops = [0.9, 0.9, 0.9, 0.95]
    s = tiny.empty_scene(33, 33, 33.0, 33.0, 16.5, 16.5)
    tiny.set_gaussians(s, [[0, 0, 2.0 + k] for k in range(4)], [[1, 0, 0, 0]] * 4, [[0.05] * 3] * 4, ops,
                       rgb=[[1, 1, 1]] * 4)
    r = _one_view(s)["comp"]
    assert r["n_incl"][16, 16] == 3
    assert abs(r["T_final"][16, 16] - (1 - float(np.float32(0.9))) ** 3) < 1e-12
    # below 1/255 an entry is skipped
    s = tiny.empty_scene(33, 33, 33.0, 33.0, 16.5, 16.5)
    tiny.set_gaussians(s, [[0, 0, 2.0]], [[1, 0, 0, 0]], [[0.05] * 3], [0.0039], rgb=[[0, 0, 0]])
    r = _one_view(s)["comp"]
    assert r["n_incl"][16, 16] == 0 and r["alpha"][16, 16] == 0


def _plane_scene(z_plane, size=33, f=33.0):
    s = tiny.empty_scene(size, size, f, f, size / 2, size / 2)
    h = 10.0
    verts = [[-h, -h, z_plane], [h, -h, z_plane], [h, h, z_plane], [-h, h, z_plane]]
    tiny.set_mesh(s, verts, [[0, 1, 2], [0, 2, 3]], vcolor=[[0.1, 0.2, 0.3]] * 4)
    return s


def test_split_half_at_surface_and_depth_output():
    """An isotropic Gaussian centred on a fronto-parallel mesh at its own depth is
    cut in half at its centre pixel: alpha_F = alpha / 2 (f = Phi(0))."""
    o = float(np.float32(0.6))
    s = _plane_scene(3.0)
    tiny.set_gaussians(s, [[0, 0, 3.0]], [[1, 0, 0, 0]], [[0.05] * 3], [o], rgb=[[0.9, 0.5, 0.1]])
    r = _one_view(s)["comp"]
    cm = np.array([0.1, 0.2, 0.3], np.float32).astype(np.float64)
    a = o / 2
    assert np.allclose(r["rgb"][16, 16], a * np.array([0.9, 0.5, 0.1], np.float32) + (1 - a) * cm, atol=1e-12)
    assert abs(r["depth"][16, 16] - (a * 3.0 + (1 - a) * 3.0)) < 1e-12
    assert r["alpha"][16, 16] == 1.0
    # in front of the mesh by many sigmas: fully in front
    s = _plane_scene(3.0)
    tiny.set_gaussians(s, [[0, 0, 2.0]], [[1, 0, 0, 0]], [[0.05] * 3], [o], rgb=[[0.9, 0.5, 0.1]])
    r = _one_view(s)["comp"]
    assert np.allclose(r["rgb"][16, 16], o * np.array([0.9, 0.5, 0.1], np.float32) + (1 - o) * cm, atol=1e-12)
    assert abs(r["depth"][16, 16] - (o * 2.0 + (1 - o) * 3.0)) < 1e-12
    # behind by many sigmas: hidden, and the pair is culled in the covered tile
    s = _plane_scene(3.0)
    tiny.set_gaussians(s, [[0, 0, 4.0]], [[1, 0, 0, 0]], [[0.05] * 3], [o], rgb=[[0.9, 0.5, 0.1]])
    res = _one_view(s)
    assert np.allclose(res["comp"]["rgb"][16, 16], cm, atol=1e-12)
    assert len(res["lists_pre"][1]) > 0 and len(res["lists"][1]) == 0


def test_mesh_only_closed_form():
    s = scenes.make_scene("c4")
    res = oracle.render_view(s, 3, backward=True)
    c = res["comp"]
    fid = res["face_id"]
    on = fid >= 0
    assert on.any() and (~on).any()
    pix = np.flatnonzero(on.ravel())
    mref = oracle.MeshRef(res["cam"], s, res["vscreen"], mips=oracle.build_mips(s.texture))
    cm, _ = oracle.shade_pixels(mref, pix, fid.ravel()[pix])
    assert np.allclose(c["rgb"].reshape(-1, 3)[pix], cm, atol=0)
    assert (c["rgb"][~on] == 1.0).all()
    assert np.array_equal(c["alpha"], on.astype(np.float64))
    assert np.array_equal(c["depth"][on], res["depth"][on].astype(np.float64))
    assert (c["depth"][~on] == 0).all()
    g = s.grads[3]
    assert np.allclose(c["g_mesh_rgb"][on], g["rgb"][on])
    assert (c["g_mesh_rgb"][~on] == 0).all()
    assert np.allclose(c["g_mesh_depth"][on], g["depth"][on])


def test_no_mesh_is_plain_splatting_brute_force():
    """face_id = -1 everywhere: plain front-to-back splatting, checked against a
    vectorised brute force over all (pixel, Gaussian) pairs with cumulative products."""
    s = tiny.random_tiny(11, n_tri=1, n_gauss=30)
    s.verts = None
    s.faces = None
    s.vcolor = None
    res = _one_view(s)
    c = res["comp"]
    rec = res["rec"].astype(np.float64)
    order = res["order"]
    H = W = s.width
    ys, xs = np.mgrid[0:H, 0:W]
    px, py = xs.ravel() + 0.5, ys.ravel() + 0.5
    tiles = (ys.ravel() // 16) * s.tiles_x + xs.ravel() // 16
    rect = res["rect"]
    al = np.zeros((H * W, len(order)))
    for k, i in enumerate(order):
        r = rec[i]
        dx, dy = px - r[0], py - r[1]
        q = 0.5 * (r[2] * dx * dx + 2 * r[3] * dx * dy + r[4] * dy * dy)
        a = np.minimum(0.99, r[5] * np.exp(-q))
        tx, ty = tiles % s.tiles_x, tiles // s.tiles_x
        inside = (tx >= rect[i, 0]) & (tx < rect[i, 2]) & (ty >= rect[i, 1]) & (ty < rect[i, 3])
        al[:, k] = np.where(inside & (a >= 1 / 255), a, 0.0)
    T = np.cumprod(np.c_[np.ones(H * W), 1 - al], axis=1)
    stop = T[:, 1:] < 1e-4
    first = np.where(stop.any(1), stop.argmax(1), len(order))
    keep = np.arange(len(order))[None, :] < first[:, None]
    w = al * T[:, :-1] * keep
    Tf = T[np.arange(H * W), first]
    col = w @ rec[order][:, 6:9] + Tf[:, None]
    assert np.allclose(c["rgb"].reshape(-1, 3), col, atol=1e-12)
    assert np.allclose(c["alpha"].ravel(), 1 - Tf, atol=1e-12)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_two_layer_equals_one_layer_and_cull_invariance(name):
    s = scenes.make_scene(name)
    a = oracle.render_view(s, cull=True, backward=True)
    b = oracle.render_view(s, cull=False, backward=True)
    ca, cb = a["comp"], b["comp"]
    for k in ("rgb", "depth", "alpha"):
        assert np.array_equal(ca[k], ca[k + "2"]), k
    for k in ("rgb", "depth", "alpha", "T_final", "g_mesh_rgb", "g_mesh_depth", "n_incl"):
        assert np.array_equal(ca[k], cb[k]), k
    # per-Gaussian sums over pixels whose order follows the OpenMP schedule: equal up
    # to fp64 summation order (observed <= 7e-13 relative)
    scale = float(np.abs(cb["grad"]).max())
    assert np.allclose(ca["grad"], cb["grad"], rtol=1e-9, atol=1e-12 * scale)
    assert len(a["lists"][1]) < len(b["lists"][1])


def test_lists_brute_force_membership_and_order():
    s = scenes.make_scene("c1")
    cam = oracle.camera(s)
    pg = oracle.project_gaussians(cam, s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    order = oracle.depth_order(pg["rec"], pg["valid"])
    zb = np.frombuffer(pg["rec"][:, 9].tobytes(), np.uint32)
    ids = np.arange(s.N)
    valid = pg["valid"].astype(bool)
    want_order = ids[valid][np.lexsort((ids[valid], zb[valid]))]
    assert np.array_equal(order, want_order)
    tiles = np.arange(s.tiles_x * s.tiles_y, dtype=np.int32)
    off, lst, _ = oracle.tile_lists(cam, pg["rec"], pg["rect"], order, tiles)
    for t in tiles:
        tx, ty = t % s.tiles_x, t // s.tiles_x
        mem = [i for i in want_order if pg["rect"][i, 0] <= tx < pg["rect"][i, 2]
               and pg["rect"][i, 1] <= ty < pg["rect"][i, 3]]
        assert lst[off[t]:off[t + 1]].tolist() == mem


def test_rect_covers_three_sigma_footprint():
    """The rect is the tile cover of the 3-sigma ellipse's bounding box: every pixel
    centre inside the ellipse (q <= 4.5) lies in a tile of it, and it reaches at most
    one tile plus a pixel beyond the box ceil(3 sqrt(Sigma2D_xx)) x ceil(3 sqrt(Sigma2D_yy)),
    with Sigma2D the inverse of the stored conic."""
    for name in ("c1", "c2"):
        s = scenes.make_scene(name)
        cam = oracle.camera(s)
        pg = oracle.project_gaussians(cam, s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
        rec = pg["rec"].astype(np.float64)
        H, W = s.height, s.width
        TX, TY = s.tiles_x, s.tiles_y
        step = 5 if name == "c1" else 997
        n = 0
        for i in range(0, s.N, step):
            if not pg["valid"][i]:
                continue
            r = rec[i]
            rc = pg["rect"][i]
            det = r[2] * r[4] - r[3] * r[3]
            sxx, syy = r[4] / det, r[2] / det  # Sigma2D from the conic
            hx, hy = math.ceil(3 * math.sqrt(sxx) - 1e-4), math.ceil(3 * math.sqrt(syy) - 1e-4)
            x0, x1 = max(0, int(r[0] - hx - 1) // 16), min(TX, -(-int(r[0] + hx + 2) // 16))
            y0, y1 = max(0, int(r[1] - hy - 1) // 16), min(TY, -(-int(r[1] + hy + 2) // 16))
            assert x0 <= rc[0] and rc[2] <= x1 and y0 <= rc[1] and rc[3] <= y1, (name, i, rc, (x0, y0, x1, y1))
            ys, xs = np.mgrid[max(0, int(r[1] - hy - 2)):min(H, int(r[1] + hy + 3)),
                              max(0, int(r[0] - hx - 2)):min(W, int(r[0] + hx + 3))]
            dx, dy = xs + 0.5 - r[0], ys + 0.5 - r[1]
            q = 0.5 * (r[2] * dx * dx + 2 * r[3] * dx * dy + r[4] * dy * dy)
            inside = q <= 4.5 * (1 - 1e-6)
            tx, ty = xs[inside] // 16, ys[inside] // 16
            assert ((tx >= rc[0]) & (tx < rc[2]) & (ty >= rc[1]) & (ty < rc[3])).all(), (name, i)
            n += 1
        assert n > 50


def test_rect_of_a_thin_diagonal_gaussian_is_its_box():
    """An elongated splat along the image diagonal: its rect follows the ellipse's box
    on each axis, ceil(3 sqrt(Sigma2D_xx + eps)) px, not the circle of its long axis
    (closed form for Sigma_uv = J Sigma J^T of an on-axis Gaussian)."""
    from scipy.spatial.transform import Rotation
    f = 400.0
    s = tiny.empty_scene(400, 400, f, f, 200.0, 200.0)
    q = Rotation.from_euler("z", 45, degrees=True).as_quat()  # x, y, z, w
    z = 4.0
    sx, sy, sz = 0.2, 0.004, 0.004
    tiny.set_gaussians(s, [[0, 0, z]], [[q[3], q[0], q[1], q[2]]], [[sx, sy, sz]], [0.9], rgb=[[1, 1, 1]])
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, -1)
    rc = pg["rect"][0]
    # on the axis J = diag(f/z, f/z): Sigma_uv = (f/z)^2 R diag(sx^2, sy^2) R^T, 45 degrees
    var_xx = (f / z) ** 2 * 0.5 * (sx ** 2 + sy ** 2) + 0.3
    h = math.ceil(3 * math.sqrt(var_xx))
    lam_max = (f / z) ** 2 * sx ** 2 + 0.3
    r_circle = math.ceil(3 * math.sqrt(lam_max))
    assert h < r_circle - 16  # the box is well inside the long axis' circle
    assert list(rc) == [int((200 - h) // 16), int((200 - h) // 16), -(-(200 + h) // 16), -(-(200 + h) // 16)]



# ---------------------------------------------------------------------------
# shading and texture
# ---------------------------------------------------------------------------

def test_phong_closed_form_on_axis():
    s = _plane_scene(2.0)
    s.vnormal = np.ascontiguousarray(np.tile([[0.0], [0.0], [-1.0]], (1, 4)), np.float32)
    s.light = {"pos": np.zeros(3, np.float32), "ambient": np.full(3, 0.1, np.float32),
               "diffuse": np.full(3, 0.8, np.float32), "specular": np.full(3, 0.3, np.float32),
               "shininess": np.float32(32.0)}
    r = _one_view(s)
    base = np.array([0.1, 0.2, 0.3], np.float32).astype(np.float64)
    want = base * (np.float32(0.1) + np.float32(0.8)) + np.float32(0.3)
    assert np.allclose(r["comp"]["rgb"][16, 16], want, atol=1e-12)
    # a pixel off axis is darker in the specular term
    assert (r["comp"]["rgb"][16, 2] < r["comp"]["rgb"][16, 16]).all()


def _tex_quad(tex, size=64, f=64.0, z=2.0, half=None):
    s = tiny.empty_scene(size, size, f, f, size / 2, size / 2)
    h = half if half is not None else 0.5 * z * size / f  # quad fills the image
    verts = [[-h, -h, z], [h, -h, z], [h, h, z], [-h, h, z]]
    tiny.set_mesh(s, verts, [[0, 1, 2], [0, 2, 3]])
    s.uv = np.ascontiguousarray(np.array([[0, 0], [1, 0], [1, 1], [0, 1]], np.float32).T)
    s.faces_uv = s.faces.copy()
    s.texture = np.ascontiguousarray(tex, np.float32)
    return s


def test_trilinear_constant_and_ramp_and_lod():
    S = 256
    # constant texture -> constant colour at every covered pixel
    s = _tex_quad(np.full((S, S, 3), 0.37))
    r = _one_view(s)["comp"]
    assert np.allclose(r["rgb"], np.float32(0.37), atol=1e-12)
    # linear ramp in u: every mip level holds the same ramp, so trilinear
    # filtering returns the ramp value in the interior
    u = (np.arange(S) + 0.5) / S
    ramp = np.repeat(np.repeat(u[None, :, None], S, 0), 3, 2)
    s = _tex_quad(ramp)
    res = _one_view(s)
    r = res["comp"]
    xs = np.arange(64)
    want = (xs + 0.5) / 64.0
    mid = slice(16, 48)
    assert np.allclose(r["rgb"][32, mid, 0], want[mid], atol=1e-6)
    # lod: 256 texels over 64 pixels -> log2(4) = 2
    cam = res["cam"]
    mref = oracle.MeshRef(cam, s, res["vscreen"], mips=oracle.build_mips(s.texture))
    pix = np.array([32 * 64 + 32, 20 * 64 + 40])
    _, lod = oracle.shade_pixels(mref, pix, res["face_id"].ravel()[pix])
    assert np.allclose(lod, 2.0, atol=1e-9)


def test_mip_pyramid_box_filter():
    rng = np.random.default_rng(0)
    tex = rng.uniform(size=(8, 8, 3)).astype(np.float32)
    m = oracle.build_mips(tex)
    l1 = m[8 * 8 * 3: 8 * 8 * 3 + 4 * 4 * 3].reshape(4, 4, 3)
    want = tex.astype(np.float64).reshape(4, 2, 4, 2, 3).mean(axis=(1, 3))
    assert np.allclose(l1, want, atol=1e-15)
    assert np.allclose(m[-3:], tex.astype(np.float64).mean(axis=(0, 1)), atol=1e-15)


# ---------------------------------------------------------------------------
# reverse mode vs central finite differences
# ---------------------------------------------------------------------------

def _loss(cam, mref, rec64, res, s, depth=None, g=None):
    off, ids = res["lists"]
    c = oracle.composite(cam, mref, rec64, res["tiles"], off, ids, res["face_id"],
                         res["depth"] if depth is None else depth, bg=s.bg, softness=s.softness)
    g = g or s.grads[0]
    return (np.sum(c["rgb"] * g["rgb"]) + np.sum(c["depth"] * g["depth"]) +
            np.sum(c["alpha"] * g["alpha"]))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_gradients_match_finite_differences(seed):
    s = tiny.random_tiny(seed, n_tri=4, n_gauss=10, size=32)
    res = oracle.render_view(s, cull=False, backward=True)
    cam = res["cam"]
    mref = oracle.MeshRef(cam, s, res["vscreen"])
    rec = res["rec"].astype(np.float64)
    grad = res["comp"]["grad"]
    c0 = res["comp"]
    # only at Gaussians whose decisions are far from thresholds
    assert np.isfinite(c0["margin"]).any()
    h = 1e-6
    checked = 0
    for i in np.unique(res["lists"][1]):
        for k in range(13):
            rp, rm = rec.copy(), rec.copy()
            rp[i, k] += h
            rm[i, k] -= h
            fd = (_loss(cam, mref, rp, res, s) - _loss(cam, mref, rm, res, s)) / (2 * h)
            an = grad[i, k]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-7, (i, k, fd, an)
            checked += 1
    assert checked >= 50
    # mesh depth: perturb D at a few covered pixels
    on = np.argwhere(res["face_id"] >= 0)
    for (y, x) in on[:: max(1, len(on) // 12)]:
        dp = res["depth"].astype(np.float64).copy()
        dm = dp.copy()
        dp[y, x] += h
        dm[y, x] -= h
        fd = (_loss(cam, mref, rec, res, s, depth=dp) - _loss(cam, mref, rec, res, s, depth=dm)) / (2 * h)
        an = c0["g_mesh_depth"][y, x]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-7


def test_mesh_colour_gradient_by_uniform_shift():
    """Shifting every vertex colour by h shifts c_m by h at every covered pixel
    (barycentrics sum to 1), so dL = sum(g_mesh_rgb) h."""
    s = tiny.random_tiny(4, n_tri=5, n_gauss=8, size=32)
    res = oracle.render_view(s, cull=False, backward=True)
    h = 1e-6
    sp, sm = tiny.random_tiny(4, n_tri=5, n_gauss=8, size=32), tiny.random_tiny(4, n_tri=5, n_gauss=8, size=32)
    sp.vcolor = (sp.vcolor.astype(np.float64) + h)
    sm.vcolor = (sm.vcolor.astype(np.float64) - h)

    def L(sc):
        r = oracle.render_view(sc, cull=False, backward=False)["comp"]
        g = s.grads[0]
        return np.sum(r["rgb"] * g["rgb"]) + np.sum(r["depth"] * g["depth"]) + np.sum(r["alpha"] * g["alpha"])

    # vcolor is handed to the oracle as fp32; use a perturbation it can represent
    sp.vcolor = np.float32(sp.vcolor)
    sm.vcolor = np.float32(sm.vcolor)
    d = (sp.vcolor.astype(np.float64) - sm.vcolor.astype(np.float64)) / 2
    assert np.allclose(d, d.flat[0], rtol=0.3)
    fd = (L(sp) - L(sm)) / 2
    an = np.sum(res["comp"]["g_mesh_rgb"] * 1.0) * d.mean()
    assert abs(fd - an) <= 2e-3 * abs(an) + 1e-9


# ---------------------------------------------------------------------------
# golden values printed by the pages
# ---------------------------------------------------------------------------

def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_golden_splat_dc_conversion():
    """The .splat conversion on the splatting reference page fixes the band-0
    constant and offset; the oracle's degree-0 colour reproduces its cases."""
    g = _golden("splat_dc.json")
    assert abs(oracle.sh_basis(0.0, 0.0, 1.0)[0] - g["sh_c0"]) < 5e-8
    s = tiny.empty_scene(32, 32, 32.0, 32.0, 16.0, 16.0)
    n = len(g["cases"])
    dc = np.array([c["f_dc"] for c in g["cases"]]).T[None]  # [1][3][n]
    tiny.set_gaussians(s, [[0.1 * k, 0, 3.0] for k in range(n)], [[1, 0, 0, 0]] * n, [[0.05] * 3] * n,
                       [0.5] * n, sh=dc, sh_degree=0)
    pg = oracle.project_gaussians(oracle.camera(s), s.means, s.quats, s.scales, s.opacity, s.sh, 0)
    for k, c in enumerate(g["cases"]):
        assert np.allclose(pg["rgb64"][k], c["rgb"], atol=2e-7)


def test_golden_defaults_used_by_workloads():
    g = _golden("renderer_defaults.json")
    s = scenes.make_scene("c1")
    assert tuple(s.bg) == tuple(g["bg_color"]) and s.softness == g["softness"]
    assert s.tiles_x == (s.width + g["tile_size"] - 1) // g["tile_size"]
