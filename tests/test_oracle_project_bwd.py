"""Pins of the oracle's projection backward (oracle/project_bwd.c).

The backward is hand-derived reverse mode of the EWA projection, the conditional
depth model and the SH colour.  It is checked against: central finite differences
of the fp64 forward (which itself is checked against the fp32 decision forward),
closed forms for an axis-aligned Gaussian on the optical axis, and the invariance
of the records under scaling of the quaternion.
"""
import numpy as np
import pytest

import oracle

FX = 300.0


def _rot(rng):
    q = rng.normal(size=4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def _setup(seed, N=16, sh_degree=3):
    """A rotated camera looking at Gaussians 2-6 units in front of it."""
    rng = np.random.default_rng(seed)
    R = _rot(rng)
    t = rng.normal(scale=0.5, size=3)
    cam = oracle.make_camera(256, 192, FX, FX * 1.1, 128.0, 96.0, R.astype(np.float32), t.astype(np.float32))
    Rf = np.array(cam.R, np.float64).reshape(3, 3)
    tf = np.array(cam.t, np.float64)
    xc = np.stack([rng.uniform(-0.8, 0.8, N), rng.uniform(-0.6, 0.6, N), rng.uniform(2.0, 6.0, N)])
    means = Rf.T @ (xc - tf[:, None])            # world positions of those camera points
    quats = rng.normal(size=(4, N)) * rng.uniform(0.5, 2.0, N)  # not normalised
    scales = np.exp(rng.normal(-3.0, 0.5, size=(3, N)))
    opacity = rng.uniform(0.05, 0.95, N)
    K = 1 if sh_degree < 0 else (sh_degree + 1) ** 2
    sh = rng.normal(scale=0.05, size=(K, 3, N))
    if sh_degree < 0:
        sh = rng.uniform(0.1, 0.9, size=(1, 3, N))
    g_rec = rng.normal(size=(N, 13))
    return cam, means, quats, scales, opacity, sh, g_rec


def test_f64_forward_matches_fp32_forward():
    cam, means, quats, scales, opacity, sh, _ = _setup(1)
    r32 = oracle.project_gaussians(cam, means.astype(np.float32), quats.astype(np.float32),
                                   scales.astype(np.float32), opacity.astype(np.float32),
                                   sh.reshape(-1, means.shape[1]).astype(np.float32), 3)
    r64 = oracle.project_f64(cam, means.astype(np.float32), quats.astype(np.float32),
                             scales.astype(np.float32), opacity.astype(np.float32),
                             sh.reshape(-1, means.shape[1]).astype(np.float32), 3)
    assert r32["valid"].all()
    a = r32["rec"][:, :13].astype(np.float64)
    np.testing.assert_allclose(r64, a, rtol=2e-4, atol=1e-5)


@pytest.mark.parametrize("sh_degree", [-1, 0, 1, 2, 3])
def test_finite_differences(sh_degree):
    cam, means, quats, scales, opacity, sh, g_rec = _setup(10 + sh_degree, sh_degree=sh_degree)
    N = means.shape[1]
    shp = sh.reshape(-1, N)
    listed = np.ones(N, np.int32)
    g = oracle.project_bwd(cam, means, quats, scales, shp, sh_degree, listed, g_rec)

    def records(m, q, s, o, c):
        return oracle.project_f64(cam, m, q, s, o, c, sh_degree)

    base = [means, quats, scales, opacity, shp]
    names = ["means", "quats", "scales", "opacity", "sh"]
    for a, name in enumerate(names):
        arr = base[a]
        flat = arr.reshape(-1)
        ana = g[name].reshape(-1)
        scale = np.sqrt(np.mean(ana ** 2)) + 1e-12
        for idx in range(flat.size):
            h = 1e-5 * max(abs(flat[idx]), 1e-2)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[a].reshape(-1)[idx] += h
            minus[a].reshape(-1)[idx] -= h
            d = (records(*plus) - records(*minus)) / (2 * h)  # difference first, then contract
            fd = float(np.sum(d * g_rec))
            assert abs(fd - ana[idx]) <= 1e-5 * (abs(ana[idx]) + scale), (name, idx, fd, ana[idx])


def _axis_case(sx, sy, sz, z0, sh_degree=0, sh=None):
    cam = oracle.make_camera(256, 256, FX, FX, 128.0, 128.0, np.eye(3, dtype=np.float32),
                             np.zeros(3, np.float32))
    means = np.array([[0.0], [0.0], [z0]])
    quats = np.array([[1.0], [0.0], [0.0], [0.0]])
    scales = np.array([[sx], [sy], [sz]])
    K = (sh_degree + 1) ** 2
    sh = np.zeros((K * 3, 1)) if sh is None else sh
    return cam, means, quats, scales, sh


def _unit(k):
    g = np.zeros((1, 13))
    g[0, k] = 1.0
    return g


def test_closed_forms_on_axis():
    sx, sy, sz, z0 = 0.05, 0.03, 0.04, 4.0
    cam, means, quats, scales, sh = _axis_case(sx, sy, sz, z0)
    one = np.ones(1, np.int32)
    a = FX * FX * sx * sx / (z0 * z0) + 0.3   # Sigma_2D[0][0] + eps; Q00 = 1 / a on the axis
    # Q00 weight: dQ00/dsx = -2 fx^2 sx / z^2 / a^2; dQ00/dz = 2 fx^2 sx^2 / (z^3 a^2)
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, one, _unit(2))
    np.testing.assert_allclose(g["scales"][:, 0], [-2 * FX * FX * sx / (z0 * z0) / a ** 2, 0.0, 0.0],
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["means"][:, 0], [0.0, 0.0, 2 * FX * FX * sx * sx / (z0 ** 3 * a * a)],
                               rtol=1e-12, atol=1e-12)
    # u weight: du/dx = fx / z, nothing else moves at x = 0
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, one, _unit(0))
    np.testing.assert_allclose(g["means"][:, 0], [FX / z0, 0.0, 0.0], rtol=1e-12, atol=1e-12)
    # g0 weight: g0 = Q00 k0, dk0/dx = -fx sz^2 / z^2 (J02 moves, C_zz = sz^2)
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, one, _unit(10))
    np.testing.assert_allclose(g["means"][:, 0], [-(1.0 / a) * FX * sz * sz / (z0 * z0), 0.0, 0.0],
                               rtol=1e-12, atol=1e-12)
    # sigma weight: sigma = sz on the axis
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, one, _unit(12))
    np.testing.assert_allclose(g["scales"][:, 0], [0.0, 0.0, 1.0], rtol=1e-12, atol=1e-12)
    # opacity passes through; z_c weight moves the mean along the axis
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, one, _unit(5) + 2.0 * _unit(9))
    assert g["opacity"][0] == 1.0
    np.testing.assert_allclose(g["means"][:, 0], [0.0, 0.0, 2.0], rtol=1e-12, atol=1e-12)


def test_sh_closed_forms():
    # band 0: colour = Y0 c + 1/2, Y0 = 1 / (2 sqrt(pi))
    cam, means, quats, scales, sh = _axis_case(0.05, 0.05, 0.05, 3.0, 0)
    gr = np.zeros((1, 13))
    gr[0, 6:9] = [1.0, 2.0, 3.0]
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, np.ones(1, np.int32), gr)
    np.testing.assert_allclose(g["sh"][0, :, 0], 0.5 / np.sqrt(np.pi) * np.array([1.0, 2.0, 3.0]), rtol=1e-14)
    # band 1 along +z (view direction from the camera at the origin): only Y_1^0 = sqrt(3/(4 pi)) z is live
    cam, means, quats, scales, sh = _axis_case(0.05, 0.05, 0.05, 3.0, 1, np.full((12, 1), 0.01))
    g = oracle.project_bwd(cam, means, quats, scales, sh, 1, np.ones(1, np.int32), gr)
    c1 = np.sqrt(3.0 / (4.0 * np.pi))
    np.testing.assert_allclose(g["sh"][2, :, 0], c1 * np.array([1.0, 2.0, 3.0]), rtol=1e-14)
    np.testing.assert_allclose(g["sh"][1, :, 0], 0.0, atol=1e-15)
    np.testing.assert_allclose(g["sh"][3, :, 0], 0.0, atol=1e-15)
    # a clamped channel (colour <= 0) passes no gradient
    cam, means, quats, scales, sh = _axis_case(0.05, 0.05, 0.05, 3.0, 0, np.array([[-5.0], [0.0], [0.0]]))
    g = oracle.project_bwd(cam, means, quats, scales, sh, 0, np.ones(1, np.int32), gr)
    assert g["sh"][0, 0, 0] == 0.0 and g["sh"][0, 1, 0] != 0.0


def test_quaternion_gradient_is_tangent():
    cam, means, quats, scales, opacity, sh, g_rec = _setup(5)
    N = means.shape[1]
    g = oracle.project_bwd(cam, means, quats, scales, sh.reshape(-1, N), 3, np.ones(N, np.int32), g_rec)
    dots = np.sum(g["quats"] * quats, axis=0)
    norms = np.linalg.norm(g["quats"], axis=0) * np.linalg.norm(quats, axis=0)
    assert np.all(np.abs(dots) <= 1e-12 * norms)


def test_unlisted_gaussians_get_zero():
    cam, means, quats, scales, opacity, sh, g_rec = _setup(6)
    N = means.shape[1]
    listed = np.zeros(N, np.int32)
    listed[::2] = 1
    g = oracle.project_bwd(cam, means, quats, scales, sh.reshape(-1, N), 3, listed, g_rec)
    for k, v in g.items():
        assert np.all(v[..., 1::2] == 0.0), k
        assert np.any(v[..., ::2] != 0.0), k
