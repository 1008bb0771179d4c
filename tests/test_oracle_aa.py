"""Pins of the oracle's analytic edge antialiasing and two-layer composite
(oracle/antialias.c, the antialiased branch of oc_composite, oc_vscreen_bwd).

Checked against: the exact area of a pixel covered by a polygon (clipping in this
file, independent of the oracle) for straight edges along each axis, where the
per-axis one-dimensional model is exact; per-row conservation and the |slope|/8
per-pixel bound for slanted edges; supersampling convergence on a sphere (the
README's test suite checks antialiasing against supersampling); the topology rules
(internal edges untouched, boundary and back-facing neighbours are silhouettes,
farther surfaces are blended over); the reduction of the two-layer composite to
the one-layer one under binary coverage; closed forms for a mesh-only image, for
one Gaussian behind a fractional pixel and for a pixel whose front layer stops
before the Gaussians behind the mesh (the pixel stops with it, so the back layer
takes none of them); central finite differences of every
reverse mode; the scaling invariance of the screen-to-world vertex chain.
"""
import numpy as np
import pytest

import oracle
import scenes
import tiny


# ---------------------------------------------------------------------------
# helpers: exact polygon coverage of a pixel (Sutherland-Hodgman + shoelace)
# ---------------------------------------------------------------------------

def _clip(poly, inside, cross):
    out = []
    for i in range(len(poly)):
        p, q = poly[i - 1], poly[i]
        ip, iq = inside(p), inside(q)
        if iq:
            if not ip:
                out.append(cross(p, q))
            out.append(q)
        elif ip:
            out.append(cross(p, q))
    return out


def _area(poly):
    if len(poly) < 3:
        return 0.0
    a = 0.0
    for i in range(len(poly)):
        (x0, y0), (x1, y1) = poly[i - 1], poly[i]
        a += x0 * y1 - x1 * y0
    return abs(a) / 2


def pixel_coverage(poly, x, y):
    """Area of the convex screen polygon inside pixel [x, x+1] x [y, y+1]."""
    def lerp(p, q, t):
        return (p[0] + t * (q[0] - p[0]), p[1] + t * (q[1] - p[1]))
    P = [tuple(map(float, v)) for v in poly]
    for axis, bound, keep_less in ((0, x, False), (0, x + 1, True), (1, y, False), (1, y + 1, True)):
        def inside(p, a=axis, b=bound, k=keep_less):
            return p[a] <= b if k else p[a] >= b

        def cross(p, q, a=axis, b=bound):
            return lerp(p, q, (b - p[a]) / (q[a] - p[a]))
        P = _clip(P, inside, cross)
        if not P:
            return 0.0
    return _area(P)


def _world(u, v, z, f, c):
    # identity camera: u = f x / z + c
    return [(u - c) * z / f, (v - c) * z / f, z]


def _scene(size=24, f=None):
    f = float(size) if f is None else f
    return tiny.empty_scene(size, size, f, f, size / 2, size / 2)


def _layer(s):
    return oracle.render_view(s, 0, antialias=True, backward=False)


# ---------------------------------------------------------------------------
# coverage
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("xe", [7.3, 7.8, 11.5001, 4.02])
@pytest.mark.parametrize("vertical", [True, False])
def test_axis_aligned_edge_is_exact(xe, vertical):
    # a quad (two triangles sharing the diagonal) covering u < xe (or v < xe)
    S, z = 24, 2.0
    s = _scene(S)
    lo, hi = -6.0, S + 6.0
    if vertical:
        poly = [(lo, lo), (xe, lo), (xe, hi), (lo, hi)]
    else:
        poly = [(lo, lo), (hi, lo), (hi, xe), (lo, xe)]
    tiny.set_mesh(s, [_world(u, v, z, S, S / 2) for u, v in poly], [[0, 1, 2], [0, 2, 3]],
                  vcolor=[[0.9, 0.2, 0.1]] * 4)
    res = _layer(s)
    a = res["layer"][..., 4]
    exact = np.array([[pixel_coverage(poly, x, y) for x in range(S)] for y in range(S)])
    np.testing.assert_allclose(a, exact, atol=2e-6)
    # the colour is the mesh colour over the covered fraction
    np.testing.assert_allclose(res["layer"][..., 0], 0.9 * exact, atol=2e-6)


@pytest.mark.parametrize("m", [0.15, -0.4, 0.9])
def test_slanted_edge_rows_conserve_area(m):
    # edge u = x0 + m (v - 12) (steeper than 45 degrees: handled by horizontal pairs)
    S, z = 32, 3.0
    s = _scene(S)
    x0 = 15.37
    lo, hi = -8.0, S + 8.0
    poly = [(lo, lo), (x0 + m * (lo - 12), lo), (x0 + m * (hi - 12), hi), (lo, hi)]
    tiny.set_mesh(s, [_world(u, v, z, S, S / 2) for u, v in poly], [[0, 1, 2], [0, 2, 3]],
                  vcolor=[[1, 1, 1]] * 4)
    a = _layer(s)["layer"][..., 4]
    exact = np.array([[pixel_coverage(poly, x, y) for x in range(S)] for y in range(S)])
    # rows whose crossing stays a pixel away from the image border (no pair exists
    # across the border)
    yc = np.arange(S) + 0.5
    xr = x0 + m * (yc - 12)
    rows = (xr - abs(m) / 2 > 1.0) & (xr + abs(m) / 2 < S - 1.0)
    assert rows.sum() > S // 2
    np.testing.assert_allclose(a.sum(1)[rows], exact.sum(1)[rows], atol=1e-5)
    err = np.abs(a - exact)[rows]
    assert np.max(err) <= abs(m) / 8 + 1e-5
    # the bound is attained order of magnitude, i.e. the test can fail
    assert np.max(err) > abs(m) / 100


def _sphere_scene(S=64, colour=(1.0, 1.0, 1.0)):
    v, f = scenes.icosphere(3)
    s = _scene(S, f=1.2 * S)
    verts = v * 0.8 + np.array([0.05, -0.03, 3.0])
    tiny.set_mesh(s, verts, f, vcolor=np.tile(colour, (len(verts), 1)))
    return s


def test_supersampling_convergence():
    S, k = 64, 16
    s = _sphere_scene(S)
    res = _layer(s)
    a = res["layer"][..., 4]
    binary = (res["face_id"] >= 0).astype(float)
    big = tiny.empty_scene(S * k, S * k, s.fx * k, s.fy * k, s.cx * k, s.cy * k)
    big.verts, big.faces = s.verts, s.faces
    cam = oracle.camera(big, 0)
    zb = oracle.zbuffer(cam, oracle.project_vertices(cam, big.verts), big.faces)
    ss = (zb["face_id"] >= 0).reshape(S, k, S, k).mean(axis=(1, 3))
    err_aa, err_bin = np.abs(a - ss).mean(), np.abs(binary - ss).mean()
    assert err_aa < 0.25 * err_bin, (err_aa, err_bin)
    assert abs(a.sum() - ss.sum()) < 2e-3 * ss.sum()
    # silhouettes only: the interior (internal edges everywhere) stays fully covered
    inner = (res["face_id"] >= 0)
    for d in (1, -1):
        inner &= np.roll(res["face_id"] >= 0, d, 0) & np.roll(res["face_id"] >= 0, d, 1)
    assert np.all(a[inner & (ss == 1.0)] == 1.0)


def test_internal_edges_untouched_and_soup_edges_blend():
    S, z = 24, 2.0
    quad = [(-6, 3), (30, 3), (30, 20), (-6, 20)]
    cols = [[1, 0, 0], [0, 0, 1]]
    # shared vertices: the diagonal is internal
    s = _scene(S)
    tiny.set_mesh(s, [_world(u, v, z, S, S / 2) for u, v in quad], [[0, 1, 2], [0, 2, 3]],
                  vcolor=[[0.5, 0.5, 0.5]] * 4)
    res = _layer(s)
    L, fid = res["layer"], res["face_id"]
    inside = (np.arange(S)[:, None] >= 4) & (np.arange(S)[:, None] <= 18)
    assert np.all(L[..., 4][inside.repeat(S, 1)] == 1.0)
    # a soup of the same two triangles (no shared vertices), one colour each
    s2 = _scene(S)
    w = [_world(u, v, z, S, S / 2) for u, v in quad]
    tiny.set_mesh(s2, [w[0], w[1], w[2], w[0], w[2], w[3]], [[0, 1, 2], [3, 4, 5]],
                  vcolor=[cols[0]] * 3 + [cols[1]] * 3)
    res2 = _layer(s2)
    L2, fid2 = res2["layer"], res2["face_id"]
    assert np.all(L2[..., 4][inside.repeat(S, 1)] == 1.0)  # mesh over mesh: full coverage
    mixed = inside.repeat(S, 1) & (L2[..., 0] > 1e-9) & (L2[..., 2] > 1e-9)
    assert mixed.sum() > 5  # pixels along the diagonal blend the two colours
    # the shared-vertex version with the same colours blends nothing
    s3 = _scene(S)
    tiny.set_mesh(s3, [_world(u, v, z, S, S / 2) for u, v in quad], [[0, 1, 2], [0, 2, 3]],
                  vcolor=[[1, 0, 0]] * 4)
    L3 = _layer(s3)["layer"]
    np.testing.assert_array_equal(L3[..., 2][inside.repeat(S, 1)], 0.0)


def test_back_facing_neighbour_is_a_silhouette():
    # triangle A and, across its edge (1, 2), a triangle folded back behind A: the
    # shared edge is a silhouette, so the layer equals that of A alone
    S, z = 24, 2.0
    pa = [(3, 3), (17.3, 4.1), (6.2, 19.7)]
    va = [_world(u, v, z, S, S / 2) for u, v in pa]
    # the fourth vertex projects back inside A (folded over the shared edge) but deeper
    p4 = _world(8.0, 8.0, 3.5, S, S / 2)
    s = _scene(S)
    tiny.set_mesh(s, va + [p4], [[0, 1, 2], [3, 2, 1]], vcolor=[[0.3, 0.6, 0.9]] * 4)
    one = _scene(S)
    tiny.set_mesh(one, va, [[0, 1, 2]], vcolor=[[0.3, 0.6, 0.9]] * 3)
    r2, r1 = _layer(s), _layer(one)
    assert r2["adj"][0, 0] == 1  # the edge is shared topologically
    np.testing.assert_array_equal(r2["face_id"], r1["face_id"])
    np.testing.assert_allclose(r2["layer"], r1["layer"], atol=0, rtol=0)
    # the same two triangles unfolded (same facing): the shared edge is internal
    p4u = _world(20.0, 18.0, 2.0, S, S / 2)
    s3 = _scene(S)
    tiny.set_mesh(s3, va + [p4u], [[0, 1, 2], [3, 2, 1]], vcolor=[[0.3, 0.6, 0.9]] * 4)
    r3 = _layer(s3)
    seam = (r3["face_id"] >= 0)
    seam &= np.roll(r3["face_id"], 1, 1) != r3["face_id"]
    seam &= np.roll(r3["face_id"], 1, 1) >= 0
    assert seam.sum() > 3 and np.all(r3["layer"][..., 4][seam] == 1.0)


def test_front_surface_blends_over_farther_mesh():
    S = 24
    xe = 9.35
    front = [(-6, -6), (xe, -6), (xe, 30), (-6, 30)]
    back = [(-6, -6), (30, -6), (30, 30), (-6, 30)]
    s = _scene(S)
    w = [_world(u, v, 2.0, S, S / 2) for u, v in front] + [_world(u, v, 4.0, S, S / 2) for u, v in back]
    tiny.set_mesh(s, w, [[0, 1, 2], [0, 2, 3], [4, 5, 6], [4, 6, 7]],
                  vcolor=[[1, 0, 0]] * 4 + [[0, 1, 0]] * 4)
    L = _layer(s)["layer"]
    cov = np.array([[pixel_coverage(front, x, y) for x in range(S)] for y in range(S)])
    np.testing.assert_allclose(L[..., 4], 1.0, atol=1e-12)
    np.testing.assert_allclose(L[..., 0], cov, atol=2e-6)
    np.testing.assert_allclose(L[..., 1], 1.0 - cov, atol=2e-6)
    # premultiplied depth: 2 on the front fraction, 4 on the rest; the split depth is
    # each pixel's own
    np.testing.assert_allclose(L[..., 3], 2.0 * cov + 4.0 * (1 - cov), atol=1e-5)


def _quads(S, rects, colours, z=2.0):
    s = _scene(S)
    verts, faces, cols = [], [], []
    for (u0, u1, v0, v1), c in zip(rects, colours):
        n = len(verts)
        verts += [_world(u, v, z, S, S / 2) for u, v in ((u0, v0), (u1, v0), (u1, v1), (u0, v1))]
        faces += [[n, n + 1, n + 2], [n, n + 2, n + 3]]
        cols += [c] * 4
    tiny.set_mesh(s, verts, faces, vcolor=cols)
    return s


def test_clamped_coverage_keeps_the_colour():
    S = 16
    # a 0.2-pixel square hole around the centre of pixel (7, 7): its four neighbours
    # each give it 0.4 (raw coverage 1.6); a 0.4-pixel square island on pixel (12, 3)
    # loses 0.3 to each side (raw -0.2)
    rects = [(-5, 7.4, -5, 20), (7.6, 20, -5, 20), (7.4, 7.6, -5, 7.4), (7.4, 7.6, 7.6, 20)]
    cols = [[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 0]]
    s = _quads(S, rects, cols)
    res = _layer(s)
    L, raw = oracle.antialias(res["cam"], res["vscreen"].astype(np.float64), s.faces, s.face_mask, res["adj"],
                              res["face_id"], res["depth"], res["colour"], raw=True)
    assert res["face_id"][7, 7] < 0
    np.testing.assert_allclose(raw[7, 7, 1:5], 0.4, atol=1e-6)
    assert abs(raw[7, 7, 5] - 1.6) < 4e-6 and L[7, 7, 4] == 1.0
    # colour kept: the premultiplied colour is the raw one scaled by 1 / 1.6
    M = sum(raw[7, 7, 1 + d] * np.array(cols[d], float) for d in range(4))  # left, right, up, down quads
    np.testing.assert_allclose(L[7, 7, :3], M / raw[7, 7, 5], rtol=1e-12)
    s2 = _quads(S, [(12.3, 12.7, 3.3, 3.7)], [[0.5, 0.5, 0.5]])
    r2 = _layer(s2)
    L2, raw2 = oracle.antialias(r2["cam"], r2["vscreen"].astype(np.float64), s2.faces, s2.face_mask, r2["adj"],
                                r2["face_id"], r2["depth"], r2["colour"], raw=True)
    assert abs(raw2[3, 12, 5] + 0.2) < 4e-6
    assert L2[3, 12, 4] == 0.0 and np.all(L2[3, 12, :4] == 0.0)
    # everywhere: coverage in [0, 1], and equal to the raw sum inside it
    for Lx, rx in ((L, raw), (L2, raw2)):
        a, ar = Lx[..., 4], rx[..., 5]
        assert np.all((a >= 0) & (a <= 1))
        ok = (ar >= 0) & (ar <= 1)
        np.testing.assert_array_equal(a[ok], ar[ok])


# ---------------------------------------------------------------------------
# two-layer composite
# ---------------------------------------------------------------------------

def _binary_layer(res):
    fid, D = res["face_id"], res["depth"].astype(np.float64)
    H, W = fid.shape
    on = fid >= 0
    cm = np.zeros((H, W, 3))
    if res.get("colour") is not None:
        cm = res["colour"]
    L = np.zeros((H, W, 6))
    L[..., :3] = np.where(on[..., None], cm, 0.0)
    L[..., 3] = np.where(on, D, 0.0)
    L[..., 4] = on
    L[..., 5] = np.where(on, D, np.inf)
    return L


def test_two_layer_reduces_to_one_layer_under_binary_coverage():
    for seed in (1, 2, 3):
        s = tiny.random_tiny(seed, n_tri=8, n_gauss=40, size=40)
        res = oracle.render_view(s, 0, antialias=True, backward=True)
        ref = oracle.render_view(s, 0, antialias=False, backward=True)
        cam = res["cam"]
        off, ids = ref["lists"]
        L = _binary_layer(res)
        mref = oracle.MeshRef(cam, s, res["vscreen"])
        two = oracle.composite(cam, mref, res["rec"].astype(np.float64), ref["tiles"], off, ids, res["face_id"],
                               res["depth"], bg=s.bg, softness=s.softness, grads=s.grads[0], layer=L)
        one = ref["comp"]
        for k in ("rgb", "depth", "alpha"):
            np.testing.assert_allclose(two[k], one[k], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(two["grad"], one["grad"], rtol=1e-9, atol=1e-12)
        on = res["face_id"] >= 0
        np.testing.assert_allclose(two["g_layer"][..., :3][on], one["g_mesh_rgb"][on], rtol=1e-12, atol=1e-14)
        # dL/dD: through M_D (depth output) and the split, as in the one-layer form
        np.testing.assert_allclose((two["g_layer"][..., 3] + two["g_layer"][..., 5])[on], one["g_mesh_depth"][on],
                                   rtol=1e-9, atol=1e-12)


def test_mesh_only_closed_form():
    s = _sphere_scene(32, colour=(0.2, 0.7, 0.4))
    res = oracle.render_view(s, 0, antialias=True, backward=False)
    L, c = res["layer"], res["comp"]
    bg = np.array(s.bg)
    np.testing.assert_allclose(c["rgb"], L[..., :3] + (1 - L[..., 4:5]) * bg, atol=1e-12)
    np.testing.assert_allclose(c["alpha"], L[..., 4], atol=1e-12)
    np.testing.assert_allclose(c["depth"], L[..., 3], atol=1e-12)
    assert np.any((L[..., 4] > 0.05) & (L[..., 4] < 0.95))


def test_gaussian_behind_a_fractional_pixel():
    # a vertical edge at u = 7.3 over background; one Gaussian well behind the mesh,
    # centred on pixel (7, 5); its back share shows through (1 - a_m)
    S, z = 16, 2.0
    s = _scene(S)
    poly = [(-4, -4), (7.3, -4), (7.3, 20), (-4, 20)]
    tiny.set_mesh(s, [_world(u, v, z, S, S / 2) for u, v in poly], [[0, 1, 2], [0, 2, 3]],
                  vcolor=[[1, 0, 0]] * 4)
    zg = 6.0
    tiny.set_gaussians(s, [_world(7.5, 5.5, zg, S, S / 2)], [[1, 0, 0, 0]], [[0.2, 0.2, 0.05]], [0.7],
                       rgb=[[0, 0.5, 1]])
    res = oracle.render_view(s, 0, antialias=True, backward=False)
    L, c = res["layer"], res["comp"]
    am = L[5, 7, 4]
    assert abs(am - 0.3) < 1e-6
    r = res["rec"][0].astype(np.float64)
    D = L[5, 7, 5]
    assert D == res["depth"][5, 6]  # the split depth of the neighbour that gives the coverage
    dx, dy = 7.5 - r[0], 5.5 - r[1]
    sv = ((D - r[9]) - (r[10] * dx + r[11] * dy)) / (r[12] * s.softness)
    f = oracle.Phi(sv)
    alpha = min(0.99, r[5] * np.exp(-0.5 * (r[2] * dx * dx + 2 * r[3] * dx * dy + r[4] * dy * dy)))
    aB = alpha * (1 - f)
    assert aB > 0.5 and alpha * f < 1 / 255
    want = L[5, 7, :3] + (1 - am) * (aB * r[6:9] + (1 - aB) * np.array(s.bg))
    np.testing.assert_allclose(c["rgb"][5, 7], want, rtol=1e-12)
    np.testing.assert_allclose(c["alpha"][5, 7], 1 - (1 - am) * (1 - aB), rtol=1e-12)


def _loss_two_layer(cam, s, rec64, tiles, off, ids, fid, depth, L, g):
    c = oracle.composite(cam, None, rec64, tiles, off, ids, fid, depth, bg=s.bg, softness=s.softness, layer=L)
    return float(np.sum(c["rgb"] * g["rgb"]) + np.sum(c["depth"] * g["depth"]) + np.sum(c["alpha"] * g["alpha"]))


def _fractional_layer(res, rng):
    L = _binary_layer(res)
    H, W = L.shape[:2]
    # fractional coverage everywhere (finite split depth where covered)
    a = rng.uniform(0.2, 0.8, size=(H, W))
    on = res["face_id"] >= 0
    L[..., 4] = np.where(on, a, 0.0)
    L[..., :4] *= np.where(on, a, 0.0)[..., None]
    return L


@pytest.mark.parametrize("seed", [7, 8])
def test_two_layer_reverse_mode_fd(seed):
    s = tiny.random_tiny(seed, n_tri=6, n_gauss=25, size=32)
    s.softness = 0.7
    res = oracle.render_view(s, 0, antialias=True, backward=False)
    cam = res["cam"]
    rng = np.random.default_rng(seed)
    L = _fractional_layer(res, rng)
    off, ids = res["lists"]
    rec64 = res["rec"].astype(np.float64)
    g = s.grads[0]
    c = oracle.composite(cam, None, rec64, res["tiles"], off, ids, res["face_id"], res["depth"], bg=s.bg,
                         softness=s.softness, grads=g, layer=L)
    assert np.nanmax(c["n_last_back"]) > 0  # the back layer is live
    args = (cam, s, None, res["tiles"], off, ids, res["face_id"], res["depth"], None, g)

    def loss(rec=rec64, layer=L):
        a = list(args)
        a[2], a[8] = rec, layer
        return _loss_two_layer(*a)
    # records: every field of the Gaussians that reach a pixel (away from decisions)
    used = np.unique(ids)
    margin = np.nanmin(np.where(np.isfinite(c["margin"]), c["margin"], np.inf))
    assert margin > 1e-5  # h below perturbs each decision quantity by ~1e-7 relative
    for i in rng.choice(used, size=min(6, len(used)), replace=False):
        for fld in range(13):
            h = 1e-7 * max(abs(rec64[i, fld]), 1.0)
            rp, rm = rec64.copy(), rec64.copy()
            rp[i, fld] += h
            rm[i, fld] -= h
            fd = (loss(rec=rp) - loss(rec=rm)) / (2 * h)
            an = c["grad"][i, fld]
            assert abs(fd - an) <= 2e-5 * (abs(an) + 1e-3 * np.abs(c["grad"]).max()), (i, fld, fd, an)
    # the layer: colour, depth, coverage and split depth of covered pixels
    on = np.argwhere(res["face_id"] >= 0)
    for (y, x) in on[rng.choice(len(on), size=min(12, len(on)), replace=False)]:
        for ch in range(6):
            h = 1e-7 * max(abs(L[y, x, ch]), 1.0)
            lp, lm = L.copy(), L.copy()
            lp[y, x, ch] += h
            lm[y, x, ch] -= h
            fd = (loss(layer=lp) - loss(layer=lm)) / (2 * h)
            an = c["g_layer"][y, x, ch]
            assert abs(fd - an) <= 2e-5 * (abs(an) + 1e-3), (y, x, ch, fd, an)


# ---------------------------------------------------------------------------
# antialiasing reverse mode
# ---------------------------------------------------------------------------

def _aa_fd_setup(seed):
    s = tiny.random_tiny(seed, n_tri=10, n_gauss=0, size=40)
    res = oracle.render_view(s, 0, antialias=True, backward=False)
    rng = np.random.default_rng(seed)
    g_layer = rng.normal(size=res["layer"].shape)
    g_layer[..., 5][~np.isfinite(res["layer"][..., 5])] = 0.0
    return s, res, g_layer, rng


def _aa_loss(cam, s, res, vs, colour, depth, g_layer):
    L = oracle.antialias(cam, vs, s.faces, s.face_mask, res["adj"], res["face_id"], depth, colour)
    Lf = np.where(np.isfinite(L), L, 0.0)
    return float(np.sum(Lf * g_layer))


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_antialias_reverse_mode_fd(seed):
    s, res, g_layer, rng = _aa_fd_setup(seed)
    cam = res["cam"]
    vs = res["vscreen"].astype(np.float64)
    col, depth = res["colour"], res["depth"]
    g = oracle.antialias_bwd(cam, vs, s.faces, s.face_mask, res["adj"], res["face_id"], depth, col, g_layer)
    assert np.abs(g["vs"]).max() > 0
    # screen vertices (continuous in the crossings: h well below the distance of any
    # crossing to 1/2 or of an edge to a pixel centre)
    nz = np.argwhere(np.abs(g["vs"]) > 0)
    for (c, i) in nz[rng.choice(len(nz), size=min(25, len(nz)), replace=False)]:
        h = 1e-6
        vp, vm = vs.copy(), vs.copy()
        vp[c, i] += h
        vm[c, i] -= h
        fd = (_aa_loss(cam, s, res, vp, col, depth, g_layer) - _aa_loss(cam, s, res, vm, col, depth, g_layer)) / (2 * h)
        an = g["vs"][c, i]
        assert abs(fd - an) <= 1e-5 * (abs(an) + 1e-3), (c, i, fd, an)
    # colours: the layer is linear in them
    cov = np.argwhere(res["face_id"] >= 0)
    for (y, x) in cov[rng.choice(len(cov), size=15, replace=False)]:
        for ch in range(3):
            cp, cm_ = col.copy(), col.copy()
            cp[y, x, ch] += 0.5
            cm_[y, x, ch] -= 0.5
            fd = (_aa_loss(cam, s, res, vs, cp, depth, g_layer) - _aa_loss(cam, s, res, vs, cm_, depth, g_layer))
            assert abs(fd - g["colour"][y, x, ch]) <= 1e-9 * (1 + abs(fd))
    # depths (fp32 input; small steps that flip no front/back decision)
    for (y, x) in cov[rng.choice(len(cov), size=15, replace=False)]:
        h = np.float32(1e-5)
        dp, dm = depth.copy(), depth.copy()
        dp[y, x] += h
        dm[y, x] -= h
        fd = (_aa_loss(cam, s, res, vs, col, dp, g_layer) - _aa_loss(cam, s, res, vs, col, dm, g_layer)) / float(
            dp[y, x] - dm[y, x])
        assert abs(fd - g["depth"][y, x]) <= 1e-4 * (1 + abs(fd)), (y, x, fd, g["depth"][y, x])


def test_end_to_end_silhouette_gradient_fd():
    # screen vertices -> antialiased layer -> two-layer composite -> loss
    s = tiny.random_tiny(31, n_tri=6, n_gauss=30, size=32)
    res = oracle.render_view(s, 0, antialias=True, backward=True)
    cam = res["cam"]
    off, ids = res["lists"]
    rec64 = res["rec"].astype(np.float64)
    vs = res["vscreen"].astype(np.float64)
    g = oracle.antialias_bwd(cam, vs, s.faces, s.face_mask, res["adj"], res["face_id"], res["depth"],
                             res["colour"], res["comp"]["g_layer"])

    def loss(v):
        L = oracle.antialias(cam, v, s.faces, s.face_mask, res["adj"], res["face_id"], res["depth"], res["colour"])
        return _loss_two_layer(cam, s, rec64, res["tiles"], off, ids, res["face_id"], res["depth"], L, s.grads[0])
    nz = np.argwhere(np.abs(g["vs"]) > 1e-6)
    assert len(nz) > 4
    for (c, i) in nz[:12]:
        h = 1e-6
        vp, vm = vs.copy(), vs.copy()
        vp[c, i] += h
        vm[c, i] -= h
        fd = (loss(vp) - loss(vm)) / (2 * h)
        assert abs(fd - g["vs"][c, i]) <= 1e-5 * (abs(fd) + 1e-2), (c, i, fd, g["vs"][c, i])


@pytest.mark.parametrize("seed", [41, 42])
def test_vscreen_chain_scaling_invariance(seed):
    # (u, v) do not change when a vertex moves along its ray from the camera centre,
    # so sum_v (X_v - centre) . dL/dX_v = 0 for any dL/d(u, v); on the optical axis
    # dL/dx_c = fx / z dL/du exactly
    rng = np.random.default_rng(seed)
    s = tiny.random_tiny(seed, n_tri=5, n_gauss=0, size=32)
    th = rng.uniform(0, 2 * np.pi)
    s.views = [scenes.look_at_y(th, 2.0, 3.0)]
    cam = oracle.camera(s, 0)
    m = oracle.MeshB64(s)
    g_vs = rng.normal(size=(2, s.V))
    gX = oracle.vscreen_bwd(cam, m, g_vs)
    R = np.array(list(cam.R), np.float64).reshape(3, 3)
    t = np.array(list(cam.t), np.float64)
    centre = -np.linalg.solve(R, t)  # where x_c = 0 (the fp32 R is not exactly orthogonal)
    rel = m.verts - centre[:, None]
    assert abs(np.sum(rel * gX)) <= 1e-9 * np.sum(np.abs(rel * gX))
    assert np.sum(np.abs(rel * gX)) > 1e-3
    s2 = tiny.empty_scene(32, 32, 40.0, 40.0, 16.0, 16.0)
    tiny.set_mesh(s2, [[0.0, 0.0, 2.5], [0.1, 0.0, 2.5], [0.0, 0.1, 2.5]], [[0, 1, 2]])
    cam2 = oracle.camera(s2, 0)
    g2 = oracle.vscreen_bwd(cam2, oracle.MeshB64(s2), np.array([[1.0, 0, 0], [0.0, 0, 0]]))
    np.testing.assert_allclose(g2[:, 0], [40.0 / 2.5, 0.0, 0.0], rtol=1e-15)


def _one_pixel_layer_composite(zs, cols, am=0.5, D=5.0, M=(0.1, 0.2, 0.3), MD=0.7, bg=(0.9, 0.8, 0.7)):
    """The two-layer composite of Gaussians centred on pixel (8, 8) of a 16x16 image
    (G = 1 there, alpha = 0.99, hard split: softness 0), listed in the given order,
    over a mesh layer (premultiplied colour M, depth MD, coverage am, split depth D)."""
    s = _scene(16)
    cam = oracle.camera(s, 0)
    n = len(zs)
    rec = np.zeros((n, oracle.NREC))
    rec[:, 0] = rec[:, 1] = 8.5                # centred on the pixel centre
    rec[:, 2] = rec[:, 4] = 1.0                # conic: q = (dx^2 + dy^2) / 2
    rec[:, 5] = 1.0                            # opacity (alpha clamps to 0.99)
    rec[:, 6:9] = cols
    rec[:, 9] = zs                             # z_c; depth slopes g0 = g1 = 0
    rec[:, 12] = 0.5                           # sigma
    L = np.zeros((16, 16, 6))
    L[..., 5] = np.inf
    L[8, 8] = [M[0], M[1], M[2], MD, am, D]
    fid = np.full((16, 16), -1, np.int32)
    depth = np.full((16, 16), np.inf, np.float32)
    c = oracle.composite(cam, None, rec, np.array([0], np.int32), np.array([0, n], np.int64),
                         np.arange(n, dtype=np.int32), fid, depth, bg=bg, softness=0.0, layer=L)
    return c, np.array(M), MD, am, np.array(bg)


def test_pixel_stops_with_its_front_layer():
    # Three Gaussians in front of the split depth D = 5, then two behind it, in depth
    # order.  The front layer takes the first two (T_F = 0.01, then 1e-4) and stops at
    # the third (T would fall to 1e-6 < 1e-4); the 3DGS stop ends the pixel, so the back
    # layer, seen through T_F, takes neither Gaussian behind the mesh.
    cols = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 0], [0, 1, 1]], float)
    zs = [1.0, 2.0, 3.0, 6.0, 7.0]
    c, M, MD, am, bg = _one_pixel_layer_composite(zs, cols)
    TF = 0.01 * 0.01
    CF = 0.99 * cols[0] + 0.99 * 0.01 * cols[1]
    ZF = 0.99 * zs[0] + 0.99 * 0.01 * zs[1]
    np.testing.assert_allclose(c["rgb"][8, 8], CF + TF * (M + (1 - am) * bg), rtol=1e-12)
    np.testing.assert_allclose(c["alpha"][8, 8], 1 - TF * (1 - am), rtol=1e-12)
    np.testing.assert_allclose(c["depth"][8, 8], ZF + TF * MD, rtol=1e-12)
    assert c["n_last"][8, 8] == 2
    # and the same front entries with the back layer composited when the front does
    # not stop: one Gaussian in front (T_F = 0.01), two behind (T_B = 0.01, 1e-4)
    c2, M, MD, am, bg = _one_pixel_layer_composite([1.0, 6.0, 7.0], cols[[0, 3, 4]])
    TF2, TB2 = 0.01, 0.01 * 0.01
    CB2 = 0.99 * cols[3] + 0.99 * 0.01 * cols[4]
    ZB2 = 0.99 * 6.0 + 0.99 * 0.01 * 7.0
    want = 0.99 * cols[0] + TF2 * (M + (1 - am) * (CB2 + TB2 * bg))
    np.testing.assert_allclose(c2["rgb"][8, 8], want, rtol=1e-12)
    np.testing.assert_allclose(c2["alpha"][8, 8], 1 - TF2 * (1 - am) * TB2, rtol=1e-12)
    np.testing.assert_allclose(c2["depth"][8, 8], 0.99 * 1.0 + TF2 * (MD + (1 - am) * ZB2), rtol=1e-12)
