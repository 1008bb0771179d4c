"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every workload is compared on every tile: the 64x64 random soup, the 512x512
icosphere, three views of the 800x800 textured soup, the 1080p sphere with 1M
Gaussians and all four views of the 1080p four-sphere scene with 3M Gaussians, and
tiny edge cases, with the workloads' full upstream gradients.
"""
import numpy as np
import pytest

import oracle
import scenes
import tiny
import parity as P

pytestmark = pytest.mark.gpu

_CACHE = {}


def _scene(name):
    if name not in _CACHE:
        _CACHE[name] = scenes.make_scene(name)
    return _CACHE[name]


def _renderer(scene):
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    return Renderer(DeviceScene(scene))


def _run(scene, view, tiles=None, cull=True, masked=False):
    """Run GPU fwd+bwd and the oracle on ``tiles`` (all tiles when None)."""
    import torch
    T = scene.tiles_x * scene.tiles_y
    tiles = np.arange(T, dtype=np.int32) if tiles is None else np.asarray(tiles, np.int32)
    g = P.masked_grads(scene, view, tiles) if masked else scene.grads[view]
    r = _renderer(scene)
    r.forward(view, cull=cull)
    gd = {k: torch.from_numpy(v).cuda() for k, v in g.items()}
    r.backward(gd["rgb"], gd["depth"], gd["alpha"])
    gpu = P.gpu_state(r, with_grads=True)
    ora = oracle.render_view(scene, view, tiles=tiles, cull=cull, backward=True, grads=g)
    return gpu, ora, tiles


def _check_all(scene, view, gpu, ora, tiles, cull, label):
    rep = {}
    rep["vscreen_mismatch"] = P.compare_vscreen(gpu, ora) if scene.F else 0
    zb = P.compare_zbuffer(scene, gpu, ora, tiles)
    rep.update({k: v for k, v in zb.items() if k != "ties"})
    rep.update(P.compare_records(gpu, ora) if scene.N else {})
    rep.update(P.compare_lists(scene, gpu, ora, tiles, cull) if scene.N else {})
    im = P.compare_images(scene, gpu, ora, tiles, ties=zb["ties"])
    rep.update({k: v for k, v in im.items() if not k.endswith("_mask")})
    gr = P.compare_grads(scene, gpu, ora, tiles, im["straddle_mask"])
    rep.update(gr)
    print(label, {k: v for k, v in rep.items()}, flush=True)
    for key in ("rgb", "depth", "alpha", "T", "g_rec", "g_mesh_rgb", "g_mesh_depth"):
        assert np.isfinite(gpu[key]).all(), key
    assert rep["vscreen_mismatch"] == 0
    assert rep["face_mismatch"] == 0 and rep["depth_mismatch"] == 0 and rep["dmax_mismatch"] == 0
    if scene.N:
        assert rep["valid_mismatch"] == 0 and rep["rect_mismatch"] == 0 and rep["ntiles_mismatch"] == 0
        assert rep["field_mismatch"] == 0 and rep["rgb_ok"]
        assert rep["list_mismatch"] == 0
    assert rep["img_bad"] == 0
    npx = len(tiles) * 256
    assert rep["straddle"] <= max(2, 1e-4 * npx), "too many straddle exemptions used"
    assert rep["grad_exempt"] <= max(2, 1e-4 * max(scene.N, 1)), "too many gradient exemptions used"
    assert not rep["planes_bad"] and rep["elem_bad"] == 0
    assert rep["mesh_rgb_bad"] == 0 and rep["mesh_depth_bad"] == 0
    return rep


@pytest.mark.parametrize("cull", [True, False])
def test_c1_full(cull):
    s = _scene("c1")
    gpu, ora, tiles = _run(s, 0, cull=cull)
    _check_all(s, 0, gpu, ora, tiles, cull, "c1 cull=%s" % cull)
    assert P.compare_bins(s, 0, gpu) == 0


def test_c2_full():
    s = _scene("c2")
    gpu, ora, tiles = _run(s, 0, cull=True)
    _check_all(s, 0, gpu, ora, tiles, True, "c2")
    assert P.compare_bins(s, 0, gpu) == 0


@pytest.mark.parametrize("view", range(16))
def test_c4_views(view):
    """Every one of the 16 views of the triangle-soup workload on every tile."""
    s = _scene("c4")
    gpu, ora, tiles = _run(s, view, cull=True)
    _check_all(s, view, gpu, ora, tiles, True, "c4 view %d" % view)
    assert P.compare_bins(s, view, gpu) == 0


def _sample_tiles(scene, n, seed=0):
    rng = np.random.default_rng(seed)
    T = scene.tiles_x * scene.tiles_y
    t = set(rng.choice(T, size=n, replace=False).tolist())
    # a band across the middle row (silhouettes, covered interior) and the ragged last row
    mid = scene.tiles_y // 2
    t.update(range(mid * scene.tiles_x + scene.tiles_x // 2 - 8, mid * scene.tiles_x + scene.tiles_x // 2 + 8))
    t.update(range((scene.tiles_y - 1) * scene.tiles_x, (scene.tiles_y - 1) * scene.tiles_x + 4))
    return np.array(sorted(t), np.int32)


@pytest.mark.slow
def test_c3_full():
    """The 1080p hybrid workload on every tile: z-buffer, records of all 1M
    Gaussians, every per-tile list, every pixel of rgb / depth / alpha and every
    gradient with the full upstream gradients."""
    s = _scene("c3")
    print("c3 full: GPU pass and oracle on all %d tiles" % (s.tiles_x * s.tiles_y), flush=True)
    gpu, ora, tiles = _run(s, 0, cull=True)
    rep = _check_all(s, 0, gpu, ora, tiles, True, "c3 full")
    assert P.compare_bins(s, 0, gpu) == 0
    assert rep["entries"] > 10_000_000


@pytest.mark.slow
@pytest.mark.parametrize("view", [0, 1, 2, 3])
def test_c5_full(view):
    """Each view of the 4-view 1080p workload (3M Gaussians, 499,280 faces) on every
    tile, as for C3."""
    s = _scene("c5")
    print("c5 view %d full: GPU pass and oracle on all %d tiles" % (view, s.tiles_x * s.tiles_y), flush=True)
    gpu, ora, tiles = _run(s, view, cull=True)
    _check_all(s, view, gpu, ora, tiles, True, "c5 view %d full" % view)
    assert P.compare_bins(s, view, gpu) == 0


# ---------------------------------------------------------------------------
# invariants and edge cases
# ---------------------------------------------------------------------------

def test_cull_invariance_and_determinism():
    """Culling on vs off: bitwise-equal images; forward bitwise repeatable."""
    import torch
    s = _scene("c2")
    r = _renderer(s)
    r.forward(0, cull=True)
    a = P.gpu_state(r)
    n_cull = r.n_keys
    r.forward(0, cull=False)
    b = P.gpu_state(r)
    assert r.n_keys > n_cull
    for k in ("rgb", "depth", "alpha", "T"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    r.forward(0, cull=True)
    c = P.gpu_state(r)
    for k in ("rgb", "depth", "alpha", "T", "last", "ids", "ranges", "face_id"):
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(c[k]).view(np.uint8)), k
    g = {k: torch.from_numpy(v).cuda() for k, v in s.grads[0].items()}
    r.forward(0, cull=True)
    r.backward(g["rgb"], g["depth"], g["alpha"])
    ga = P.to_np(r.g_rec).copy()
    r.forward(0, cull=False)
    r.backward(g["rgb"], g["depth"], g["alpha"])
    gb = P.to_np(r.g_rec)
    assert np.isfinite(ga).all() and np.isfinite(gb).all()
    assert np.allclose(ga, gb, rtol=1e-5, atol=1e-6 * np.abs(ga).max())


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_tiny_random_scenes(seed):
    s = tiny.random_tiny(seed, n_tri=8, n_gauss=16, size=32 + 7 * seed)  # ragged tiles
    gpu, ora, tiles = _run(s, 0, cull=True)
    _check_all(s, 0, gpu, ora, tiles, True, "tiny %d" % seed)


def _screen_soup(s, tris, rng):
    """Soup of triangles given in screen space (u, v, z) for the scene's identity camera."""
    pts = np.asarray(tris, np.float64).reshape(-1, 3)
    x = (pts[:, 0] - s.cx) * pts[:, 2] / s.fx
    y = (pts[:, 1] - s.cy) * pts[:, 2] / s.fy
    tiny.set_mesh(s, np.stack([x, y, pts[:, 2]], 1), np.arange(len(pts)).reshape(-1, 3),
                  vcolor=rng.uniform(size=(len(pts), 3)))


def test_thin_triangles_zbuffer():
    """Slivers: long thin triangles with a vertex far off screen (the z-buffer tests
    every pixel of their tiles), thin ones inside the image (tested on the pixels
    near their bounding box) and right triangles whose legs run along pixel-centre
    rows and columns (edge functions exactly zero there): face ids and depths equal
    the oracle's, which tests every pixel of every binned tile."""
    s = tiny.random_tiny(23, n_tri=2, n_gauss=10, size=48)
    rng = np.random.default_rng(23)
    tris = []
    for k in range(6):  # far vertex nearly on the line through two on-screen ones
        p0 = rng.uniform(2, 46, 2)
        p1 = rng.uniform(2, 46, 2)
        d = p1 - p0
        n = np.array([-d[1], d[0]]) / np.linalg.norm(d)
        p2 = p0 + 1e6 * d + rng.uniform(0.3e6, 1.5e6) * rng.choice([-1.0, 1.0]) * n  # 0.3-1.5 px wide on screen
        z = rng.uniform(2.5, 3.5)
        tris.append([[p0[0], p0[1], z], [p1[0], p1[1], z + 0.2], [p2[0], p2[1], z]])
    for k in range(10):  # thin slivers inside the image
        p0 = rng.uniform(1, 47, 2)
        p1 = rng.uniform(1, 47, 2)
        d = p1 - p0
        n = np.array([-d[1], d[0]]) / np.linalg.norm(d)
        p2 = p0 + rng.uniform(-1.0, 2.0) * d + rng.uniform(-0.05, 0.05) * n
        zz = rng.uniform(2.0, 4.0, 3)
        tris.append([[p0[0], p0[1], zz[0]], [p1[0], p1[1], zz[1]], [p2[0], p2[1], zz[2]]])
    for k in range(6):  # legs on pixel-centre lines
        x0, y0 = rng.integers(0, 40, 2) + 0.5
        a, b = rng.integers(1, 9, 2) * (1 if k % 2 else -1)
        z = 3.0 + 0.1 * k
        tris.append([[x0, y0, z], [x0 + a, y0, z], [x0, y0 + b, z]])
    _screen_soup(s, tris, rng)
    gpu, ora, tiles = _run(s, 0, cull=True)
    _check_all(s, 0, gpu, ora, tiles, True, "thin triangles")
    # the far-vertex slivers are thin enough that their tiles are tested in full
    vs = gpu["vscreen"].astype(np.float64)
    u, v = vs[0][s.faces], vs[1][s.faces]
    A = (u[1] - u[0]) * (v[2] - v[0]) - (v[1] - v[0]) * (u[2] - u[0])
    L2 = np.max([(u[(k + 1) % 3] - u[k]) ** 2 + (v[(k + 1) % 3] - v[k]) ** 2 for k in range(3)], 0)
    R_low = np.max(np.abs(u - 24.0) + np.abs(v - 24.0), 0) - 48.0  # below R for any tile
    full = np.abs(A) <= 2.0 ** -40 * R_low * L2
    assert full[:6].sum() >= 3, (A[:6], L2[:6])
    covered = np.unique(ora["face_id"][ora["face_id"] >= 0])
    assert np.isin(np.arange(6)[full[:6]], covered).any()  # some fully tested sliver is visible


def _lists_large_image(W, H, seed, name):
    """Lists of a large image on sampled tiles against the oracle's, culling on, with
    triangles covering whole tiles; returns (tiles, ranges, tile_dmax sample)."""
    import torch
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    rng = np.random.default_rng(seed)
    s = tiny.empty_scene(W, H, 2000.0, 2000.0, W / 2, H / 2, name=name)
    n = 3000
    u = np.concatenate([rng.uniform(0, W, n - 300), rng.uniform(0, W, 300)])
    v = np.concatenate([rng.uniform(0, H, n - 300), rng.uniform(H - 20, H, 300)])  # the last tile row too
    z = rng.uniform(2.0, 4.0, n)
    means = np.stack([(u - s.cx) * z / s.fx, (v - s.cy) * z / s.fy, z], 1)
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    sc = np.exp(rng.normal(-6.0, 0.4, size=(n, 3)))  # a few pixels on screen
    op = 1.0 / (1.0 + np.exp(-rng.normal(size=n)))
    tiny.set_gaussians(s, means, q, sc, op, rgb=rng.uniform(size=(n, 3)))
    tris = []
    for k in range(60):  # large triangles: fully covered tiles for the cull
        c = rng.uniform([0, 0], [W, H])
        r = rng.uniform(100, 400)
        a = rng.uniform(0, 2 * np.pi) + np.array([0, 2.1, 4.2])
        zz = rng.uniform(2.5, 3.5)
        tris.append([[c[0] + r * np.cos(t), c[1] + r * np.sin(t), zz] for t in a])
    _screen_soup(s, tris, rng)
    r = Renderer(DeviceScene(s))
    r.fit_lists(0, cull=True)
    torch.cuda.synchronize()
    T = r.T
    txn = (W + 15) // 16
    assert T == txn * ((H + 15) // 16)
    ranges = P.to_np(r.tile_ranges).reshape(-1, 2)
    ids = P.to_np(r.sorted_ids)
    tx = (u // 16).astype(int)
    ty = (v // 16).astype(int)
    near = np.unique(np.clip(ty, 0, (H + 15) // 16 - 1) * txn + np.clip(tx, 0, txn - 1))
    tiles = np.unique(np.concatenate([rng.choice(near, 250, replace=False), rng.integers(0, T, 50),
                                      near[near >= 65536][:40], near[-40:]])).astype(np.int32)
    cam = oracle.camera(s, 0)
    vs = oracle.project_vertices(cam, s.verts)
    zb = oracle.zbuffer(cam, vs, s.faces, s.face_mask, tiles=tiles, prefilter=True)
    dm = np.where(np.isnan(zb["tile_dmax"]), np.inf, zb["tile_dmax"]).astype(np.float32)
    assert np.array_equal(P.to_np(r.tile_dmax)[tiles].view(np.uint32), dm[tiles].view(np.uint32))
    pg = oracle.project_gaussians(cam, s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    order = oracle.depth_order(pg["rec"], pg["valid"])
    pre = oracle.tile_lists(cam, pg["rec"], pg["rect"], order, tiles, tile_dmax=dm, softness=s.softness)
    rep = P.compare_lists(s, {"ranges": ranges, "ids": ids}, {"lists_pre": pre}, tiles, True)
    print(name, rep, flush=True)
    assert rep["list_mismatch"] == 0 and rep["entries"] > 300
    assert int((dm[tiles] < np.inf).sum()) >= 5  # some sampled tiles are fully covered
    return tiles, ranges


def test_lists_above_65536_tiles():
    """A 4112 x 4096 image has 257 x 256 = 65792 tiles: the tile sort keeps 32-bit
    keys (16-bit at most 65536 tiles) and the count pass reads tile_dmax from memory
    (staged in LDS up to 10240 tiles).  Lists on sampled tiles, ids above 65535
    among them, are the oracle's."""
    tiles, ranges = _lists_large_image(4112, 4096, 41, "65792 tiles")
    hi = tiles[tiles >= 65536]
    assert len(hi) >= 20
    assert (ranges[hi, 1] > ranges[hi, 0]).sum() >= 10  # lists of tiles past 16-bit ids


def test_lists_above_10240_tiles():
    """A 2064 x 1296 image has 129 x 81 = 10449 tiles: 16-bit tile keys over 14 bits
    (two 7-bit passes), and more tiles than the count pass stages in LDS, so it reads
    tile_dmax from memory.  Lists on sampled tiles, the last ones among them, are the
    oracle's."""
    tiles, ranges = _lists_large_image(2064, 1296, 43, "10449 tiles")
    assert tiles.max() >= 10449 - 200
    assert (ranges[tiles[tiles >= 10240], 1] > 0).sum() >= 1


def test_backward_above_16384_tiles():
    """A 2080 x 2080 image has 130 x 130 = 16900 tiles, more than the backward's tile
    order keeps in registers (it reads the walk lengths in loops instead).  Forward
    and backward on sampled tiles against the oracle, upstream gradients zero
    elsewhere, so every Gaussian's gradient comes from the sampled tiles only."""
    W = H = 2080
    rng = np.random.default_rng(47)
    s = tiny.empty_scene(W, H, 1500.0, 1500.0, W / 2, H / 2, name="16900 tiles")
    n = 400
    u, v = rng.uniform(0, W, n), rng.uniform(0, H, n)
    z = rng.uniform(2.0, 4.0, n)
    means = np.stack([(u - s.cx) * z / s.fx, (v - s.cy) * z / s.fy, z], 1)
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    sc = np.exp(rng.normal(-4.5, 0.4, size=(n, 3)))  # a few tiles across on screen
    op = 1.0 / (1.0 + np.exp(-rng.normal(1.0, 1.0, size=n)))
    tiny.set_gaussians(s, means, q, sc, op, rgb=rng.uniform(size=(n, 3)))
    tris = []
    for k in range(40):
        c = rng.uniform([0, 0], [W, H])
        r = rng.uniform(60, 300)
        a = rng.uniform(0, 2 * np.pi) + np.array([0, 2.1, 4.2])
        zz = rng.uniform(2.5, 3.5)
        tris.append([[c[0] + r * np.cos(t), c[1] + r * np.sin(t), zz] for t in a])
    _screen_soup(s, tris, rng)
    s.grads = [scenes.upstream_grads(s, 0, 47)]
    T = s.tiles_x * s.tiles_y
    assert T == 16900
    txn = s.tiles_x
    near = np.unique(np.clip(v // 16, 0, s.tiles_y - 1).astype(int) * txn + np.clip(u // 16, 0, txn - 1).astype(int))
    tiles = np.unique(np.concatenate([rng.choice(near, 150, replace=False), rng.integers(0, T, 50),
                                      [T - 1]])).astype(np.int32)
    gpu, ora, tiles = _run(s, 0, tiles, masked=True)
    rep = _check_all(s, 0, gpu, ora, tiles, True, "16900 tiles")
    assert rep["entries"] > 150  # the sample reaches a couple of hundred list entries
    assert np.abs(gpu["g_rec"]).max() > 0


def test_no_mesh_plain_splatting():
    s = tiny.random_tiny(5, n_tri=1, n_gauss=40, size=48)
    s.verts, s.faces, s.vcolor = None, None, None
    gpu, ora, tiles = _run(s, 0, cull=True)
    _check_all(s, 0, gpu, ora, tiles, True, "no mesh")


def test_empty_gaussians_and_empty_mesh():
    s = tiny.random_tiny(6, n_tri=5, n_gauss=1, size=40)
    s.means = np.zeros((3, 0), np.float32)
    s.quats = np.zeros((4, 0), np.float32)
    s.scales = np.zeros((3, 0), np.float32)
    s.opacity = np.zeros(0, np.float32)
    s.sh = np.zeros((1, 3, 0), np.float32)
    gpu, ora, tiles = _run(s, 0, cull=True)
    _check_all(s, 0, gpu, ora, tiles, True, "N=0")


def test_softness_zero_and_sh_degrees():
    for deg in (0, 1, 2, 3):
        s = tiny.random_tiny(10 + deg, n_tri=6, n_gauss=24, size=40)
        rng = np.random.default_rng(deg)
        K = (deg + 1) ** 2
        s.sh = rng.normal(0, 0.3, size=(K, 3, s.N)).astype(np.float32)
        s.sh_degree = deg
        s.softness = 0.0 if deg == 1 else 0.5
        gpu, ora, tiles = _run(s, 0, cull=True)
        _check_all(s, 0, gpu, ora, tiles, True, "deg %d softness %g" % (deg, s.softness))


def test_list_overflow_reports_needed_size():
    """A list above its capacity is not written, reads as empty downstream, and its
    length is reported on the device; the renderer then grows it and succeeds."""
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    s = _scene("c1")
    r = Renderer(DeviceScene(s), pair_cap=1, key_cap=1)
    st = torch.cuda.current_stream().cuda_stream
    r.tile_tris.fill_(-7)
    G.gm_bin_triangles(r.ds.cams[0], r.ds.mesh, r.vscreen, r.tile_offsets, r.tile_tris, 1, r.counts[0:1],
                       r.ws_bin, st)
    torch.cuda.synchronize()
    n = int(r.counts[0].item())
    assert n > 1
    assert int(r.tile_tris[0].item()) == -7 and int(r.tile_offsets.abs().sum().item()) == 0
    r.forward(0)  # grows both lists and succeeds
    assert r.n_pairs == n and r.key_cap >= r.n_keys > 1
    k = r.n_keys
    # the sort with one slot: nothing written beyond it, every range empty, length reported
    r.sorted_ids.fill_(-7)
    G.gm_sort_tile_keys(r.ds.cams[0], r.N, r.rec, r.tile_dmax, s.softness, r.tile_ranges, r.sorted_ids, 1,
                        r.counts[1:2], r.ws_sort, st)
    torch.cuda.synchronize()
    assert int(r.counts[1].item()) == k
    assert int((r.sorted_ids[1:] != -7).sum().item()) == 0 and int(r.tile_ranges.abs().sum().item()) == 0
