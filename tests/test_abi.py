"""The C-ABI library loads, exports every call include/gm.h declares, and rejects
bad arguments on the host before any GPU work (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gm.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gm_status|size_t|const char\*|int32_t)\s+(gm_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def G():
    from differentiable_hybrid_mesh_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _lib.lib()
    return _lib


def test_header_declares_the_six_calls():
    d = _declared()
    for name in ("gm_bin_triangles", "gm_raster_zbuffer", "gm_project_gaussians", "gm_sort_tile_keys",
                 "gm_composite_hybrid_fwd", "gm_composite_hybrid_bwd"):
        assert name in d


def test_library_exports_every_declared_symbol(G):
    L = G.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert set(_declared()) == set(G.EXPORTS)
    assert G.gm_version() == 100


def test_workspace_queries_are_host_only(G):
    a = G.gm_bin_triangles_ws(100, 200, 64, 64)
    b = G.gm_sort_tile_keys_ws(500, 10000, 64, 64)
    assert a > 0 and b > 0
    assert G.gm_sort_tile_keys_ws(500, 20000, 64, 64) > b
    assert G.gm_mipmaps_floats(1024) == sum((1024 >> l) ** 2 * 3 for l in range(11))


def _cam(G, w=64, h=64):
    from differentiable_hybrid_mesh_amd.pipeline import make_camera
    return make_camera(w, h, 64.0, 64.0, 32.0, 32.0, [1, 0, 0, 0, 1, 0, 0, 0, 1], [0, 0, 0])


def test_argument_errors_before_any_launch(G):
    L = G.lib()
    cam = _cam(G)
    # NULL camera
    assert L.gm_project_gaussians(None, 1, 1, 1, 1, 1, 1, 0, 1, None) == G.GM_ERR_ARG
    assert b"camera" in L.gm_last_error()
    # sh_degree out of range
    assert L.gm_project_gaussians(C.byref(cam), 1, 1, 1, 1, 1, 1, 4, 1, None) == G.GM_ERR_ARG
    assert b"sh_degree" in L.gm_last_error()
    # negative N
    assert L.gm_project_gaussians(C.byref(cam), -1, 1, 1, 1, 1, 1, 0, 1, None) == G.GM_ERR_ARG
    # zero-sized image
    bad = _cam(G, 0, 64)
    assert L.gm_raster_zbuffer(C.byref(bad), None, None, None, None, None, None, None, None, 0, None) == G.GM_ERR_ARG
    # z-buffer workspace missing or too small
    mz = G.GmMesh()
    zws = G.gm_raster_zbuffer_ws(64, 64)
    assert zws == 256  # 16 tiles of int32, one 256-byte block
    assert L.gm_raster_zbuffer(C.byref(cam), C.byref(mz), None, 16, None, 16, 16, 16, None, zws, None) == G.GM_ERR_ARG
    assert L.gm_raster_zbuffer(C.byref(cam), C.byref(mz), None, 16, None, 16, 16, 16, 16, zws - 1,
                               None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    # workspace too small
    m = G.GmMesh()
    assert L.gm_bin_triangles(C.byref(cam), C.byref(m), 16, 16, 16, 0, 16, 16, 1, None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    # missing count pointer
    assert L.gm_bin_triangles(C.byref(cam), C.byref(m), 16, 16, 16, 0, None, 16, 1 << 20, None) == G.GM_ERR_ARG
    # negative softness
    assert L.gm_sort_tile_keys(C.byref(cam), 0, None, None, C.c_float(-1.0), 16, None, 0, 16, 16,
                               1 << 20, None) == G.GM_ERR_ARG
    # the two halves of the sort: workspace too small, negative softness
    assert L.gm_sort_depth(C.byref(cam), 10, 16, 100, 16, 16, None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    # projection and depth sort in one call: the projection's checks, then the sort's
    assert L.gm_project_sort_depth(C.byref(cam), -1, 16, 16, 16, 16, 16, 0, 16, 100, 16, 1 << 20,
                                   None) == G.GM_ERR_ARG
    assert L.gm_project_sort_depth(C.byref(cam), 10, 16, 16, 16, 16, 16, 4, 16, 100, 16, 1 << 20,
                                   None) == G.GM_ERR_ARG
    assert b"sh_degree" in L.gm_last_error()
    assert L.gm_project_sort_depth(C.byref(cam), 10, 16, 16, 16, 16, 16, 0, 16, 100, 16, 16, None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    assert L.gm_sort_tiles(C.byref(cam), 0, None, None, C.c_float(-1.0), 16, None, 0, 16, 16,
                           1 << 20, None) == G.GM_ERR_ARG
    assert b"softness" in L.gm_last_error()
    # the two halves of the composite forward: NULL face_id / bg / state_cm, a textured
    # mesh without uv; NULL state_cm, negative softness, a NULL output
    m3 = G.GmMesh()
    bg = (C.c_float * 3)(0.0, 0.0, 0.0)
    assert L.gm_shade_surface(C.byref(cam), None, C.byref(m3), None, None, bg, 16, None) == G.GM_ERR_ARG
    assert L.gm_shade_surface(C.byref(cam), 16, C.byref(m3), None, None, None, 16, None) == G.GM_ERR_ARG
    assert L.gm_shade_surface(C.byref(cam), 16, C.byref(m3), None, None, bg, None, None) == G.GM_ERR_ARG
    assert b"state_cm" in L.gm_last_error()
    m3.F, m3.faces, m3.mips, m3.tex_size = 1, 16, 16, 8
    assert L.gm_shade_surface(C.byref(cam), 16, C.byref(m3), 16, None, bg, 16, None) == G.GM_ERR_ARG
    assert b"uv" in L.gm_last_error()
    assert L.gm_shade_surface(C.byref(_cam(G, 64, 0)), 16, C.byref(m3), 16, None, bg, 16, None) == G.GM_ERR_ARG
    assert L.gm_composite_hybrid_fwd_shaded(C.byref(cam), 16, 16, 16, 16, 16, C.c_float(1.0), None, 16, 16, 16, 16,
                                            16, None) == G.GM_ERR_ARG
    assert b"state_cm" in L.gm_last_error()
    assert L.gm_composite_hybrid_fwd_shaded(C.byref(cam), 16, 16, 16, 16, 16, C.c_float(-1.0), 16, 16, 16, 16, 16,
                                            16, None) == G.GM_ERR_ARG
    assert b"softness" in L.gm_last_error()
    assert L.gm_composite_hybrid_fwd_shaded(C.byref(cam), 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, None, 16, 16,
                                            16, None) == G.GM_ERR_ARG
    assert b"output" in L.gm_last_error()
    # texture side not a power of two
    assert L.gm_build_mipmaps(16, 100, 16, None) == G.GM_ERR_ARG
    # rec misaligned
    assert L.gm_project_gaussians(C.byref(cam), 1, 16, 16, 16, 16, 16, 0, 17, None) == G.GM_ERR_ARG
    # projection backward: degree out of range, a NULL output, logit chain without opacity
    bw = [16] * 5
    assert L.gm_project_gaussians_bwd(C.byref(cam), 1, 16, 16, 16, 16, 16, 5, 16, 16, *bw, None, None,
                                      None) == G.GM_ERR_ARG
    assert L.gm_project_gaussians_bwd(C.byref(cam), 1, 16, 16, 16, 16, 16, 0, 16, 16, 16, None, 16, 16, 16,
                                      None, None, None) == G.GM_ERR_ARG
    assert L.gm_project_gaussians_bwd(C.byref(cam), 1, 16, 16, 16, None, 16, 0, 16, 16, *bw, None, 16,
                                      None) == G.GM_ERR_ARG
    assert b"opacity" in L.gm_last_error()
    # batched projection: NULL camera array, negative view count, an invalid camera
    # among valid ones, degree out of range, misaligned rec
    cams = (G.GmCamera * 3)(_cam(G), _cam(G, 64, 0), _cam(G))
    assert L.gm_project_gaussians_multi(None, 1, 1, 16, 16, 16, 16, 16, 0, 16, None) == G.GM_ERR_ARG
    assert L.gm_project_gaussians_multi(cams, -1, 1, 16, 16, 16, 16, 16, 0, 16, None) == G.GM_ERR_ARG
    assert L.gm_project_gaussians_multi(cams, 3, 1, 16, 16, 16, 16, 16, 0, 16, None) == G.GM_ERR_ARG
    assert L.gm_project_gaussians_multi(cams, 1, 1, 16, 16, 16, 16, 16, 4, 16, None) == G.GM_ERR_ARG
    assert b"sh_degree" in L.gm_last_error()
    assert L.gm_project_gaussians_multi(cams, 1, 1, 16, 16, 16, 16, 16, 0, 17, None) == G.GM_ERR_ARG
    # nothing to do: no views, or no Gaussians (no pointer is touched)
    assert L.gm_project_gaussians_multi(cams, 0, 5, None, None, None, None, None, 0, None, None) == G.GM_OK
    assert L.gm_project_gaussians_multi(cams, 1, 0, None, None, None, None, None, 0, None, None) == G.GM_OK


def test_antialias_argument_errors(G):
    L = G.lib()
    cam = _cam(G)
    m = G.GmMesh()
    m.V, m.F = 3, 1
    # adjacency: NULL faces / adj, workspace too small
    assert L.gm_edge_adjacency(C.byref(m), 16, 16, 1, None) == G.GM_ERR_ARG
    assert L.gm_edge_adjacency(None, 16, 16, 1 << 20, None) == G.GM_ERR_ARG
    m0 = G.GmMesh()
    assert L.gm_edge_adjacency(C.byref(m0), None, None, 0, None) == G.GM_OK  # F = 0: nothing to do
    m.faces, m.verts = 16, 16
    # the layer: missing adjacency, misaligned layer
    assert L.gm_antialias(C.byref(cam), C.byref(m), 16, None, None, 16, 16, 16, 16, None, None, None) == G.GM_ERR_ARG
    assert L.gm_antialias(C.byref(cam), C.byref(m), 16, 16, None, 16, 16, 16, 17, None, None, None) == G.GM_ERR_ARG
    assert L.gm_antialias(C.byref(cam), C.byref(m), 16, 16, None, 16, 16, 16, 16, 17, None, None) == G.GM_ERR_ARG
    # two-layer composite: NULL layer, misaligned state, negative softness
    assert L.gm_composite_hybrid_fwd_aa(C.byref(cam), 16, 16, 16, None, 16, C.c_float(1.0), 16, 16, 16, 16,
                                        None) == G.GM_ERR_ARG
    assert L.gm_composite_hybrid_fwd_aa(C.byref(cam), 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, 16, 17,
                                        None) == G.GM_ERR_ARG
    assert L.gm_composite_hybrid_bwd_aa(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(-1.0), 16, 16, None, None, 16,
                                        16, 16, 1 << 20, None) == G.GM_ERR_ARG
    assert b"softness" in L.gm_last_error()
    # composite reverse modes: workspace missing or too small
    need = G.gm_composite_hybrid_bwd_ws(64, 64)
    assert need >= 2 * 16 * 4
    assert L.gm_composite_hybrid_bwd_aa(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, None, None, 16,
                                        16, 16, need - 1, None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    assert L.gm_composite_hybrid_bwd(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, 16, 16, None,
                                     None, 16, None, None, None, need, None) == G.GM_ERR_ARG
    assert b"workspace" in L.gm_last_error()
    # antialiasing reverse mode: workspace too small, NULL screen-vertex gradient
    ws = G.gm_antialias_bwd_ws(64, 64)
    assert ws == 64 * 64 * 32
    assert L.gm_antialias_bwd(C.byref(cam), C.byref(m), 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, ws - 1,
                              None) == G.GM_ERR_ARG
    assert L.gm_antialias_bwd(C.byref(cam), C.byref(m), 16, 16, 16, 16, 16, 16, 16, 16, None, 16, ws,
                              None) == G.GM_ERR_ARG
    assert L.gm_antialias_bwd(C.byref(cam), C.byref(m), 16, None, 16, 16, 16, 16, 16, 16, 16, 16, ws,
                              None) == G.GM_ERR_ARG
    assert b"pairs" in L.gm_last_error()
    # the vertex chain: NULL verts
    m.verts = None
    assert L.gm_vscreen_bwd(C.byref(cam), C.byref(m), 16, 16, None) == G.GM_ERR_ARG
    assert G.gm_edge_adjacency_ws(10) > 0


def test_noalloc_backward_rejects_on_the_host(G):
    """The fixed-scratch backward checks its arguments and the image size (at most
    GM_NOALLOC_MAX_TILES tiles) before it touches the device."""
    L = G.lib()
    text = open(HEADER).read()
    assert re.search(r"#define GM_NOALLOC_MAX_TILES 65536", text)
    args = (1, 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, 16, 16, None, None, 16, None, None, None)
    big = G.GmCamera(4112, 4096, 4000.0, 4000.0, 2056.0, 2048.0)
    big.R[0] = big.R[4] = big.R[8] = 1.0
    big.near_z = 0.01
    assert L.gm_composite_hybrid_bwd_noalloc(C.byref(big), *args) == G.GM_ERR_ARG
    assert b"tiles" in L.gm_last_error()
    cam = _cam(G)
    # NULL upstream gradient, NULL record gradients, negative softness: rejected first
    assert L.gm_composite_hybrid_bwd_noalloc(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, 16, None,
                                             None, None, 16, None, None, None) == G.GM_ERR_ARG
    assert L.gm_composite_hybrid_bwd_noalloc(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(1.0), 16, 16, 16, 16,
                                             None, None, None, None, None, None) == G.GM_ERR_ARG
    assert L.gm_composite_hybrid_bwd_noalloc(C.byref(cam), 1, 16, 16, 16, 16, 16, C.c_float(-1.0), 16, 16, 16, 16,
                                             None, None, 16, None, None, None) == G.GM_ERR_ARG


def test_binding_rejects_bad_tensors_before_the_call(G):
    """The Python binding refuses host tensors, non-tensors, missing required tensors
    and images of the wrong shape with ValueError (a GPU would fault on a host
    pointer or read past a short buffer)."""
    import torch
    from differentiable_hybrid_mesh_amd.pipeline import make_camera
    cam = make_camera(64, 48, 64.0, 64.0, 32.0, 24.0, [1, 0, 0, 0, 1, 0, 0, 0, 1], [0, 0, 0])
    with pytest.raises(ValueError, match="GPU tensor"):
        G.dev(torch.zeros(4), "x", G.F32, 4)
    with pytest.raises(ValueError, match="torch tensor"):
        G.dev(np_array := __import__("numpy").zeros(4, "float32"), "x", G.F32, 4)
    assert np_array.shape == (4,)
    with pytest.raises(ValueError, match="required"):
        G.dev(None, "x", G.F32, 4)
    assert G.dev(None, "x", G.F32, 4, optional=True) is None
    # an image laid out (3, H, W) instead of (H, W, 3) is caught by its shape
    with pytest.raises(ValueError, match="shape"):
        G.img(torch.zeros(3, 48, 64), "g_rgb", cam, 3)
    with pytest.raises(ValueError, match="shape"):
        G.img(torch.zeros(64, 48), "g_depth", cam, 1)
    # whole calls: a host upstream gradient never reaches the library
    t = torch.zeros(48, 64)
    with pytest.raises(ValueError):
        G.gm_composite_hybrid_bwd(cam, 1, t, t, t, t, t, 1.0, t, t, t, torch.zeros(48, 64, 3), None, None, t, None,
                                  None, torch.zeros(G.gm_composite_hybrid_bwd_ws(64, 48), dtype=torch.uint8), None)
    with pytest.raises(ValueError):
        G.gm_composite_hybrid_bwd_noalloc(cam, 1, t, t, t, t, t, 1.0, t, t, t, torch.zeros(48, 64, 3), None, None,
                                          t, None, None, None)
