"""The composite forward as two calls, and the backward's clearing of the record
gradients.

gm_composite_hybrid_fwd is gm_shade_surface followed by
gm_composite_hybrid_fwd_shaded (the renderer shades on its second stream beside the
tile sort).  The pin is bitwise equality of every output and state buffer with the
single call over the same lists, whose own parity against the oracle the other GPU
tests establish.  The backward clears the record gradients in the launch that takes
the tile walks, also in a buffer that does not start on a 16-byte boundary: against
the renderer's own buffer the gradients agree up to the summation order of the float
atomics (|d| <= 1e-3 (|ref| + rms), the gradient rule of the parity tests), and no
float outside the buffer is written.
"""
import functools

import numpy as np
import pytest

import scenes

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _scene(name):
    return scenes.make_scene(name)


def _lit_c2():
    """c2 with vertex normals (the icosphere's radial directions) and the Phong light."""
    s = _scene("c2")
    v = s.verts.astype(np.float64)
    n = v - v.mean(1, keepdims=True)
    n /= np.linalg.norm(n, axis=0, keepdims=True)
    return scenes.Scene(**{**s.__dict__, "vnormal": n.astype(np.float32), "light": scenes._phong_light()})


def _bits(t):
    import torch
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("name", ["c1", "c2_lit", "c4"])
def test_split_forward_is_the_single_call(name, monkeypatch):
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd import pipeline
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer, _stream
    s = _lit_c2() if name == "c2_lit" else _scene(name)
    ds = DeviceScene(s)
    r = Renderer(ds)
    calls = []
    shaded = G.gm_composite_hybrid_fwd_shaded
    monkeypatch.setattr(pipeline.G, "gm_composite_hybrid_fwd_shaded",
                        lambda *a: (calls.append(1), shaded(*a))[1])
    v = len(s.views) - 1
    r.forward(v)
    torch.cuda.synchronize()
    assert calls, "the renderer did not take the two-call forward"
    got = {"rgb": r.out_rgb, "depth": r.out_depth, "alpha": r.out_alpha, "T": r.state_T, "last": r.state_last,
           "cm": r.state_cm}
    got = {k: t.clone() for k, t in got.items()}
    ref = {k: torch.full_like(t, -7) for k, t in got.items()}
    G.gm_composite_hybrid_fwd(ds.cams[v], r.rec, r.tile_ranges, r.sorted_ids, r.face_id, r.depth, ds.mesh,
                              r.vscreen, ds.light, s.bg, s.softness, ref["rgb"], ref["depth"], ref["alpha"],
                              ref["T"], ref["last"], ref["cm"], _stream())
    torch.cuda.synchronize()
    for k in got:
        assert torch.equal(_bits(got[k]), _bits(ref[k])), (name, k)
    covered = int((r.face_id >= 0).sum())
    assert covered > 0 and (s.N == 0 or int(r.state_last.sum()) > 0)


def test_shaded_forward_without_overlap_matches():
    # without the second stream the renderer takes the single call; same bits
    import torch
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    s = _lit_c2()
    ds = DeviceScene(s)
    a, b = Renderer(ds), Renderer(ds)
    a.forward(0)
    b.fit_lists(0)
    b.lists(0, True, overlap=False)
    b.composite_fwd(0)
    torch.cuda.synchronize()
    for k in ("out_rgb", "out_depth", "out_alpha", "state_T", "state_last", "state_cm"):
        assert torch.equal(_bits(getattr(a, k)), _bits(getattr(b, k))), k


def test_backward_clears_unaligned_record_gradients():
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer, _stream
    s = _scene("c2")
    ds = DeviceScene(s)
    r = Renderer(ds)
    g = ds.grads(0)
    r.step(0, g)
    torch.cuda.synchronize()
    N = s.N
    ref = r.g_rec[:N].clone()
    n = N * G.GM_GRAD
    # offsets 1-3 floats: 3-1 floats before the first 16-byte boundary and (n = 4k)
    # 1-3 after the last float4; offset 4: aligned
    buf = torch.empty(n + 8, device="cuda")
    g_rgb, g_depth = torch.empty_like(r.g_mesh_rgb), torch.empty_like(r.g_mesh_depth)
    rms = float(ref.pow(2).mean().sqrt())
    for off in (1, 2, 3, 4):
        buf.fill_(float("nan"))
        out = buf[off: off + n]
        G.gm_composite_hybrid_bwd(ds.cams[0], N, r.rec, r.tile_ranges, r.sorted_ids, r.face_id, r.depth,
                                  s.softness, r.state_T, r.state_last, r.state_cm, g["rgb"], g["depth"], g["alpha"],
                                  out, g_rgb, g_depth, r.ws_comp_bwd, _stream())
        torch.cuda.synchronize()
        got = out.view(N, G.GM_GRAD)
        assert bool(torch.isfinite(got).all()), off
        err = float(((got - ref).abs() / (ref.abs() + rms + 1e-30)).max())
        assert err <= 1e-3, (off, err)
        assert bool(torch.isnan(buf[:off]).all()) and bool(torch.isnan(buf[off + n:]).all()), off
    assert int((ref != 0).sum()) > 0
