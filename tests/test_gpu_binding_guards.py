"""The Python binding's checks of device tensors: a wrongly typed, permuted,
wrongly shaped or short tensor raises ValueError before any launch, and a correct
call still goes through."""
import pytest

import scenes

pytestmark = pytest.mark.gpu


def test_backward_rejects_bad_upstream_gradients():
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer, _stream
    s = scenes.make_scene("c1")
    ds = DeviceScene(s)
    r = Renderer(ds)
    g = ds.grads(0)
    r.forward(0)

    def call(g_rgb, g_depth=g["depth"], g_rec=r.g_rec):
        G.gm_composite_hybrid_bwd(ds.cams[0], s.N, r.rec, r.tile_ranges, r.sorted_ids, r.face_id, r.depth,
                                  s.softness, r.state_T, r.state_last, r.state_cm, g_rgb, g_depth, None, g_rec,
                                  r.g_mesh_rgb, r.g_mesh_depth, r.ws_comp_bwd, _stream())
    with pytest.raises(ValueError, match="dtype"):
        call(g["rgb"].double())
    with pytest.raises(ValueError, match="shape"):
        call(g["rgb"].permute(2, 0, 1).contiguous())
    with pytest.raises(ValueError, match="contiguous"):
        call(g["rgb"].permute(1, 0, 2).reshape(-1).view(s.width, s.height, 3).transpose(0, 1))
    with pytest.raises(ValueError, match="GPU tensor"):
        call(g["rgb"].cpu())
    with pytest.raises(ValueError, match="elements"):
        call(g["rgb"], g_rec=r.g_rec[: s.N - 1])
    with pytest.raises(ValueError, match="elements"):
        call(g["rgb"].reshape(-1)[:-3])
    call(g["rgb"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(r.g_rec[: s.N]).all())
