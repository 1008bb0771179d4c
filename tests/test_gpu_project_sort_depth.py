"""gm_project_sort_depth against gm_project_gaussians followed by gm_sort_depth: the
records and the depth order (and so the tile lists built from it) bit for bit, on
the 512x512 and 1920x1080 workloads and on an empty Gaussian set."""
import numpy as np
import pytest
import torch

import scenes
from differentiable_hybrid_mesh_amd import _lib as G
from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer

pytestmark = pytest.mark.gpu


def _lists(r):
    torch.cuda.synchronize()
    n = int(r.counts[1].item())
    return r.rec.clone(), r.tile_ranges.clone(), r.sorted_ids[:n].clone()


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_fused_equals_two_calls(name):
    s = scenes.make_scene(name)
    print(f"project_sort_depth {name}", flush=True)
    ds = DeviceScene(s)
    r = Renderer(ds)
    r.lists(0)  # sizes the buffers
    torch.cuda.synchronize()
    # the two calls
    r.project(0)
    r.sort_depth(0)
    r.sort_tiles(0, True)
    rec_a, rng_a, ids_a = _lists(r)
    # the fused call on poisoned buffers
    r.rec.fill_(float("nan"))
    r.ws_sort.fill_(0x7F)
    r.project_sort_depth(0)
    r.sort_tiles(0, True)
    rec_b, rng_b, ids_b = _lists(r)
    assert torch.equal(rec_a.view(torch.int32), rec_b.view(torch.int32))
    assert torch.equal(rng_a, rng_b)
    assert torch.equal(ids_a, ids_b)


def test_fused_empty_gaussians():
    s = scenes.make_scene("c1")
    ds = DeviceScene(s)
    r = Renderer(ds)
    r.lists(0)
    torch.cuda.synchronize()
    e = torch.empty(0, device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream().cuda_stream
    G.gm_project_sort_depth(ds.cams[0], 0, e, e, e, e, e, s.sh_degree, e, r.key_cap, r.ws_sort, stream)
    G.gm_sort_tiles(ds.cams[0], 0, e, r.tile_dmax, s.softness, r.tile_ranges, r.sorted_ids, r.key_cap,
                    r.counts[1:2], r.ws_sort, stream)
    torch.cuda.synchronize()
    assert int(r.counts[1].item()) == 0
    assert int(r.tile_ranges.abs().sum().item()) == 0
