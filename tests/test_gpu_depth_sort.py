"""The depth sort against the oracle's depth order, on scenes large enough for the
multi-block scan (more than 131072 Gaussians), where the sort may skip its top-byte
pass on the device.

Every Gaussian covers the whole 64 x 64 image, so with culling off each tile's list
is the whole depth order of the listed Gaussians; one tile's list is compared with
oracle.depth_order (keys = bits of z_c, ties by index) element by element.  Three
depth ranges cover the two outcomes of the skip test: all listed depths in one
binade-pair sharing the keys' top byte (the pass is skipped), depths across 2.0 (two
top bytes: not skipped), and depths sharing the top byte with one depth whose key has
all ones in its low 24 bits (not skipped).  Depths are quantised so that many keys
tie, and some Gaussians lie behind the camera (unlisted, all-ones keys).
"""
import numpy as np
import pytest

import oracle
import parity as P
import tiny

pytestmark = pytest.mark.gpu

N = 150_000


def _scene(case, seed):
    rng = np.random.default_rng(seed)
    s = tiny.empty_scene(64, 64, 100.0, 100.0, 32.0, 32.0, name="depth sort " + case)
    if case == "one_top_byte":
        z = 2.5 + rng.integers(0, 64, N) / 64.0          # [2.5, 3.5): top byte 0x40
    elif case == "two_top_bytes":
        z = 1.25 + rng.integers(0, 160, N) / 64.0        # [1.25, 3.75): 0x3f and 0x40
    else:
        z = 4.0 + rng.integers(0, 200, N) / 64.0         # [4, 7.2): top byte 0x40 ...
        z[rng.integers(0, N)] = np.float32(np.uint32(0x40FFFFFF).view(np.float32))  # ... and low 24 bits all ones
    z = z.astype(np.float32).astype(np.float64)
    behind = rng.random(N) < 0.05
    z[behind] = -z[behind]                                # behind the camera: not listed
    u = rng.uniform(28, 36, N)
    v = rng.uniform(28, 36, N)
    means = np.stack([(u - 32.0) * np.abs(z) / 100.0, (v - 32.0) * np.abs(z) / 100.0, z], 1)
    q = np.tile([1.0, 0.0, 0.0, 0.0], (N, 1))
    sc = np.full((N, 3), 3.0)                             # ~100 px sigma: every tile of the image
    op = rng.uniform(0.2, 0.9, N)
    tiny.set_gaussians(s, means, q, sc, op, rgb=rng.uniform(size=(N, 3)))
    return s


@pytest.mark.parametrize("case", ["one_top_byte", "two_top_bytes", "low_bits_all_ones"])
def test_depth_order_matches_oracle(case):
    import torch
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    s = _scene(case, {"one_top_byte": 1, "two_top_bytes": 2, "low_bits_all_ones": 3}[case])
    cam = oracle.camera(s, 0)
    pg = oracle.project_gaussians(cam, s.means, s.quats, s.scales, s.opacity, s.sh, s.sh_degree)
    valid = pg["valid"].astype(bool)
    keys = pg["rec"][valid, 9].view(np.uint32)
    tops = np.unique(keys >> 24)
    low_ones = bool(((keys & 0xFFFFFF) == 0xFFFFFF).any())
    assert (len(tops), low_ones) == {"one_top_byte": (1, False), "two_top_bytes": (2, False),
                                     "low_bits_all_ones": (1, True)}[case]
    assert (~valid).sum() > 1000 and len(np.unique(keys)) < len(keys)  # unlisted ones and ties
    expect = oracle.depth_order(pg["rec"], pg["valid"])
    r = Renderer(DeviceScene(s))
    r.fit_lists(0, cull=False)
    torch.cuda.synchronize()
    ranges = P.to_np(r.tile_ranges).reshape(-1, 2)
    ids = P.to_np(r.sorted_ids)
    for t in (0, 5, r.T - 1):
        a, b = ranges[t]
        got = ids[a:b]
        print(case, "tile", t, "entries", len(got), "expected", len(expect), flush=True)
        assert len(got) == len(expect)
        assert np.array_equal(got, expect)
