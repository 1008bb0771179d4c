"""The counting build of the composite forward (gm_composite_hybrid_fwd_stats): its
outputs are the uncounted call's bit for bit, and its count of included (pixel,
entry) pairs equals the oracle's per-pixel included counts summed over the image
(pixels the oracle marks as straddling a decision threshold may differ by the
entries that straddle)."""
import numpy as np
import pytest

import oracle
import scenes
import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_stats_forward_counts_and_outputs(name):
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer, _stream
    s = scenes.make_scene(name)
    ds = DeviceScene(s)
    r = Renderer(ds)
    r.forward(0)
    torch.cuda.synchronize()
    ref = {k: getattr(r, k).clone() for k in ("out_rgb", "out_depth", "out_alpha", "state_T", "state_last")}
    out = {k: torch.full_like(v, float("nan")) if v.dtype == torch.float32 else torch.full_like(v, -7)
           for k, v in ref.items()}
    stats = torch.zeros(3, dtype=torch.int64, device="cuda")
    G.gm_composite_hybrid_fwd_stats(ds.cams[0], r.rec, r.tile_ranges, r.sorted_ids, r.face_id, r.depth, s.softness,
                                    r.state_cm, out["out_rgb"], out["out_depth"], out["out_alpha"], out["state_T"],
                                    out["state_last"], stats, _stream())
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(out[k].view(torch.int32), ref[k].view(torch.int32)), k
    inc, ev, staged = (int(x) for x in stats.tolist())
    ora = oracle.render_view(s, 0, cull=True, backward=False)
    c = ora["comp"]
    n_incl = c["n_incl"]
    strad = c["margin"] < P.STRADDLE
    want = int(n_incl[n_incl >= 0].sum())
    print(name, "included", inc, "oracle", want, "evaluated", ev, "staged", staged, "straddle px", int(strad.sum()),
          flush=True)
    assert abs(inc - want) <= int(strad.sum())
    assert staged <= r.n_keys and ev >= inc / 64
