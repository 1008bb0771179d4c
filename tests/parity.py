"""GPU-vs-oracle comparison helpers shared by the parity tests and the smoke check.

Rules (each exemption is counted and returned, never silent):
  * face ids bit-exact, except pixels whose two nearest oracle depths differ by
    <= 1e-6 relative (depth ties);
  * projected records: decision fields bit-exact, colour within 1e-6;
  * per-tile lists bit-exact without culling; with culling the GPU list is an
    ordered subset of the pre-cull list and differs from the oracle's post-cull
    list only at pairs whose cull ratio lies within 1e-3 of the threshold;
  * rgb / depth / alpha within 1e-4 absolute, except "straddle" pixels where an
    oracle skip/stop decision lies within STRADDLE relative of its threshold;
  * gradients: per plane ||d||_2 <= 1e-3 ||ref||_2 and elementwise
    |d| <= 1e-3 (|ref| + rms(ref)), except Gaussians listed in a tile that holds a
    straddle pixel.
"""
from __future__ import annotations

import numpy as np

import oracle

STRADDLE = 1e-5       # relative distance of an oracle decision to its threshold
DEPTH_TIE = 1e-6      # relative gap between the two nearest triangles
CULL_BAND = 1e-3      # relative distance of the cull ratio to 1
IMG_TOL = 1e-4
GRAD_TOL = 1e-3
REC_DECISION_FIELDS = [0, 1, 2, 3, 4, 5, 9, 10, 11, 12]


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_state(r, with_grads=False):
    """Copy every buffer of a Renderer that parity looks at to host numpy."""
    import torch
    torch.cuda.synchronize()
    N = r.N
    out = {
        "face_id": to_np(r.face_id), "zdepth": to_np(r.depth), "tile_dmax": to_np(r.tile_dmax),
        "tile_offsets": to_np(r.tile_offsets), "tile_tris": to_np(r.tile_tris[: r.n_pairs]),
        "rec": to_np(r.rec[:N]) if N else np.zeros((0, 16), np.float32),
        "ranges": to_np(r.tile_ranges), "ids": to_np(r.sorted_ids[: r.n_keys]),
        "rgb": to_np(r.out_rgb), "depth": to_np(r.out_depth), "alpha": to_np(r.out_alpha),
        "T": to_np(r.state_T), "last": to_np(r.state_last), "vscreen": to_np(r.vscreen),
        "n_keys": r.n_keys, "n_pairs": r.n_pairs,
    }
    if with_grads:
        out["g_rec"] = to_np(r.g_rec[:N]) if N else np.zeros((0, 13), np.float32)
        out["g_mesh_rgb"] = to_np(r.g_mesh_rgb)
        out["g_mesh_depth"] = to_np(r.g_mesh_depth)
    return out


def tile_pixel_mask(scene, tiles):
    m = np.zeros((scene.height, scene.width), bool)
    for t in np.asarray(tiles):
        ty, tx = divmod(int(t), scene.tiles_x)
        m[ty * 16:(ty + 1) * 16, tx * 16:(tx + 1) * 16] = True
    return m


def masked_grads(scene, view, tiles):
    """The scene's upstream gradients, zero outside ``tiles``."""
    g = scene.grads[view]
    m = tile_pixel_mask(scene, tiles)
    return {"rgb": np.where(m[..., None], g["rgb"], 0).astype(np.float32),
            "depth": np.where(m, g["depth"], 0).astype(np.float32),
            "alpha": np.where(m, g["alpha"], 0).astype(np.float32)}


def compare_vscreen(gpu, ora):
    a, b = gpu["vscreen"][:, : ora["vscreen"].shape[1]], ora["vscreen"]
    return int(np.count_nonzero(a.view(np.uint32) != b.view(np.uint32)))


def compare_zbuffer(scene, gpu, ora, tiles):
    m = tile_pixel_mask(scene, tiles)
    with np.errstate(invalid="ignore"):
        tie = (ora["z2"] - ora["z1"]) <= DEPTH_TIE * ora["z1"]
    gf, of = gpu["face_id"], ora["face_id"]
    bad = m & (gf != of) & ~tie
    exempt = int(np.count_nonzero(m & (gf != of) & tie))
    same = m & (gf == of)
    dbad = same & (gpu["zdepth"].view(np.uint32) != ora["depth"].view(np.uint32))
    t = np.asarray(tiles)
    dm_bad = int(np.count_nonzero(gpu["tile_dmax"][t].view(np.uint32) != ora["tile_dmax"][t].view(np.uint32)))
    return {"face_mismatch": int(np.count_nonzero(bad)), "tie_exempt": exempt,
            "depth_mismatch": int(np.count_nonzero(dbad)), "dmax_mismatch": dm_bad,
            "ties": m & tie}


def compare_bins(scene, view, gpu):
    cam = oracle.camera(scene, view)
    off, ids = oracle.tile_bins(cam, gpu["vscreen"][:, : scene.V], scene.faces, scene.face_mask)
    go = gpu["tile_offsets"]
    if not np.array_equal(go, off):
        return int(np.count_nonzero(go != off)) or 1
    bad = 0
    for t in range(len(off) - 1):
        a = np.sort(gpu["tile_tris"][go[t]:go[t + 1]])
        if not np.array_equal(a, ids[off[t]:off[t + 1]]):
            bad += 1
    return bad


def compare_records(gpu, ora, rgb_tol=1e-6):
    g, o = gpu["rec"], ora["rec"]
    valid = ora["valid"].astype(bool)
    gi = g.view(np.int32)
    lo, hi, nt = gi[:, 13], gi[:, 14], gi[:, 15]
    grect = np.stack([lo & 0xFFFF, lo >> 16, hi & 0xFFFF, hi >> 16], 1)
    res = {"valid_mismatch": int(np.count_nonzero((nt > 0) != valid)),
           "rect_mismatch": int(np.count_nonzero((grect != ora["rect"]).any(1))),
           "ntiles_mismatch": int(np.count_nonzero(
               nt != (ora["rect"][:, 2] - ora["rect"][:, 0]) * (ora["rect"][:, 3] - ora["rect"][:, 1])))}
    fb = g[valid][:, REC_DECISION_FIELDS].view(np.uint32) != o[valid][:, REC_DECISION_FIELDS].view(np.uint32)
    res["field_mismatch"] = int(np.count_nonzero(fb))
    res["rgb_maxdiff"] = float(np.abs(g[valid][:, 6:9].astype(np.float64) - ora["rgb64"][valid]).max()) \
        if valid.any() else 0.0
    res["rgb_ok"] = bool(res["rgb_maxdiff"] <= rgb_tol) and bool(np.isfinite(g[valid][:, :13]).all())
    return res


def _segments(lengths):
    """Segment index of every element of the concatenation of segments of ``lengths``."""
    return np.repeat(np.arange(len(lengths)), lengths)


def _gpu_lists(gpu, tiles):
    """The GPU's per-tile lists of ``tiles``, concatenated, and their lengths."""
    rg = gpu["ranges"][np.asarray(tiles)]
    lens = np.maximum(rg[:, 1] - rg[:, 0], 0).astype(np.int64)
    starts = rg[:, 0].astype(np.int64)
    idx = np.repeat(starts - np.concatenate([[0], np.cumsum(lens)[:-1]]), lens) + np.arange(int(lens.sum()))
    return gpu["ids"][idx] if len(idx) else np.zeros(0, np.int32), lens


def _list_mismatch_tiles(got, glens, exp, elens):
    """Indices (into the tile sample) of tiles whose GPU list differs from ``exp``."""
    bad = glens != elens
    same = ~bad
    if same.any():
        gseg, eseg = _segments(glens), _segments(elens)
        g_in, e_in = same[gseg], same[eseg]
        diff = got[g_in] != exp[e_in]  # both concatenations hold the same-length tiles in order
        if diff.any():
            bad[np.unique(gseg[g_in][diff])] = True
    return np.flatnonzero(bad)


def compare_lists(scene, gpu, ora, tiles, cull):
    """Per-tile lists of the sampled tiles (vectorised: a tile whose GPU list equals
    the oracle's exactly passes; only the others are examined one by one)."""
    off_pre, ids_pre, cq = ora["lists_pre"]
    tiles = np.asarray(tiles)
    lens_pre = np.diff(off_pre).astype(np.int64)
    got, glens = _gpu_lists(gpu, tiles)
    if not cull:
        bad = _list_mismatch_tiles(got, glens, ids_pre, lens_pre)
        return {"list_mismatch": int(len(bad)), "cull_exempt": 0, "entries": int(len(ids_pre))}
    keep_o = cq >= 1.0
    seg = _segments(lens_pre)
    exp = ids_pre[keep_o]
    elens = np.bincount(seg[keep_o], minlength=len(tiles)).astype(np.int64)
    suspects = _list_mismatch_tiles(got, glens, exp, elens)
    gstart = np.concatenate([[0], np.cumsum(glens)])
    bad, band_exempt = 0, 0
    for k in suspects:
        gl = got[gstart[k]:gstart[k + 1]]
        pre = ids_pre[off_pre[k]:off_pre[k + 1]]
        q = cq[off_pre[k]:off_pre[k + 1]]
        # ordered subset of the pre-cull list
        pos = {int(i): j for j, i in enumerate(pre)}
        idx = [pos.get(int(i), -1) for i in gl]
        if (np.asarray(idx) < 0).any() or (np.diff(idx) <= 0).any():
            bad += 1
            continue
        keep_g = np.zeros(len(pre), bool)
        keep_g[idx] = True
        diff = keep_g != (q >= 1.0)
        near = np.abs(q - 1.0) <= CULL_BAND
        if (diff & ~near).any():
            bad += 1
        band_exempt += int(np.count_nonzero(diff & near))
    return {"list_mismatch": bad, "cull_exempt": band_exempt, "entries": int(len(ids_pre))}


def compare_images(scene, gpu, ora, tiles, ties=None):
    """Every pixel of the sampled tiles is checked; a pixel that misses the tolerance
    is exempt only when the oracle marks it as a straddle (or a depth tie)."""
    c = ora["comp"]
    m = tile_pixel_mask(scene, tiles)
    strad = m & (c["margin"] < STRADDLE)
    if ties is not None:
        strad |= ties
    d_rgb = np.abs(gpu["rgb"].astype(np.float64) - c["rgb"]).max(-1)
    d_dep = np.abs(gpu["depth"].astype(np.float64) - c["depth"])
    d_alp = np.abs(gpu["alpha"].astype(np.float64) - c["alpha"])
    worst = np.maximum(np.maximum(d_rgb, d_dep), d_alp)
    fail = m & ~(worst <= IMG_TOL)
    used = fail & strad
    ok = m & ~used
    return {"img_bad": int(np.count_nonzero(fail & ~strad)), "straddle": int(np.count_nonzero(used)),
            "straddle_candidates": int(np.count_nonzero(strad)),
            "rgb_max": float(d_rgb[ok].max()) if ok.any() else 0.0,
            "depth_max": float(d_dep[ok].max()) if ok.any() else 0.0,
            "alpha_max": float(d_alp[ok].max()) if ok.any() else 0.0,
            "straddle_mask": strad, "fail_mask": fail}


def exempt_gaussians(scene, ora, tiles, strad_mask):
    """Ids listed in any sampled tile that holds a straddle pixel."""
    off, ids = ora["lists"]
    out = set()
    for k, t in enumerate(np.asarray(tiles)):
        ty, tx = divmod(int(t), scene.tiles_x)
        if strad_mask[ty * 16:(ty + 1) * 16, tx * 16:(tx + 1) * 16].any():
            out.update(ids[off[k]:off[k + 1]].tolist())
    return np.array(sorted(out), np.int64)


def compare_grads(scene, gpu, ora, tiles, strad_mask):
    """All Gaussians are checked; a Gaussian that misses the tolerance is exempt only
    when it is listed in a tile holding a straddle pixel."""
    c = ora["comp"]
    ref = c["grad"]
    got = gpu["g_rec"].astype(np.float64)
    ex = exempt_gaussians(scene, ora, tiles, strad_mask)
    exm = np.zeros(len(ref), bool)
    exm[ex] = True
    res = {"grad_exempt": 0, "planes_bad": [], "elem_bad": 0}
    used = np.zeros(len(ref), bool)
    for k in range(13):
        r, g = ref[:, k], got[:, k]
        d = g - r
        rms = np.sqrt(np.mean(r * r)) if len(r) else 0.0
        fail = ~(np.abs(d) <= GRAD_TOL * (np.abs(r) + rms) + 1e-12)  # NaN fails
        res["elem_bad"] += int(np.count_nonzero(fail & ~exm))
        used |= fail & exm
    res["grad_exempt"] = int(np.count_nonzero(used))
    keep = ~used
    for k in range(13):
        r, g = ref[keep, k], got[keep, k]
        nr = np.linalg.norm(r)
        if not np.linalg.norm(g - r) <= GRAD_TOL * nr + 1e-12:  # NaN fails
            res["planes_bad"].append((k, float(np.linalg.norm(g - r) / max(nr, 1e-30))))
    m = tile_pixel_mask(scene, tiles)
    for name, key in (("mesh_rgb", "g_mesh_rgb"), ("mesh_depth", "g_mesh_depth")):
        r = c[key][m]
        g = gpu[key][m].astype(np.float64)
        rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
        fail = ~(np.abs(g - r) <= GRAD_TOL * (np.abs(r) + rms) + 1e-9)  # NaN fails
        if fail.ndim > 1:
            fail = fail.any(-1)
        sm = strad_mask[m]
        res[name + "_bad"] = int(np.count_nonzero(fail & ~sm))
        res[name + "_exempt"] = int(np.count_nonzero(fail & sm))
    return res
