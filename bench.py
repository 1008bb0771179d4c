"""Benchmark: hybrid render fwd+bwd throughput at 1080p on one MI355X.

One step = the whole hot path over one view of the workload, inputs resident in
HBM: gm_bin_triangles -> gm_raster_zbuffer, beside them on a second stream
gm_project_gaussians -> gm_sort_depth (then gm_shade_surface once the z-buffer is
done), then gm_sort_tiles -> gm_composite_hybrid_fwd_shaded ->
gm_composite_hybrid_bwd.

Prints one JSON line with the metric (K steps timed with no event inside them),
per-stage times (HIP events between the stages on the two streams, over K further
steps, whose own time is reported beside), a roofline entry for the dominant
kernel, the measured HBM traffic of a whole step when its counter summary matches
the kernel sources, and the CPU oracle's throughput on a bounded sample of the same
workload.

``--copy-calibration`` instead runs a plain device copy of known size; profiled
with ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` it gives the factors that turn
those counters into bytes.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (counts packed FMA)
# Stages of one step on the library's (main) stream, and on the second stream that
# runs the projection and the depth half of the sort beside the mesh's binning and
# z-buffer, then the mesh shading beside the tile sort; "wait_lists" is the time the
# main stream waits for the second one, "wait_zbuffer" the second one's wait for the
# z-buffer.
STAGES = ["bin", "zbuffer", "wait_lists", "sort", "fwd", "bwd"]
STAGES_AA = ["bin", "zbuffer", "antialias", "wait_lists", "sort", "fwd", "bwd", "antialias_bwd"]
SIDE_STAGES = ["project", "sort_depth", "wait_zbuffer", "shade"]  # shade: the composite's first half
SIDE_STAGES_AA = ["project", "sort_depth"]  # the layer call shades the mesh on the main stream

WORKLOADS = {
    "c3": "1920x1080, 200k-face displaced sphere (vertex colour + Phong), 1M Gaussians SH3",
    "c5": "1920x1080, 4 displaced spheres (499,280 faces, Phong), 3M Gaussians SH3, one of 4 views",
    "c2": "512x512, 5120-face icosphere, 100k Gaussians",
    "c4": "800x800 textured 4096-triangle soup, no Gaussians, one of 16 views",
}

# Algorithmic flops of the composite per (pixel, list entry) pair, counted on the
# definition (transcendentals count 1): evaluating a pair (offset, quadratic form,
# exp, opacity clamp, split numerator, Phi, alpha_F) is 26; the reverse-mode
# gradient of an included pair (transmittance recovery, colour/depth terms, conic,
# mean, opacity, split terms) is 62 more; the forward's accumulation of an included
# pair is 10 more.
FLOPS_EVAL = 26
FLOPS_GRAD = 62
FLOPS_ACCUM = 10


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--view", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=0,
                    help="tiles in the oracle's timed sample (0: every tile of the view)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--batch-views", action="store_true",
                    help="one step = every view of the workload with one batched projection")
    ap.add_argument("--antialias", action="store_true",
                    help="the path with analytic edge antialiasing (two-layer composite)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))


def source_digest(kernel_file):
    with open(os.path.join(ROOT, "differentiable_hybrid_mesh_amd", "csrc", kernel_file), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, kernel_file, config):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary of this
    kernel, or None when the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m or not b or m.group(1) != source_digest(kernel_file):
        return None
    return float(b.group(1))


def sources_digest():
    """SHA-256 (first 16 hex digits) of all kernel sources, *.hip then *.h in name order."""
    import glob
    h = hashlib.sha256()
    d = os.path.join(ROOT, "differentiable_hybrid_mesh_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(d, "*.hip"))) + sorted(glob.glob(os.path.join(d, "*.h"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_step_traffic(config):
    """HBM bytes of one whole step (every kernel) from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None when any kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_step_{config}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"sources_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_step:\s*([0-9.e+]+)", text)
    if not m or not b or m.group(1) != sources_digest():
        return None
    return float(b.group(1))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the renderer has no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import scenes
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer

    torch.cuda.set_device(0)
    scene = scenes.make_scene(args.config)
    if args.batch_views:
        main_batch(args, scene)
        return
    view = args.view % len(scene.views)
    ds = DeviceScene(scene)
    r = Renderer(ds)
    g = ds.grads(view)
    cam = ds.cams[view]
    torch.cuda.synchronize()

    aa = args.antialias and scene.F > 0
    stages = STAGES_AA if aa else STAGES
    side_stages = SIDE_STAGES_AA if aa else SIDE_STAGES

    def step(ev=None, ev_side=None):
        # the calls of Renderer.lists() with the overlap, spelled out to mark stages
        main, side = torch.cuda.current_stream(), r._side_stream()
        st = main.cuda_stream
        i, j = [0], [0]

        def mark():
            if ev is not None:
                ev[i[0]].record(main)
            i[0] += 1

        def mark_side():
            if ev_side is not None:
                ev_side[j[0]].record(side)
            j[0] += 1
        r._ev_main.record(main)
        side.wait_event(r._ev_main)
        with torch.cuda.stream(side):
            mark_side()
            r.project(view)
            mark_side()
            r.sort_depth(view)
            mark_side()
            r._ev_side.record(side)
        mark()
        G.gm_bin_triangles(cam, ds.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.pair_cap, r.counts[0:1],
                           r.ws_bin, st)
        mark()
        G.gm_raster_zbuffer(cam, ds.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.face_id, r.depth,
                            r.tile_dmax, r.ws_zb, st)
        mark()
        if aa:
            r.antialias(view)
            mark()
        else:
            r._ev_zb.record(main)
            side.wait_event(r._ev_zb)
            with torch.cuda.stream(side):
                mark_side()
                r.shade(view)
                mark_side()
                r._ev_shade.record(side)
            r._shaded = view
        main.wait_event(r._ev_side)
        mark()
        r.sort_tiles(view, True)
        mark()
        if aa:
            r.composite_fwd_aa(view)
            mark()
            r.composite_bwd_aa(view, g["rgb"], g["depth"], g["alpha"])
            mark()
            r.antialias_bwd(view)
            mark()
        else:
            r.composite_fwd(view)
            mark()
            r.composite_bwd(view, g["rgb"], g["depth"], g["alpha"])
            mark()
        r.fetch_counts()  # list lengths to pinned host memory, checked after the run

    # list capacities first (binning, projection and sorting only), then the warm-up;
    # no step synchronises: the lengths are read back once the stream has finished
    r.fit_lists(view, True, antialias=aa)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    while not r.read_counts():
        step()
        torch.cuda.synchronize()

    # timed region: K whole steps, no events inside (each event is one more packet
    # for the command processor); then K more steps with events between the stages
    # on both streams for the per-stage times
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for k in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if not r.read_counts():  # every timed step used the same capacities as the warm-up
        raise RuntimeError("a list outgrew its capacity inside the timed region")
    ms = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    evs_side = [[torch.cuda.Event(enable_timing=True) for _ in range(len(side_stages) + 1)]
                for _ in range(args.steps)]
    e_inst = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e_inst[0].record()
    for k in range(args.steps):
        step(evs[k], evs_side[k])
    e_inst[1].record()
    torch.cuda.synchronize()
    ms_instrumented = e_inst[0].elapsed_time(e_inst[1]) / args.steps
    stage_ms = {s: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, s in enumerate(stages)}
    stage_ms.update({s: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs_side]))
                     for i, s in enumerate(side_stages)})

    px = scene.width * scene.height
    value = px / (ms * 1e-3) / 1e6
    N = scene.N
    nvis = int((r.rec[:N, 15].view(torch.int32) > 0).sum().item()) if N else 0
    if aa:  # pairs up to each pixel's last included entry of either layer
        st_aa = r.state_aa.view(-1, 8)
        walked = int(torch.maximum(st_aa[:, 1].view(torch.int32), st_aa[:, 3].view(torch.int32)).sum().item())
    else:
        walked = int(r.state_last.sum().item())  # pairs up to each pixel's last included entry
    incl_frac = included_fraction(scene, view) if N else 0.0

    # compulsory HBM bytes per stage (each input read once, each output written once)
    V, F, HW, T, K, Pp = scene.V, scene.F, px, r.T, r.n_keys, r.n_pairs
    d = scene.sh_degree
    shb = 12 * (d + 1) ** 2 if d >= 0 else 12
    alg_bytes = {
        "bin": 12 * V + 12 * V + 12 * F + 8 * Pp + 4 * T,
        "zbuffer": 4 * Pp + 12 * F + 12 * V + 8 * HW + 4 * T,
        "project": N * (12 + 16 + 12 + 4 + shb + 64),
        "sort_depth": 64 * N,
        "sort": 28 * K + 8 * T,
        # the composite forward: ids, records, face id + depth, colour behind (state_cm),
        # rgb + depth + alpha, state_T + state_last
        "fwd": 4 * K + 64 * nvis + 8 * HW + 12 * HW + 20 * HW + 8 * HW,
        "bwd": 4 * K + 64 * nvis + 8 * HW + 8 * HW + 12 * HW + 20 * HW + 52 * nvis + 16 * HW,
    }
    if not aa:  # face ids read, state_cm written, screen vertices, colours and faces once
        alg_bytes["shade"] = 4 * HW + 12 * HW + 24 * V + 12 * F
    if aa:
        # the layer: face ids, depths and colours of each pixel and its neighbours
        # (one read each), screen vertices and faces once, the layer written (32 B)
        alg_bytes["antialias"] = 4 * HW + 4 * HW + 12 * HW + 12 * V + 12 * F + 32 * HW
        # the two-layer composite reads the layer instead of face id, depth and colour,
        # and keeps 32 B of state instead of 8
        alg_bytes["fwd"] += 32 * HW - 20 * HW + 24 * HW
        alg_bytes["bwd"] += 32 * HW - 20 * HW + 24 * HW + 32 * HW
        alg_bytes["antialias_bwd"] = 4 * HW + 4 * HW + 12 * HW + 32 * HW + 12 * V + 12 * F + 16 * HW + 8 * V
    alg_flops = {
        "fwd": walked * FLOPS_EVAL + walked * incl_frac * FLOPS_ACCUM,
        "bwd": walked * FLOPS_EVAL + walked * incl_frac * FLOPS_GRAD,
    }
    # dominant single kernel: bin and sort are chains of many small kernels, the other
    # stages are one main kernel each (the backward adds the tile walk, which also
    # clears the record gradients, and the tile order: a few percent)
    dom = max(["zbuffer", "project", "fwd", "bwd"], key=stage_ms.get)
    kname = {"bwd": "k_composite_bwd", "fwd": "k_composite_fwd", "sort": "gm_sort_tiles",
             "project": "k_project_gaussians", "zbuffer": "k_zbuffer", "bin": "gm_bin_triangles"}[dom]
    kfile = {"bwd": "gm_composite.hip", "fwd": "gm_composite.hip", "sort": "gm_sort.hip",
             "project": "gm_project.hip", "zbuffer": "gm_raster.hip", "bin": "gm_raster.hip"}[dom]
    dom_s = stage_ms[dom] * 1e-3
    if dom in alg_flops:
        ach = alg_flops[dom] / dom_s / 1e12
        roof = {"kernel": kname, "bound": "alu", "achieved": round(ach, 3), "peak": FP32_VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP32_VALU_PEAK_TFLOPS, 4)}
    else:
        ach = alg_bytes[dom] / dom_s / 1e9
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    tname = kname
    if aa and dom in ("fwd", "bwd"):  # the two-layer instantiation of the composite kernel
        roof["kernel"] = kname + "<two-layer>"
        tname = kname + "_aa"
    roof["traffic"] = measured_traffic(tname, kfile, args.config)
    roof["units"] = {"walked_pairs": walked, "included_fraction": round(incl_frac, 4)} if dom in alg_flops \
        else {"algorithmic_bytes": alg_bytes[dom]}
    roof["launch_ms"] = round(stage_ms[dom], 4)

    next_stages = {"project_bwd": time_project_bwd(r, scene, view, args.steps)} if N else {}
    if scene.F:
        next_stages["mesh_bwd"] = time_mesh_bwd(r, scene, view, args.steps)
        if aa:
            next_stages["vscreen_bwd_ms"] = time_call(lambda: G.gm_vscreen_bwd(
                cam, ds.mesh, r.g_vscreen, r.gm_verts, torch.cuda.current_stream().cuda_stream), args.steps)

    total_alg = sum(alg_bytes.values())
    # measured HBM traffic of a whole step (rocprofv3 counters, separate run) over the
    # unprofiled step time; only for the default-path workload it was taken on
    step_bytes = None if aa else measured_step_traffic(args.config)
    hbm_measured = None if step_bytes is None else {
        "bytes_per_step": step_bytes, "GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "source": f"profiles/traffic_step_{args.config}.md"}
    out = {
        "metric": "hybrid render Mpixels/s fwd+bwd at 1080p",
        "value": round(value, 3), "unit": "Mpixels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64 scene generators)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}" + (", edge antialiasing" if aa else ""),
                   "view": view,
                   "width": scene.width, "height": scene.height, "faces": scene.F, "gaussians": N,
                   "tri_tile_pairs": r.n_pairs, "keys": r.n_keys, "visible": nvis, "parallelism": "single GPU"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "ms_per_step_with_stage_events": round(ms_instrumented, 4),
        "hbm_algorithmic_GBps": round(total_alg / (ms * 1e-3) / 1e9, 1),
        "hbm_algorithmic_frac": round(total_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_measured": hbm_measured,
        "roofline": roof,
        "next_stages": next_stages,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(scene, view, args.cpu_tiles)
    print(json.dumps(out), flush=True)


def main_batch(args, scene):
    """Every view of the workload per step: one gm_project_gaussians_multi for all
    views, then per view the lists, composite forward and backward, with each view's
    mesh half and lists overlapped with the previous view's composite
    (Renderer.views_step_pipelined).  Also times the views one after
    another, and the batched projection against the per-view projection loop it
    replaces."""
    import torch
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
    ds = DeviceScene(scene)
    r = Renderer(ds)
    views = list(range(len(scene.views)))
    grads = [ds.grads(v) for v in views]
    r.fit_lists_views(views)
    for _ in range(max(args.warmup, 1)):
        r.views_step_pipelined(views, grads)
    torch.cuda.synchronize()
    if not r.read_counts():
        raise RuntimeError("a list outgrew its capacity after fitting")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        r.views_step_pipelined(views, grads)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if not r.read_counts():
        raise RuntimeError("a list outgrew its capacity inside the timed region")
    ms = t0.elapsed_time(t1) / args.steps
    # the same views one after another (each view's halves overlapped only with each
    # other), for comparison
    t0.record()
    for _ in range(args.steps):
        r.views_step_async(views, grads)
    t1.record()
    torch.cuda.synchronize()
    if not r.read_counts():
        raise RuntimeError("a list outgrew its capacity inside the timed region")
    ms_serial = t0.elapsed_time(t1) / args.steps
    px = len(views) * scene.width * scene.height
    value = px / (ms * 1e-3) / 1e6

    # the projection alone: batched call vs one call per view (events on the stream)
    N, d = scene.N, scene.sh_degree
    shb = 12 * (d + 1) ** 2 if d >= 0 else 12
    per_in = 12 + 16 + 12 + 4 + shb
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(args.steps):
        r.project_views(views)
    e[1].record()
    for _ in range(args.steps):
        for v in views:
            r.project(v)
    e[2].record()
    torch.cuda.synchronize()
    ms_multi = e[0].elapsed_time(e[1]) / args.steps
    ms_loop = e[1].elapsed_time(e[2]) / args.steps
    b_multi = N * (per_in + 64 * len(views))
    b_loop = len(views) * N * (per_in + 64)
    ach = b_multi / (ms_multi * 1e-3) / 1e9
    out = {
        "metric": "hybrid render Mpixels/s fwd+bwd at 1080p",
        "value": round(value, 3), "unit": "Mpixels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64 scene generators)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}; all {len(views)} views per step, "
                               "one batched projection, views pipelined", "views": len(views), "width": scene.width,
                   "height": scene.height, "faces": scene.F, "gaussians": N, "parallelism": "single GPU"},
        "roofline": {"kernel": "k_project_gaussians_multi", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "units": {"algorithmic_bytes": b_multi}, "launch_ms": round(ms_multi, 4)},
        "views_one_after_another_ms_per_step": round(ms_serial, 4),
        "projection": {"batched_ms": round(ms_multi, 4), "per_view_loop_ms": round(ms_loop, 4),
                       "batched_algorithmic_bytes": b_multi, "loop_algorithmic_bytes": b_loop,
                       "speedup": round(ms_loop / ms_multi, 3)},
        "wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def time_call(fn, steps):
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) / steps, 4)


def time_project_bwd(r, scene, view, steps):
    """The projection backward (gradients of the Gaussian parameters from the record
    gradients of the composite backward), timed on its own: it follows the composite
    backward in a training step but is not part of the rendering step measured above.
    HBM-bound; algorithmic bytes per listed Gaussian = inputs read (means, quaternion,
    scales, SH coefficients, the record's colour and list words, 13 record gradients)
    plus outputs written (3 + 4 + 3 + 1 + 3K gradients); an unlisted one reads its list
    word and writes zeros."""
    import torch
    N = scene.N
    K = 1 if scene.sh_degree < 0 else (scene.sh_degree + 1) ** 2
    nl = int((r.rec[:N, 15].view(torch.int32) > 0).sum().item())
    per_listed = 4 * (3 + 4 + 3 + 3 * K + 4 + 13) + 4 * (3 + 4 + 3 + 1 + 3 * K)
    per_unlisted = 4 + 4 * (3 + 4 + 3 + 1 + 3 * K)
    nbytes = nl * per_listed + (N - nl) * per_unlisted
    r.project_bwd(view)  # allocates the gradient buffers
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        r.project_bwd(view)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "k_project_bwd", "ms": round(ms, 4), "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "listed": nl}


def time_mesh_bwd(r, scene, view, steps):
    """The mesh-side backward (gradients of vertex positions, colours, normals, texels
    and light from the composite backward's per-pixel dL/dc_m and dL/dD), timed on its
    own like the projection backward.  Algorithmic bytes: the face-id buffer, the two
    per-pixel gradients at covered pixels, the mesh's faces and per-vertex inputs once,
    and the per-vertex gradients written once (the float atomics' traffic is the
    implementation's, not the algorithm's)."""
    import torch
    V, F = scene.V, scene.F
    covered = int((r.face_id >= 0).sum().item())
    per_vertex = 12 * (1 + (scene.vcolor is not None) + (scene.vnormal is not None))
    nbytes = (4 * scene.width * scene.height + 16 * covered + 12 * F + per_vertex * V + per_vertex * V)
    r.mesh_bwd(view)  # allocates the gradient buffers
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        r.mesh_bwd(view)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "k_mesh_bwd", "ms": round(ms, 4), "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "covered_pixels": covered}


def included_fraction(scene, view, ntiles=48):
    """Included / walked pairs of the reverse pass, counted by the oracle on a fixed
    sample of tiles of the same view (used to weight the per-pair flop figures)."""
    import oracle
    T = scene.tiles_x * scene.tiles_y
    rng = np.random.default_rng(5)
    tiles = np.sort(rng.choice(T, size=min(ntiles, T), replace=False)).astype(np.int32)
    res = oracle.render_view(scene, view, tiles=tiles, cull=True, backward=False)
    c = res["comp"]
    m = c["n_last"] >= 0
    w = int(c["n_last"][m].sum())
    return float(c["n_incl"][m].sum()) / w if w else 0.0


def cpu_baseline(scene, view, ntiles):
    """The oracle (fwd+bwd, OpenMP on the host cores) on a bounded sample of tiles."""
    import oracle
    T = scene.tiles_x * scene.tiles_y
    rng = np.random.default_rng(123)
    n = T if ntiles <= 0 else min(ntiles, T)
    tiles = np.sort(rng.choice(T, size=n, replace=False)).astype(np.int32)
    t = time.perf_counter()
    oracle.render_view(scene, view, tiles=tiles, cull=True, backward=True)
    dt = time.perf_counter() - t
    px = len(tiles) * 256
    return {"value": round(px / dt / 1e6, 6), "unit": "Mpixels/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(tiles)} of {T} 16x16 tiles of view {view} ({px} px): projection and depth order of "
                      f"all Gaussians, z-buffer, lists, composite and reverse mode of those tiles; {dt:.1f} s"}


if __name__ == "__main__":
    main()
