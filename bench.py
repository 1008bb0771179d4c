"""Benchmark: hybrid render fwd+bwd throughput on one MI355X.

One step = the whole hot path over every view of the workload, inputs resident in
HBM.  Per view: gm_bin_triangles -> gm_raster_zbuffer, beside them on a second
stream gm_project_sort_depth (then gm_shade_surface once the z-buffer is done),
then gm_sort_tiles -> gm_composite_hybrid_fwd_shaded ->
gm_composite_hybrid_bwd.  The one-view workloads (64x64, 512x512 and the default
1920x1080 sphere) time that sequence; the multi-view ones (the 800x800 soup's 16
views, the 1920x1080 four-sphere scene's 4 views) time the pipelined pass that
projects every view in one launch and overlaps each view's mesh half and lists with
the previous view's composite.

Prints one JSON line per workload: the metric over K steps timed with no event
inside them; the median and 10th / 90th percentiles of the step time and of every
stage (HIP events between the stages, over K further steps whose own mean is
reported beside); a roofline entry for the dominant kernel, timed on its own stream
with HIP events, with its work units counted on the GPU by the counting build of
the composite; the measured HBM traffic of a whole step when its counter summary
matches the kernel sources; and the CPU oracle's throughput on a bounded sample of
the same workload.

``--all-configs`` prints one line for each workload (each measured in a process of
its own).  ``--copy-calibration`` instead
runs a plain device copy of known size; profiled with ``rocprofv3 --pmc FETCH_SIZE``
/ ``WRITE_SIZE`` it gives the factors that turn those counters into bytes.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# fp32 vector peak attainable without packed fp32 instructions (disabled in this
# build): 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 78.6
FP32_VALU_PACKED_TFLOPS = 157.3  # the published fp32 vector figure (packed FMA)
# Stages of one view on the library's (main) stream, and on the second stream that
# runs the projection and the depth half of the sort beside the mesh's binning and
# z-buffer, then the mesh shading beside the tile sort; "wait_lists" is the time the
# main stream waits for the second one, "wait_zbuffer" the second one's wait for the
# z-buffer.
STAGES = ["bin", "zbuffer", "wait_lists", "sort", "fwd", "bwd"]
STAGES_AA = ["bin", "zbuffer", "antialias", "wait_lists", "sort", "fwd", "bwd", "antialias_bwd"]
SIDE_STAGES = ["project_sort_depth", "wait_zbuffer", "shade"]  # shade: the composite's first half
SIDE_STAGES_AA = ["project_sort_depth"]  # the layer call shades the mesh on the main stream

WORKLOADS = {
    "c1": "64x64, 200 random triangles (vertex colour), 500 Gaussians",
    "c2": "512x512, 5120-face icosphere (vertex colour), 100k Gaussians",
    "c3": "1920x1080, 200k-face displaced sphere (vertex colour + Phong), 1M Gaussians SH3",
    "c4": "800x800 textured 4096-triangle soup (stochastic masks), no Gaussians, 16 views per step",
    "c5": "1920x1080, 4 displaced spheres (499,280 faces, Phong), 3M Gaussians SH3, 4 views per step",
}
MULTI_VIEW = ("c4", "c5")

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
    ap.add_argument("--all-configs", action="store_true", help="one JSON line per workload")
    ap.add_argument("--view", type=int, default=0, help="view of a one-view run (--single-view)")
    ap.add_argument("--single-view", action="store_true",
                    help="time one view of a multi-view workload instead of all its views per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=0,
                    help="tiles in the oracle's timed sample (0: every tile of one view)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--batch-views", action="store_true", help="kept for compatibility: the multi-view "
                                                                "workloads always time all their views per step")
    ap.add_argument("--antialias", action="store_true",
                    help="the path with analytic edge antialiasing (two-layer composite), one view")
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


def measured_traffic(kernel, config):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary of this
    kernel, or None when any kernel source changed since it was taken (a kernel's
    traffic also depends on what the kernels before it produce, e.g. the lists)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"sources_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m or not b or m.group(1) != sources_digest():
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


def pct(xs):
    """Median, 10th and 90th percentiles (ms)."""
    a = np.asarray(xs, np.float64)
    return {"p50": round(float(np.percentile(a, 50)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the renderer has no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.all_configs:
        # one child process per workload: the streams a process creates are spread
        # over the GPU's hardware queues in creation order, so a workload measured
        # after others in one process can find its streams sharing a queue
        import subprocess
        rc = 0
        for name in WORKLOADS:
            argv = [sys.executable, "-u", os.path.abspath(__file__), "--config", name, "--steps", str(args.steps),
                    "--warmup", str(args.warmup), "--cpu-tiles", str(args.cpu_tiles)]
            if args.no_cpu_baseline:
                argv.append("--no-cpu-baseline")
            rc |= subprocess.run(argv).returncode
        sys.exit(rc)
    import torch
    torch.cuda.set_device(0)
    print(json.dumps(run_config(args, args.config)), flush=True)


class Bench:
    """One workload's device state and its per-view step with stage events."""

    def __init__(self, scene, antialias=False):
        import torch
        from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer
        self.torch = torch
        self.scene = scene
        self.ds = DeviceScene(scene)
        self.r = Renderer(self.ds)
        self.grads = [self.ds.grads(v) for v in range(len(scene.views))]
        self.aa = antialias and scene.F > 0
        self.stages = STAGES_AA if self.aa else STAGES
        self.side_stages = SIDE_STAGES_AA if self.aa else SIDE_STAGES

    def step_view(self, view, ev=None, ev_side=None):
        """The calls of Renderer.lists() with the overlap, then the composite forward and
        backward, spelled out to mark stages with events."""
        from differentiable_hybrid_mesh_amd import _lib as G
        torch, r, ds = self.torch, self.r, self.ds
        g = self.grads[view]
        cam = ds.cams[view]
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
        r._single()
        r._ev_main.record(main)
        side.wait_event(r._ev_main)
        with torch.cuda.stream(side):
            mark_side()
            r.project_sort_depth(view)
            mark_side()
            r._ev_side.record(side)
        mark()
        G.gm_bin_triangles(cam, ds.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.pair_cap, r.counts[0:1],
                           r.ws_bin, st)
        mark()
        G.gm_raster_zbuffer(cam, ds.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.face_id, r.depth,
                            r.tile_dmax, r.ws_zb, st)
        mark()
        if self.aa:
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
        if self.aa:
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


def run_config(args, name):
    import torch
    import scenes
    scene = scenes.make_scene(name)
    multi = name in MULTI_VIEW and not args.single_view and not args.antialias
    views = list(range(len(scene.views))) if multi else [args.view % len(scene.views)]
    b = Bench(scene, antialias=args.antialias)
    r = b.r
    if multi:
        def step():
            r.views_step_pipelined(views, b.grads)
        r.fit_lists_views(views)
    else:
        def step():
            b.step_view(views[0])
        r.fit_lists(views[0], True, antialias=b.aa)
    # warm-up; no step synchronises: the list lengths are read back once the stream
    # has finished, and a list that outgrew its capacity is enlarged before timing
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    while not r.read_counts():
        step()
        torch.cuda.synchronize()

    # timed region: K whole steps, no events inside
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if not r.read_counts():  # every timed step used the same capacities as the warm-up
        raise RuntimeError("a list outgrew its capacity inside the timed region")
    ms = t0.elapsed_time(t1) / args.steps
    counts = r.counts_host[: r._rows].tolist()

    # step-time distribution: K more steps, one event between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for k in range(args.steps):
        step()
        evs[k + 1].record()
    torch.cuda.synchronize()
    step_dist = [evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)]

    # per-stage times: every view one after another with events between the stages on
    # both streams (the instrumented steps' own time is reported beside)
    nst = max(1, args.steps // len(views))
    ev_main = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(b.stages) + 1)] for _ in views]
               for _ in range(nst)]
    ev_side = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(b.side_stages) + 1)] for _ in views]
               for _ in range(nst)]
    e_inst = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e_inst[0].record()
    for k in range(nst):
        for j, v in enumerate(views):
            b.step_view(v, ev_main[k][j], ev_side[k][j])
    e_inst[1].record()
    torch.cuda.synchronize()
    ms_instrumented = e_inst[0].elapsed_time(e_inst[1]) / nst
    stage_times = {s: [e[i].elapsed_time(e[i + 1]) for row in ev_main for e in row] for i, s in enumerate(b.stages)}
    stage_times.update({s: [e[i].elapsed_time(e[i + 1]) for row in ev_side for e in row]
                        for i, s in enumerate(b.side_stages)})
    stage_ms = {s: pct(x) for s, x in stage_times.items()}
    stage_mean = {s: float(np.mean(x)) for s, x in stage_times.items()}

    # the last view's buffers hold its lists and state: work units and the dominant
    # kernel's launch time are taken there
    last_view = views[-1]
    px_view = scene.width * scene.height
    value = len(views) * px_view / (ms * 1e-3) / 1e6
    N = scene.N
    recs = [r.rec_views[k] for k in range(len(views))] if multi else [r.rec]
    nvis = [int((x[:N, 15].view(torch.int32) > 0).sum().item()) if N else 0 for x in recs]
    if b.aa:  # pairs up to each pixel's last included entry of either layer
        st_aa = r.state_aa.view(-1, 8)
        walked = int(torch.maximum(st_aa[:, 1].view(torch.int32), st_aa[:, 3].view(torch.int32)).sum().item())
        units = {"walked_pairs": walked}
    else:
        walked = int(r.state_last.sum().item())  # pairs up to each pixel's last included entry
        units = composite_units(b, last_view) if N else {"walked_pairs": walked}
    incl = units.get("included_pairs", 0)

    alg = algorithmic_bytes(scene, r, counts, nvis, b.aa)
    total_alg = sum(sum(v.values()) for v in alg)
    alg_flops = {"fwd": walked * FLOPS_EVAL + incl * FLOPS_ACCUM, "bwd": walked * FLOPS_EVAL + incl * FLOPS_GRAD}

    # dominant single kernel by stage time (the sort and binning are chains of many
    # small kernels; the other stages are one main kernel each)
    dom = max(["zbuffer", "project_sort_depth", "fwd", "bwd"], key=lambda s: stage_mean.get(s, 0.0))
    roof = roofline(b, dom, last_view, alg[-1], alg_flops, units, args)

    step_bytes = None if b.aa else measured_step_traffic(name)
    hbm_measured = None if step_bytes is None else {
        "bytes_per_step": step_bytes, "GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "source": f"profiles/traffic_step_{name}.md"}
    out = {
        "metric": "hybrid render Mpixels/s fwd+bwd at 1080p" if scene.height == 1080
        else "hybrid render Mpixels/s fwd+bwd",
        "value": round(value, 3), "unit": "Mpixels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64 scene generators)",
        "config": {"workload": f"{name}: {WORKLOADS[name]}" + (", edge antialiasing" if b.aa else "")
                   + ("" if multi or len(scene.views) == 1 else f", view {views[0]} of {len(scene.views)}"),
                   "views_per_step": len(views), "width": scene.width, "height": scene.height,
                   "faces": scene.F, "gaussians": N, "tri_tile_pairs": [c[0] for c in counts],
                   "keys": [c[1] for c in counts], "visible": nvis, "parallelism": "single GPU"},
        "step_ms": pct(step_dist),
        "view_ms": round(ms / len(views), 4),
        "stage_ms": stage_ms,
        "ms_per_view_with_stage_events": round(ms_instrumented / len(views), 4),
        "hbm_algorithmic_GBps": round(total_alg / (ms * 1e-3) / 1e9, 1),
        "hbm_algorithmic_frac": round(total_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_measured": hbm_measured,
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if multi and N:
        out["projection"] = time_projection(b, views, args.steps)
    if not multi:
        ns = {"project_bwd": time_project_bwd(r, scene, views[0], args.steps)} if N else {}
        if scene.F:
            ns["mesh_bwd"] = time_mesh_bwd(r, scene, views[0], args.steps)
        for st in ns.values():  # HBM bytes per launch from the committed counters, when current
            st["traffic"] = measured_traffic(st["kernel"], name)
        out["next_stages"] = ns
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(scene, views[0], args.cpu_tiles, len(views))
    return out


def composite_units(b, view):
    """Work units of the composite on the view whose state the renderer holds,
    counted on the GPU: walked pairs (sum over pixels of the index of the last
    included entry) from the forward state, and the counting build of the forward
    (gm_composite_hybrid_fwd_stats, one launch outside the timed region): included
    pairs, entries evaluated wave-wide, entries staged."""
    import torch
    from differentiable_hybrid_mesh_amd import _lib as G
    from differentiable_hybrid_mesh_amd.pipeline import _stream
    r, s = b.r, b.scene
    stats = torch.zeros(3, dtype=torch.int64, device="cuda")
    out = [torch.empty_like(t) for t in (r.out_rgb, r.out_depth, r.out_alpha, r.state_T, r.state_last)]
    G.gm_composite_hybrid_fwd_stats(b.ds.cams[view], r.rec, r.tile_ranges, r.sorted_ids, r.face_id, r.depth,
                                    s.softness, r.state_cm, *out, stats, _stream())
    torch.cuda.synchronize()
    inc, ev, staged = (int(x) for x in stats.tolist())
    walked = int(r.state_last.sum().item())
    return {"walked_pairs": walked, "included_pairs": inc, "included_fraction": round(inc / max(walked, 1), 4),
            "wave_entries_fwd": ev, "entries_staged_fwd": staged, "counted_by": "gm_composite_hybrid_fwd_stats"}


def algorithmic_bytes(scene, r, counts, nvis, aa):
    """Compulsory HBM bytes per stage and view (each input read once, each output
    written once), from each view's own counts."""
    out = []
    V, F, HW, T = scene.V, scene.F, scene.width * scene.height, r.T
    N, d = scene.N, scene.sh_degree
    shb = 12 * (d + 1) ** 2 if d >= 0 else 12
    for (Pp, K), nv in zip(counts, nvis):
        a = {
            "bin": 12 * V + 12 * V + 12 * F + 8 * Pp + 4 * T,
            "zbuffer": 4 * Pp + 12 * F + 12 * V + 8 * HW + 4 * T,
            # the projection's inputs and records, and the depth sort's keys and ids
            "project_sort_depth": N * (12 + 16 + 12 + 4 + shb + 64) + 8 * N,
            "sort": 28 * K + 8 * T,
            # the composite forward: ids, records, face id + depth, colour behind (state_cm),
            # rgb + depth + alpha, state_T + state_last
            "fwd": 4 * K + 64 * nv + 8 * HW + 12 * HW + 20 * HW + 8 * HW,
            "bwd": 4 * K + 64 * nv + 8 * HW + 8 * HW + 12 * HW + 20 * HW + 52 * nv + 16 * HW,
        }
        if not aa:  # face ids read, state_cm written, screen vertices, colours and faces once
            a["shade"] = 4 * HW + 12 * HW + 24 * V + 12 * F
        else:
            # the layer: face ids, depths and colours of each pixel and its neighbours
            # (one read each), screen vertices and faces once, the layer written (32 B)
            a["antialias"] = 4 * HW + 4 * HW + 12 * HW + 12 * V + 12 * F + 32 * HW
            # the two-layer composite reads the layer instead of face id, depth and colour,
            # and keeps 32 B of state instead of 8
            a["fwd"] += 32 * HW - 20 * HW + 24 * HW
            a["bwd"] += 32 * HW - 20 * HW + 24 * HW + 32 * HW
            a["antialias_bwd"] = 4 * HW + 4 * HW + 12 * HW + 32 * HW + 12 * V + 12 * F + 16 * HW + 8 * V
        out.append(a)
    return out


KERNEL_OF = {"bwd": "k_composite_bwd", "fwd": "k_composite_fwd", "project_sort_depth": "k_project_gaussians",
             "zbuffer": "k_zbuffer"}


def roofline(b, dom, view, alg_bytes, alg_flops, units, args):
    """Roofline entry of the dominant kernel, its launch timed on its own (K launches
    on the current stream between two HIP events, after the timed steps, on the
    buffers of ``view``)."""
    import torch
    r = b.r
    g = b.grads[view]
    launch = {
        "bwd": (lambda: r.composite_bwd_aa(view, g["rgb"], g["depth"], g["alpha"])) if b.aa else
               (lambda: r.composite_bwd(view, g["rgb"], g["depth"], g["alpha"])),
        "fwd": (lambda: r.composite_fwd_aa(view)) if b.aa else (lambda: r.composite_fwd_shaded(view)),
        "project_sort_depth": lambda: r.project_sort_depth(view),
        "zbuffer": lambda: r.bin_and_zbuffer(view),
    }[dom]
    launch_ms = time_call(launch, args.steps)
    kname = KERNEL_OF[dom]
    if dom in alg_flops and units.get("included_pairs") is not None:
        ach = alg_flops[dom] / (launch_ms * 1e-3) / 1e12
        roof = {"kernel": kname, "bound": "alu", "achieved": round(ach, 3), "peak": FP32_VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP32_VALU_PEAK_TFLOPS, 4),
                "frac_of_packed_fp32_peak": round(ach / FP32_VALU_PACKED_TFLOPS, 4)}
    else:
        nbytes = alg_bytes[dom] if dom != "zbuffer" else alg_bytes["bin"] + alg_bytes["zbuffer"]
        ach = nbytes / (launch_ms * 1e-3) / 1e9
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
        units = {"algorithmic_bytes": nbytes}
    tname = kname + ("_aa" if b.aa and dom in ("fwd", "bwd") else "")
    roof["traffic"] = measured_traffic(tname, b.scene.name)
    roof["units"] = units
    roof["launch_ms"] = round(launch_ms, 4)
    roof["launch"] = "gm_composite_hybrid_bwd (tile walk + order + composite)" if dom == "bwd" else dom
    return roof


def time_projection(b, views, steps):
    """The batched projection of every view against one projection call per view."""
    import torch
    r, scene = b.r, b.scene
    N, d = scene.N, scene.sh_degree
    shb = 12 * (d + 1) ** 2 if d >= 0 else 12
    per_in = 12 + 16 + 12 + 4 + shb
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(steps):
        r.project_views(views)
    e[1].record()
    for _ in range(steps):
        for v in views:
            r.project(v)
    e[2].record()
    torch.cuda.synchronize()
    ms_multi = e[0].elapsed_time(e[1]) / steps
    ms_loop = e[1].elapsed_time(e[2]) / steps
    b_multi = N * (per_in + 64 * len(views))
    ach = b_multi / (ms_multi * 1e-3) / 1e9
    return {"kernel": "k_project_gaussians_multi", "batched_ms": round(ms_multi, 4),
            "per_view_loop_ms": round(ms_loop, 4), "batched_algorithmic_bytes": b_multi,
            "loop_algorithmic_bytes": len(views) * N * (per_in + 64), "achieved_GBps": round(ach, 1),
            "frac": round(ach / HBM_PEAK_GBS, 4), "speedup": round(ms_loop / ms_multi, 3)}


def time_call(fn, steps):
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


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
    ms = time_call(lambda: r.project_bwd(view), steps)
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
    ms = time_call(lambda: r.mesh_bwd(view), steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "k_mesh_bwd", "ms": round(ms, 4), "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "covered_pixels": covered}


def cpu_baseline(scene, view, ntiles, views_per_step):
    """The oracle (fwd+bwd, OpenMP on the host cores) on a bounded sample of tiles of
    one view; seconds per view scaled from the sample to every tile."""
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
            "cpu_model": cpu_model(), "s_per_view": round(dt * T / len(tiles), 3),
            "sample": f"{len(tiles)} of {T} 16x16 tiles of view {view} ({px} px): projection and depth order of "
                      f"all Gaussians, z-buffer, lists, composite and reverse mode of those tiles; {dt:.1f} s"
                      + (f"; a step renders {views_per_step} views" if views_per_step > 1 else "")}


if __name__ == "__main__":
    main()
