"""Benchmark: hybrid render fwd+bwd throughput at 1080p on one MI355X.

One step = the whole hot path over one view of the workload:
gm_bin_triangles -> gm_raster_zbuffer -> gm_project_gaussians -> gm_sort_tile_keys
-> gm_composite_hybrid_fwd -> gm_composite_hybrid_bwd, inputs resident in HBM.

Prints one JSON line (rank 0): the metric, per-stage times, a roofline entry for
the dominant kernel (timed live with HIP events on the library's stream) and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (256 CU x 4 SIMD x 16 lanes... x 2 x 2.4 GHz)

WORKLOADS = {
    "c3": "1920x1080, 200k-face displaced sphere (vertex colour + Phong), 1M Gaussians SH3",
    "c5": "1920x1080, 4 displaced spheres (499,280 faces, Phong), 3M Gaussians SH3, one of 4 views",
    "c2": "512x512, 5120-face icosphere, 100k Gaussians",
    "c4": "800x800 textured 4096-triangle soup, no Gaussians, one of 16 views",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--view", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=640, help="tiles in the oracle's timed sample")
    return ap.parse_args()


def algorithmic_bytes(r, scene):
    """Compulsory HBM bytes of one view per stage (each input read once, each output
    written once), from the run's own counts."""
    import torch
    N, V, F, HW, T = scene.N, scene.V, scene.F, scene.width * scene.height, r.T
    K, P = r.n_keys, r.n_pairs
    nvis = int((r.rec[:N, 15].view(torch.int32) > 0).sum().item()) if N else 0
    d = scene.sh_degree
    shb = 12 * (d + 1) ** 2 if d >= 0 else 12
    return {
        "bin": 12 * V + 12 * V + 12 * F + 8 * P + 4 * T,
        "zbuffer": 4 * P + 12 * F + 12 * V + 8 * HW + 4 * T,
        "project": N * (12 + 16 + 12 + 4 + shb + 64),
        "sort": 64 * N + 28 * K + 8 * T,
        "fwd": 4 * K + 64 * nvis + 8 * HW + 20 * HW + 8 * HW,
        "bwd": 4 * K + 64 * nvis + 8 * HW + 8 * HW + 20 * HW + 52 * nvis + 16 * HW,
    }, nvis


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (the renderer has no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import scenes
    from differentiable_hybrid_mesh_amd.pipeline import DeviceScene, Renderer

    torch.cuda.set_device(0)
    scene = scenes.make_scene(args.config)
    view = args.view % len(scene.views)
    ds = DeviceScene(scene)
    r = Renderer(ds)
    g = ds.grads(view)
    torch.cuda.synchronize()

    stages = ["bin", "zbuffer", "project", "sort", "fwd", "bwd"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        r.bin_and_zbuffer(view) if ev is None else _bin_z(ev)
        if ev is not None:
            ev[2].record()
        r.project(view)
        if ev is not None:
            ev[3].record()
        r.sort(view, True)
        if ev is not None:
            ev[4].record()
        r.composite_fwd(view)
        if ev is not None:
            ev[5].record()
        r.composite_bwd(view, g["rgb"], g["depth"], g["alpha"])
        if ev is not None:
            ev[6].record()

    def _bin_z(ev):
        ds_, cam, st = r.ds, r.ds.cams[view], torch.cuda.current_stream().cuda_stream
        from differentiable_hybrid_mesh_amd import _lib as G
        status, n = G.gm_bin_triangles(cam, ds_.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.pair_cap,
                                       r.ws_bin, st)
        assert status == G.GM_OK
        r.n_pairs = n
        ev[1].record()
        G.gm_raster_zbuffer(cam, ds_.mesh, r.vscreen, r.tile_offsets, r.tile_tris, r.face_id, r.depth,
                            r.tile_dmax, st)

    for _ in range(max(args.warmup, 1)):
        step()  # the first step also grows the list capacities
    torch.cuda.synchronize()

    # timed region: K whole steps, no per-stage events
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
    ms = t0.elapsed_time(t1) / args.steps

    # per-stage split (separate pass, same work, HIP events on the library's stream)
    per = {k: [] for k in stages}
    for _ in range(max(3, min(args.steps, 10))):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        step(ev)
        torch.cuda.synchronize()
        for i, k in enumerate(stages):
            per[k].append(ev[i].elapsed_time(ev[i + 1]))
    stage_ms = {k: float(np.median(v)) for k, v in per.items()}

    px = scene.width * scene.height
    value = px / (ms * 1e-3) / 1e6
    alg, nvis = algorithmic_bytes(r, scene)
    dom = max(stage_ms, key=stage_ms.get)
    dom_s = stage_ms[dom] * 1e-3
    roof = {"kernel": {"bwd": "k_composite_bwd", "fwd": "k_composite_fwd", "sort": "gm_sort_tile_keys",
                       "project": "k_project_gaussians", "zbuffer": "k_zbuffer", "bin": "gm_bin_triangles"}[dom],
            "bound": "hbm", "achieved": alg[dom] / dom_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None}
    roof["frac"] = roof["achieved"] / roof["peak"]

    total_alg = sum(alg.values())
    out = {
        "metric": "hybrid render Mpixels/s fwd+bwd at 1080p",
        "value": round(value, 3), "unit": "Mpixels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64 scene generators)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "view": view,
                   "width": scene.width, "height": scene.height, "faces": scene.F, "gaussians": scene.N,
                   "pairs": r.n_pairs, "keys": r.n_keys, "visible": nvis, "parallelism": "single GPU"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "hbm_algorithmic_GBps": round(total_alg / (ms * 1e-3) / 1e9, 1),
        "hbm_algorithmic_frac": round(total_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(scene, view, args.cpu_tiles)
    print(json.dumps(out), flush=True)


def cpu_baseline(scene, view, ntiles):
    """The oracle (fwd+bwd, OpenMP on the host cores) on a bounded sample of tiles."""
    import oracle
    T = scene.tiles_x * scene.tiles_y
    rng = np.random.default_rng(123)
    tiles = np.sort(rng.choice(T, size=min(ntiles, T), replace=False)).astype(np.int32)
    t = time.perf_counter()
    oracle.render_view(scene, view, tiles=tiles, cull=True, backward=True)
    dt = time.perf_counter() - t
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    px = len(tiles) * 256
    return {"value": round(px / dt / 1e6, 6), "unit": "Mpixels/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(tiles)} random 16x16 tiles of view {view} ({px} px), fwd+bwd incl. projection of "
                      f"all Gaussians and z-buffer of the sampled tiles; {dt:.1f} s"}


if __name__ == "__main__":
    main()
