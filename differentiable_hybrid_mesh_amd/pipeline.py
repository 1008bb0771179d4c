"""Buffer management around the six C-ABI calls (allocation and call order only).

``DeviceScene`` uploads a scene's arrays to the GPU once.  ``Renderer`` owns the
per-view device buffers (torch tensors used as plain device memory), reads the two
list lengths back once per forward pass (the calls themselves never synchronise),
grows a list that overflowed and runs the pass again, and runs

    gm_bin_triangles -> gm_raster_zbuffer ----------.----------> gm_shade_surface --.
    gm_project_sort_depth --------------------------+-> gm_sort_tiles ---------------+->
    gm_composite_hybrid_fwd_shaded                   (forward)
    gm_composite_hybrid_bwd                          (backward)

on the current torch stream, except the projection and the depth sort, which run
on a second stream beside the binning and z-buffer, followed there by the mesh
shading (the composite forward's first half) beside the tile sort
(``Renderer.lists``).  In the pipelined multi-view pass
(``Renderer.views_step_pipelined``) each view's mesh half and lists run on two
producer streams beside the previous view's composite.  Every step
of the path runs in libgm's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as G


def _stream():
    return torch.cuda.current_stream().cuda_stream


def make_camera(width, height, fx, fy, cx, cy, R, t, near_z=0.01) -> G.GmCamera:
    cam = G.GmCamera()
    cam.width, cam.height = int(width), int(height)
    cam.fx, cam.fy, cam.cx, cam.cy = float(fx), float(fy), float(cx), float(cy)
    R = np.asarray(R, np.float32).reshape(-1)
    t = np.asarray(t, np.float32).reshape(-1)
    for i in range(9):
        cam.R[i] = float(R[i])
    for i in range(3):
        cam.t[i] = float(t[i])
    cam.near_z = float(near_z)
    return cam


def make_light(light: Optional[dict]) -> Optional[G.GmLight]:
    if light is None:
        return None
    L = G.GmLight()
    for i in range(3):
        L.pos[i] = float(light["pos"][i])
        L.ambient[i] = float(light["ambient"][i])
        L.diffuse[i] = float(light["diffuse"][i])
        L.specular[i] = float(light["specular"][i])
    L.shininess = float(light["shininess"])
    return L


class DeviceScene:
    """A scene's inputs resident in GPU memory (SoA planes, as the ABI takes them)."""

    def __init__(self, scene, device: str = "cuda"):
        self.scene = scene
        self.device = device

        def up(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

        self.verts, self.faces, self.face_mask = up(scene.verts), up(scene.faces), up(scene.face_mask)
        self.vcolor, self.vnormal = up(scene.vcolor), up(scene.vnormal)
        self.uv, self.faces_uv, self.texture = up(scene.uv), up(scene.faces_uv), up(scene.texture)
        self.means, self.quats, self.scales = up(scene.means), up(scene.quats), up(scene.scales)
        self.opacity, self.sh = up(scene.opacity), up(scene.sh)
        self.mips = None
        self.tex_size = 0
        if self.texture is not None:
            S = int(scene.texture.shape[0])
            self.tex_size = S
            self.mips = torch.empty(G.gm_mipmaps_floats(S), dtype=torch.float32, device=device)
            G.gm_build_mipmaps(self.texture, S, self.mips, _stream())
        m = G.GmMesh()
        m.V, m.F = scene.V, scene.F
        m.Vt = 0 if scene.uv is None else int(scene.uv.shape[1])
        m.tex_size = self.tex_size
        V, F = scene.V, scene.F
        m.verts = G.dev(self.verts, "verts", G.F32, 3 * V, optional=V == 0)
        m.faces = G.dev(self.faces, "faces", G.I32, 3 * F, optional=F == 0)
        m.face_mask = G.dev(self.face_mask, "face_mask", G.U8, F, optional=True)
        m.vcolor = G.dev(self.vcolor, "vcolor", G.F32, 3 * V, optional=True)
        m.vnormal = G.dev(self.vnormal, "vnormal", G.F32, 3 * V, optional=True)
        m.uv = G.dev(self.uv, "uv", G.F32, 2 * m.Vt, optional=True)
        m.faces_uv = G.dev(self.faces_uv, "faces_uv", G.I32, 3 * F, optional=True)
        m.mips = G.dev(self.mips, "mips", G.F32, 0, optional=True)
        self.mesh = m
        self.light = make_light(scene.light)
        self.cams = [make_camera(scene.width, scene.height, scene.fx, scene.fy, scene.cx, scene.cy,
                                 v.R, v.t, scene.near_z) for v in scene.views]

    def adjacency(self):
        """Edge adjacency [3][F] of the mesh (built once, on first use)."""
        if getattr(self, "_adj", None) is None:
            F = self.scene.F
            self._adj = torch.empty((3, max(F, 1)), dtype=torch.int32, device=self.device)
            ws = torch.empty(G.gm_edge_adjacency_ws(F), dtype=torch.uint8, device=self.device)
            G.gm_edge_adjacency(self.mesh, self._adj, ws, _stream())
        return self._adj

    def grads(self, view: int):
        g = self.scene.grads[view]
        return {k: torch.from_numpy(np.ascontiguousarray(v)).to(self.device) for k, v in g.items()}


class Renderer:
    """Per-view device buffers and the call sequence of one forward / backward."""

    MAX_BATCH = 64  # views of one batched pass

    def __init__(self, ds: DeviceScene, pair_cap: Optional[int] = None, key_cap: Optional[int] = None):
        s = ds.scene
        self.ds = ds
        dev = ds.device
        self.W, self.H = s.width, s.height
        self.T = s.tiles_x * s.tiles_y
        self.N = s.N
        i32, f32 = torch.int32, torch.float32
        self.vscreen = torch.empty((3, max(s.V, 1)), dtype=f32, device=dev)
        self.tile_offsets = torch.empty(self.T + 1, dtype=i32, device=dev)
        self.ws_bin = torch.empty(G.gm_bin_triangles_ws(s.V, s.F, s.width, s.height), dtype=torch.uint8,
                                  device=dev)
        self.pair_cap = pair_cap if pair_cap is not None else 4 * s.F + 1024
        self.tile_tris = torch.empty(max(self.pair_cap, 1), dtype=i32, device=dev)
        self.face_id = torch.empty((self.H, self.W), dtype=i32, device=dev)
        self.depth = torch.empty((self.H, self.W), dtype=f32, device=dev)
        self.tile_dmax = torch.empty(self.T, dtype=f32, device=dev)
        self.ws_zb = torch.empty(G.gm_raster_zbuffer_ws(s.width, s.height), dtype=torch.uint8, device=dev)
        self.rec = torch.empty((max(self.N, 1), G.GM_REC), dtype=f32, device=dev)
        self._rec_own = self.rec
        self.rec_views = None  # [views][N][GM_REC] of project_views()
        self.tile_ranges = torch.empty((self.T, 2), dtype=i32, device=dev)
        self.key_cap = key_cap if key_cap is not None else 8 * self.N + 1024
        self._alloc_keys(self.key_cap)
        self.out_rgb = torch.empty((self.H, self.W, 3), dtype=f32, device=dev)
        self.out_depth = torch.empty((self.H, self.W), dtype=f32, device=dev)
        self.out_alpha = torch.empty((self.H, self.W), dtype=f32, device=dev)
        self.state_T = torch.empty((self.H, self.W), dtype=f32, device=dev)
        self.state_last = torch.empty((self.H, self.W), dtype=i32, device=dev)
        self.state_cm = torch.empty((self.H, self.W, 3), dtype=f32, device=dev)
        self.g_rec = torch.empty((max(self.N, 1), G.GM_GRAD), dtype=f32, device=dev)
        self.g_mesh_rgb = torch.empty((self.H, self.W, 3), dtype=f32, device=dev)
        self.g_mesh_depth = torch.empty((self.H, self.W), dtype=f32, device=dev)
        self.ws_comp_bwd = torch.empty(G.gm_composite_hybrid_bwd_ws(s.width, s.height), dtype=torch.uint8,
                                       device=dev)
        self.n_pairs = 0
        self.n_keys = 0
        # device list lengths (n_pairs, n_keys), one row per view of a batched pass
        self.counts_all = torch.zeros((self.MAX_BATCH, 2), dtype=torch.int64, device=dev)
        self.counts_host = torch.zeros((self.MAX_BATCH, 2), dtype=torch.int64, pin_memory=True)
        self.counts = self.counts_all[0]
        self._rows = 1
        self.view = 0
        self.cull = True
        self._side = None  # second stream of lists(), made on first use
        self._shaded = None  # view whose state_cm lists() queued on the second stream
        self._slots = None  # two buffer sets of views_step_pipelined(), made on first use
        self._mesh_stream = None

    def _alloc_keys(self, cap):
        s = self.ds.scene
        self.key_cap = int(cap)
        self.sorted_ids = torch.empty(max(self.key_cap, 1), dtype=torch.int32, device=self.ds.device)
        self.ws_sort = torch.empty(G.gm_sort_tile_keys_ws(self.N, self.key_cap, s.width, s.height),
                                   dtype=torch.uint8, device=self.ds.device)

    # -- the six calls ---------------------------------------------------------
    def bin_and_zbuffer(self, view: int):
        ds, cam, st = self.ds, self.ds.cams[view], _stream()
        G.gm_bin_triangles(cam, ds.mesh, self.vscreen, self.tile_offsets, self.tile_tris, self.pair_cap,
                           self.counts[0:1], self.ws_bin, st)
        G.gm_raster_zbuffer(cam, ds.mesh, self.vscreen, self.tile_offsets, self.tile_tris, self.face_id,
                            self.depth, self.tile_dmax, self.ws_zb, st)

    def project(self, view: int):
        ds, s = self.ds, self.ds.scene
        self.rec = self._rec_own
        G.gm_project_gaussians(ds.cams[view], self.N, ds.means, ds.quats, ds.scales, ds.opacity, ds.sh,
                               s.sh_degree, self.rec, _stream())

    def project_sort_depth(self, view: int):
        """project() then sort_depth() in one call (the projection also writes the depth
        sort's keys, one kernel fewer)."""
        ds, s = self.ds, self.ds.scene
        self.rec = self._rec_own
        G.gm_project_sort_depth(ds.cams[view], self.N, ds.means, ds.quats, ds.scales, ds.opacity, ds.sh,
                                s.sh_degree, self.rec, self.key_cap, self.ws_sort, _stream())

    def sort(self, view: int, cull: bool = True):
        ds, s = self.ds, self.ds.scene
        dmax = self.tile_dmax if cull else None
        G.gm_sort_tile_keys(ds.cams[view], self.N, self.rec, dmax, s.softness, self.tile_ranges, self.sorted_ids,
                            self.key_cap, self.counts[1:2], self.ws_sort, _stream())

    def sort_depth(self, view: int):
        """First half of sort(): the depth order (reads the records only)."""
        ds, s = self.ds, self.ds.scene
        G.gm_sort_depth(ds.cams[view], self.N, self.rec, self.key_cap, self.ws_sort, _stream())

    def sort_tiles(self, view: int, cull: bool = True):
        """Second half of sort(): cull, lists, tile order (after sort_depth and the z-buffer)."""
        ds, s = self.ds, self.ds.scene
        dmax = self.tile_dmax if cull else None
        G.gm_sort_tiles(ds.cams[view], self.N, self.rec, dmax, s.softness, self.tile_ranges, self.sorted_ids,
                        self.key_cap, self.counts[1:2], self.ws_sort, _stream())

    def _side_stream(self):
        if self._side is None:  # default priority, like every stream here
            self._side = torch.cuda.Stream(device=self.ds.device)
            self._ev_main = torch.cuda.Event()
            self._ev_side = torch.cuda.Event()
            self._ev_zb = torch.cuda.Event()
            self._ev_shade = torch.cuda.Event()
        return self._side

    def shade(self, view: int):
        """The colour behind the Gaussians (state_cm) from the z-buffer: the first half
        of the composite forward."""
        ds, s = self.ds, self.ds.scene
        G.gm_shade_surface(ds.cams[view], self.face_id, ds.mesh, self.vscreen, ds.light, s.bg, self.state_cm,
                           _stream())

    def lists(self, view: int, cull: bool = True, antialias: bool = False, overlap: bool = True,
              project: bool = True):
        """Mesh visibility (bin, z-buffer, antialiased layer) and Gaussian lists
        (projection unless the records are already there, sort).  With overlap the
        projection and the depth sort run on a second stream beside the binning and
        z-buffer: the two branches share no buffer, and only the tile lists need both
        (tile_dmax and the depth order).  Once the z-buffer is done, the side stream
        also shades the mesh (state_cm, needed by the composite, not by the sort) beside
        the tile sort; composite_fwd() then waits for it.  The side stream first waits
        for everything queued before (the previous step's composite still reads the
        records, the lists and state_cm)."""
        self._shaded = None
        if not overlap:
            self.bin_and_zbuffer(view)
            if antialias:
                self.antialias(view)
            if project:
                self.project(view)
            self.sort(view, cull)
            return
        main, side = torch.cuda.current_stream(), self._side_stream()
        self._ev_main.record(main)
        side.wait_event(self._ev_main)
        with torch.cuda.stream(side):
            if project:
                self.project_sort_depth(view)
            else:
                self.sort_depth(view)
            self._ev_side.record(side)
        self.bin_and_zbuffer(view)
        if antialias:
            self.antialias(view)
        else:
            self._ev_zb.record(main)
            side.wait_event(self._ev_zb)
            with torch.cuda.stream(side):
                self.shade(view)
                self._ev_shade.record(side)
            self._shaded = view
        main.wait_event(self._ev_side)
        self.sort_tiles(view, cull)

    def fetch_counts(self):
        """Queue a copy of the list lengths to pinned host memory (no wait)."""
        self.counts_host[: self._rows].copy_(self.counts_all[: self._rows], non_blocking=True)

    def read_counts(self) -> bool:
        """After the stream has passed fetch_counts(): store the lengths (the largest
        over the views of a batched pass), grow any list that overflowed; True when
        every list fitted."""
        rows = self.counts_host[: self._rows]
        if bool((rows < 0).any()):
            raise RuntimeError("list construction reported a failure (negative length)")
        n_pairs, n_keys = (int(x) for x in rows.max(0).values.tolist())
        self.n_pairs, self.n_keys = n_pairs, n_keys
        ok = True
        if n_pairs > self.pair_cap:
            self.pair_cap = int(n_pairs * 1.25) + 1024
            self.tile_tris = torch.empty(self.pair_cap, dtype=torch.int32, device=self.ds.device)
            ok = False
        if n_keys > self.key_cap:
            self._alloc_keys(int(n_keys * 1.25) + 1024)
            ok = False
        if not ok:
            self._slots = None  # rebuilt at the new capacities
        return ok

    def composite_fwd(self, view: int):
        """The composite forward; when lists() has queued this view's shading on the
        side stream, only its second half, after that shading."""
        ds, s = self.ds, self.ds.scene
        if self._shaded == view:
            self._shaded = None
            torch.cuda.current_stream().wait_event(self._ev_shade)
            self.composite_fwd_shaded(view)
            return
        G.gm_composite_hybrid_fwd(ds.cams[view], self.rec, self.tile_ranges, self.sorted_ids, self.face_id,
                                  self.depth, ds.mesh, self.vscreen, ds.light, s.bg, s.softness, self.out_rgb,
                                  self.out_depth, self.out_alpha, self.state_T, self.state_last, self.state_cm,
                                  _stream())

    def composite_fwd_shaded(self, view: int):
        """The composite forward's second half: state_cm must already hold this view's
        shading, ordered before on the current stream."""
        ds, s = self.ds, self.ds.scene
        G.gm_composite_hybrid_fwd_shaded(ds.cams[view], self.rec, self.tile_ranges, self.sorted_ids, self.face_id,
                                         self.depth, s.softness, self.state_cm, self.out_rgb, self.out_depth,
                                         self.out_alpha, self.state_T, self.state_last, _stream())

    def composite_bwd(self, view: int, g_rgb, g_depth=None, g_alpha=None):
        ds, s = self.ds, self.ds.scene
        G.gm_composite_hybrid_bwd(ds.cams[view], self.N, self.rec, self.tile_ranges, self.sorted_ids,
                                  self.face_id, self.depth, s.softness, self.state_T, self.state_last,
                                  self.state_cm, g_rgb, g_depth, g_alpha, self.g_rec, self.g_mesh_rgb,
                                  self.g_mesh_depth, self.ws_comp_bwd, _stream())

    def project_bwd(self, view: int, g_rec=None, log_params: bool = False):
        """Gradients of the Gaussian parameters from record gradients (default: the
        last composite backward's).  Buffers are allocated on first use."""
        ds, s = self.ds, self.ds.scene
        N = self.N
        if not hasattr(self, "g_means"):
            dev, f32 = ds.device, torch.float32
            K = 1 if s.sh_degree < 0 else (s.sh_degree + 1) ** 2
            self.g_means = torch.empty((3, max(N, 1)), dtype=f32, device=dev)
            self.g_quats = torch.empty((4, max(N, 1)), dtype=f32, device=dev)
            self.g_scales = torch.empty((3, max(N, 1)), dtype=f32, device=dev)
            self.g_opacity = torch.empty(max(N, 1), dtype=f32, device=dev)
            self.g_sh = torch.empty((K, 3, max(N, 1)), dtype=f32, device=dev)
            self.g_log_scales = torch.empty((3, max(N, 1)), dtype=f32, device=dev)
            self.g_logit = torch.empty(max(N, 1), dtype=f32, device=dev)
        G.gm_project_gaussians_bwd(ds.cams[view], N, ds.means, ds.quats, ds.scales, ds.opacity, ds.sh, s.sh_degree,
                                   self.rec, self.g_rec if g_rec is None else g_rec, self.g_means, self.g_quats,
                                   self.g_scales, self.g_opacity, self.g_sh,
                                   self.g_log_scales if log_params else None, self.g_logit if log_params else None,
                                   _stream())
        return {"means": self.g_means[:, :N], "quats": self.g_quats[:, :N], "scales": self.g_scales[:, :N],
                "opacity": self.g_opacity[:N], "sh": self.g_sh[..., :N]}

    def mesh_bwd(self, view: int, g_mesh_rgb=None, g_mesh_depth=None, g_vscreen=None):
        """Gradients of the mesh parameters from per-pixel dL/dc_m and dL/dD (default:
        the last backward's, with the silhouette gradients g_vscreen when it was
        antialiased).  Buffers are allocated on first use."""
        ds, s = self.ds, self.ds.scene
        dev, f32 = ds.device, torch.float32
        if not hasattr(self, "gm_verts"):
            V = max(s.V, 1)
            self.gm_verts = torch.empty((3, V), dtype=f32, device=dev)
            self.gm_vcolor = torch.empty((3, V), dtype=f32, device=dev) if s.vcolor is not None else None
            lit = ds.light is not None and s.vnormal is not None
            self.gm_vnormal = torch.empty((3, V), dtype=f32, device=dev) if lit else None
            self.gm_light = torch.empty(13, dtype=f32, device=dev) if lit else None
            tex = ds.mips is not None
            self.gm_uv = torch.empty((2, max(ds.mesh.Vt, 1)), dtype=f32, device=dev) if tex else None
            self.gm_mips = torch.empty(G.gm_mipmaps_floats(ds.tex_size), dtype=f32, device=dev) if tex else None
        G.gm_mesh_bwd(ds.cams[view], ds.mesh, ds.light, self.face_id,
                      self.g_mesh_rgb if g_mesh_rgb is None else g_mesh_rgb,
                      self.g_mesh_depth if g_mesh_depth is None else g_mesh_depth, self.gm_verts, self.gm_vcolor,
                      self.gm_vnormal, self.gm_uv, self.gm_mips, self.gm_light, _stream())
        if g_vscreen is not None or (g_mesh_rgb is None and getattr(self, "aa", False)):
            # silhouettes: the crossings' screen-vertex gradients
            G.gm_vscreen_bwd(ds.cams[view], ds.mesh, self.g_vscreen if g_vscreen is None else g_vscreen,
                             self.gm_verts, _stream())
        out = {"verts": self.gm_verts[:, : s.V]}
        if self.gm_vcolor is not None:
            out["vcolor"] = self.gm_vcolor[:, : s.V]
        if self.gm_vnormal is not None:
            out["vnormal"], out["light"] = self.gm_vnormal[:, : s.V], self.gm_light
        if self.gm_mips is not None:
            S = ds.tex_size
            out["uv"], out["tex"] = self.gm_uv[:, : ds.mesh.Vt], self.gm_mips[: S * S * 3].view(S, S, 3)
        return out

    # -- analytic edge antialiasing ---------------------------------------------
    def _aa_buffers(self):
        if getattr(self, "layer", None) is not None:
            return
        dev, f32 = self.ds.device, torch.float32
        H, W = self.H, self.W
        self.colour = torch.empty((H, W, 3), dtype=f32, device=dev)
        self.layer = torch.empty((H, W, 8), dtype=f32, device=dev)
        self.aa_pairs = torch.empty((H, W, 12), dtype=f32, device=dev)
        self.state_aa = torch.empty((H, W, 8), dtype=f32, device=dev)
        self.g_layer = torch.empty((H, W, 8), dtype=f32, device=dev)
        self.ws_aa_bwd = torch.empty(G.gm_antialias_bwd_ws(W, H), dtype=torch.uint8, device=dev)
        self.g_vscreen = torch.empty((2, max(self.ds.scene.V, 1)), dtype=f32, device=dev)

    def antialias(self, view: int):
        """Antialiased mesh layer of the current z-buffer; marks the tiles whose back
        layer shows so that the cull skips them."""
        self._aa_buffers()
        ds = self.ds
        G.gm_antialias(ds.cams[view], ds.mesh, self.vscreen, ds.adjacency(), ds.light, self.face_id, self.depth,
                       self.colour, self.layer, self.aa_pairs, self.tile_dmax, _stream())

    def composite_fwd_aa(self, view: int):
        ds, s = self.ds, self.ds.scene
        G.gm_composite_hybrid_fwd_aa(ds.cams[view], self.rec, self.tile_ranges, self.sorted_ids, self.layer, s.bg,
                                     s.softness, self.out_rgb, self.out_depth, self.out_alpha, self.state_aa,
                                     _stream())

    def composite_bwd_aa(self, view: int, g_rgb, g_depth=None, g_alpha=None):
        ds, s = self.ds, self.ds.scene
        G.gm_composite_hybrid_bwd_aa(ds.cams[view], self.N, self.rec, self.tile_ranges, self.sorted_ids, self.layer,
                                     s.bg, s.softness, self.state_aa, g_rgb, g_depth, g_alpha, self.g_rec,
                                     self.g_layer, self.ws_comp_bwd, _stream())

    def antialias_bwd(self, view: int, g_layer=None):
        """dL/dc and dL/dD at covered pixels (into g_mesh_rgb / g_mesh_depth) and
        dL/d(u, v) of the screen vertices (g_vscreen) from dL/d(layer)."""
        ds = self.ds
        G.gm_antialias_bwd(ds.cams[view], ds.mesh, self.vscreen, self.aa_pairs, self.face_id, self.depth,
                           self.colour, self.g_layer if g_layer is None else g_layer, self.g_mesh_rgb,
                           self.g_mesh_depth, self.g_vscreen, self.ws_aa_bwd, _stream())

    # -- several views -----------------------------------------------------------
    def project_views(self, views):
        """Project the Gaussians into every view of ``views`` in one pass
        (gm_project_gaussians_multi: the parameters are read once for all views);
        use_view(k) then makes the k-th view's records the current ones."""
        ds, s = self.ds, self.ds.scene
        nv = len(views)
        if self.rec_views is None or self.rec_views.shape[0] < nv:
            self.rec_views = torch.empty((nv, max(self.N, 1), G.GM_REC), dtype=torch.float32, device=ds.device)
        G.gm_project_gaussians_multi([ds.cams[v] for v in views], self.N, ds.means, ds.quats, ds.scales,
                                     ds.opacity, ds.sh, s.sh_degree, self.rec_views, _stream())

    def use_view(self, k: int):
        """Select the records of the k-th view of the last project_views() and the k-th
        row of list lengths."""
        self.rec = self.rec_views[k]
        self.counts = self.counts_all[k]

    def _single(self):
        self.rec = self._rec_own
        self.counts = self.counts_all[0]
        self._rows = 1

    def views_step_async(self, views, grads, cull: bool = True, backward: bool = True, hook=None):
        """Forward (+ backward) of several views with one batched projection; no
        synchronisation.  grads[k] holds view k's upstream gradients.  The lists are
        rebuilt per view in the same buffers, so only the last view's outputs remain;
        hook(k), if given, runs after view k (e.g. to copy its outputs).  Check the
        lengths with read_counts() once the stream has run."""
        if len(views) > self.MAX_BATCH:
            raise ValueError(f"at most {self.MAX_BATCH} views per batch")
        self.project_views(views)
        self._rows = len(views)
        for k, v in enumerate(views):
            self.use_view(k)
            self.view, self.cull = v, cull
            self.lists(v, cull, project=False)  # the records come from the batched projection
            self.composite_fwd(v)
            if backward:
                self.composite_bwd(v, grads[k]["rgb"], grads[k].get("depth"), grads[k].get("alpha"))
            if hook is not None:
                hook(k)
        self.fetch_counts()

    # buffers written by the first half of a view (mesh visibility, shading, depth
    # order, lists); the second half's outputs and gradients are shared
    _SLOT_KEYS = ("vscreen", "tile_offsets", "ws_bin", "tile_tris", "face_id", "depth", "tile_dmax", "ws_zb",
                  "state_cm", "tile_ranges", "sorted_ids", "ws_sort")

    def _use_slot(self, i: int):
        if self._slots is None:
            a = {k: getattr(self, k) for k in self._SLOT_KEYS}
            self._slots = [a, {k: torch.empty_like(t) for k, t in a.items()}]
        for k, t in self._slots[i].items():
            setattr(self, k, t)

    def views_step_pipelined(self, views, grads, cull: bool = True, backward: bool = True, hook=None):
        """views_step_async() with the views' halves overlapped: the mesh half of view
        k (binning, z-buffer, shading) and its lists (depth sort, then the tile sort
        once the z-buffer is done) run on two producer streams into one of two buffer
        sets while the main stream composites view k - 1 from the other set.  A
        producer waits for the main stream to be done with view k - 2 (the last user of
        its set) and the main stream for both producers before view k's composite.
        Same results as views_step_async(), bit for bit; hook(k) runs on the main
        stream after view k."""
        if len(views) > self.MAX_BATCH:
            raise ValueError(f"at most {self.MAX_BATCH} views per batch")
        main, gs = torch.cuda.current_stream(), self._side_stream()
        if self._mesh_stream is None:  # default priority, like every stream here
            self._mesh_stream = torch.cuda.Stream(device=self.ds.device)
            self._ev_slot_free = [torch.cuda.Event(), torch.cuda.Event()]
            self._ev_mesh = [torch.cuda.Event(), torch.cuda.Event()]
            self._ev_gauss = [torch.cuda.Event(), torch.cuda.Event()]
            self._ev_start = torch.cuda.Event()
        ms = self._mesh_stream
        # everything queued before (readers of either buffer set) precedes the producers
        self._ev_start.record(main)
        ms.wait_event(self._ev_start)
        self.project_views(views)
        self._ev_main.record(main)  # the records of every view
        gs.wait_event(self._ev_main)
        self._rows = len(views)
        for k, v in enumerate(views):
            slot = k & 1
            self._use_slot(slot)
            self.use_view(k)
            self.view, self.cull = v, cull
            if k >= 2:
                ms.wait_event(self._ev_slot_free[slot])
                gs.wait_event(self._ev_slot_free[slot])
            with torch.cuda.stream(ms):
                self.bin_and_zbuffer(v)
                self._ev_zb.record(ms)
                self.shade(v)
                self._ev_mesh[slot].record(ms)
            with torch.cuda.stream(gs):
                self.sort_depth(v)
                gs.wait_event(self._ev_zb)
                self.sort_tiles(v, cull)
                self._ev_gauss[slot].record(gs)
            main.wait_event(self._ev_gauss[slot])
            main.wait_event(self._ev_mesh[slot])
            self.composite_fwd_shaded(v)
            if backward:
                self.composite_bwd(v, grads[k]["rgb"], grads[k].get("depth"), grads[k].get("alpha"))
            if hook is not None:
                hook(k)
            self._ev_slot_free[slot].record(main)
        self.fetch_counts()

    def fit_lists_views(self, views, cull: bool = True):
        """fit_lists() for a batched pass: grow the lists until every view's fit."""
        while True:
            self.project_views(views)
            self._rows = len(views)
            for k, v in enumerate(views):
                self.use_view(k)
                self.lists(v, cull, project=False)
            self.fetch_counts()
            torch.cuda.current_stream().synchronize()
            if self.read_counts():
                return

    # -- whole passes -----------------------------------------------------------
    def forward_async(self, view: int = 0, cull: bool = True, antialias: bool = False):
        """Queue one forward pass and the copy of the list lengths; no synchronisation.
        The outputs are valid once read_counts() returns True for this pass."""
        self._single()
        self.view, self.cull, self.aa = view, cull, antialias
        self.lists(view, cull, antialias)
        if antialias:
            self.composite_fwd_aa(view)
        else:
            self.composite_fwd(view)
        self.fetch_counts()

    def fit_lists(self, view: int = 0, cull: bool = True, antialias: bool = False):
        """Run the list-producing calls (no compositing) until both lists fit."""
        self._single()
        while True:
            self.lists(view, cull, antialias)
            self.fetch_counts()
            torch.cuda.current_stream().synchronize()
            if self.read_counts():
                return

    def forward(self, view: int = 0, cull: bool = True, antialias: bool = False):
        while True:
            self.forward_async(view, cull, antialias)
            torch.cuda.current_stream().synchronize()
            if self.read_counts():
                break
        return {"rgb": self.out_rgb, "depth": self.out_depth, "alpha": self.out_alpha}

    def backward(self, g_rgb, g_depth=None, g_alpha=None):
        """Reverse mode of the last forward: record gradients and dL/dc, dL/dD at the
        covered pixels (with antialiasing through the layer, plus g_vscreen)."""
        if getattr(self, "aa", False):
            self.composite_bwd_aa(self.view, g_rgb, g_depth, g_alpha)
            self.antialias_bwd(self.view)
        else:
            self.composite_bwd(self.view, g_rgb, g_depth, g_alpha)
        return {"rec": self.g_rec[: self.N], "mesh_rgb": self.g_mesh_rgb, "mesh_depth": self.g_mesh_depth}

    def step(self, view: int, grads: dict, cull: bool = True, antialias: bool = False):
        """One forward + backward of one view (the benchmark's unit of work)."""
        self.forward(view, cull, antialias)
        return self.backward(grads["rgb"], grads.get("depth"), grads.get("alpha"))

    def step_async(self, view: int, grads: dict, cull: bool = True, antialias: bool = False):
        """step() without synchronisation: the lengths are checked by the caller with
        read_counts() after the stream has run (the lists must already be large enough)."""
        self.forward_async(view, cull, antialias)
        if antialias:
            self.composite_bwd_aa(view, grads["rgb"], grads.get("depth"), grads.get("alpha"))
        else:
            self.composite_bwd(view, grads["rgb"], grads.get("depth"), grads.get("alpha"))
