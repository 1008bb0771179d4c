/*
 * gm.h — C ABI of the MI355X (gfx950) hybrid mesh + 3D Gaussian tile rasterizer.
 *
 * The method is the one of the gmesh README ("A Lightweight and Differentiable
 * Renderer for Joint Mesh and 3D Gaussian Splat Scenes", section "Design Details"):
 * triangles are binned into 16x16 tiles and a z-buffer finds the nearest triangle
 * at every pixel centre; 3D Gaussians are projected to 2D conics with an affine
 * (EWA) model of their depth; Gaussians certainly hidden behind the mesh in fully
 * covered tiles are culled; the rest are sorted per tile by centre depth and
 * composited front to back, each one split at the mesh surface by
 * f = Phi((D - z*(p)) / (sigma softness)), with the mesh colour filling the
 * remaining transmittance; the backward pass of that composite gives gradients of
 * every Gaussian record and of the mesh colour and depth.
 *
 * Conventions (the README states that meshes and Gaussians share one pinhole
 * camera and pixel convention; its camera-axes section carries no text, so the
 * gsplat/OpenCV reading is used):
 *   x_c = R x_w + t, R row-major; +x right, +y down, +z forward;
 *   u = fx x_c / z_c + cx, v = fy y_c / z_c + cy;
 *   pixel (i, j) is column i, row j, with centre (i + 0.5, j + 0.5);
 *   tiles are 16x16 pixels, TX = ceil(W/16), TY = ceil(H/16), T = TX*TY,
 *   tile id = ty*TX + tx.
 *
 * Memory.  Every array pointer is a DEVICE pointer to caller-owned memory unless
 * marked (host).  "[k][N]" is k contiguous planes of N values (structure of
 * arrays).  The library never allocates, frees or keeps a pointer after a call
 * returns.  Every call is asynchronous on `stream` and never synchronises it.
 *
 * Variable-length lists.  The two calls that produce one (gm_bin_triangles,
 * gm_sort_tile_keys) write its length to a device int64 (`n_pairs`, `n_keys`) and
 * take the list's capacity `cap`.  Nothing is written beyond cap, and when the
 * length exceeds cap the call's other outputs describe an empty list (empty bins,
 * every tile range empty), so later calls stay in bounds; the caller reads the
 * length once the stream has reached it, and on overflow enlarges the list and
 * calls again.
 *
 * Layout choices.  Three choices shape the signatures below.  (1) No call reads a
 * count back to the host: a list's length goes to a device int64 and an overflow is
 * visible there (there is no capacity error status), so a whole forward and
 * backward can be queued without a synchronisation.  (2) The projected Gaussians
 * are one 64-byte record each ([N][16] floats) rather than separate planes: the
 * composite gathers one record per list entry, a single 64-byte load.  (3) The
 * forward keeps the colour behind the Gaussians of every pixel (state_cm) for the
 * backward, which then needs no mesh attributes, and its shading half can run on
 * another stream beside the tile sort.
 *
 * Errors.  Every call returns a gm_status.  GM_ERR_ARG: a required pointer is
 * NULL, a size is negative or out of range, the workspace is too small; checked on
 * the host before anything is launched.  GM_ERR_HIP: a HIP call failed.  gm_last_error() returns a
 * thread-local message for the last non-OK status.  Degenerate data follow rules,
 * not errors: zero-area triangles cover nothing, Gaussians with det <= 0 or behind
 * the near plane are not listed, N = 0 and F = 0 are legal.
 */
#ifndef GM_H
#define GM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GM_TILE 16
/* Floats per projected Gaussian record (64 bytes, see gm_project_gaussians). */
#define GM_REC 16
/* Floats per Gaussian gradient record (see gm_composite_hybrid_bwd). */
#define GM_GRAD 13

typedef enum {
    GM_OK = 0,
    GM_ERR_ARG = -1,
    GM_ERR_HIP = -3
} gm_status;

/* Pinhole camera; passed by host pointer and read at call time. */
typedef struct gm_camera {
    int32_t width, height; /* pixels, > 0 */
    float fx, fy, cx, cy;  /* pixel units */
    float R[9];            /* world -> camera rotation, row-major */
    float t[3];            /* world -> camera translation */
    float near_z;          /* near plane, > 0 (0.01 in every workload) */
} gm_camera;

/* World-space point light for per-pixel Phong shading of the mesh (README v1.1:
 * a point light shades the mesh per pixel with interpolated vertex normals and a
 * specular highlight that follows the camera).  Host pointer; NULL = unlit. */
typedef struct gm_light {
    float pos[3];
    float ambient[3], diffuse[3], specular[3];
    float shininess;
} gm_light;

/* Mesh attributes (README "Mesh rasterizer" and v1.1: vertex colours, or a texture
 * with per-corner texture coordinates as in OBJ files; optional vertex normals for
 * lighting).  Host pointer to a struct of device pointers; unused ones NULL. */
typedef struct gm_mesh {
    int32_t V, F;             /* vertices, faces (>= 0) */
    int32_t Vt;               /* texture coordinates (0 when untextured) */
    int32_t tex_size;         /* S: square power-of-two texture side, 0 when untextured */
    const float* verts;       /* [3][V] world positions */
    const int32_t* faces;     /* [3][F] vertex ids */
    const uint8_t* face_mask; /* [F] 0 = triangle absent (stochastic binary opacity), or NULL */
    const float* vcolor;      /* [3][V] base colour, or NULL */
    const float* vnormal;     /* [3][V] world normals, or NULL (then unlit) */
    const float* uv;          /* [2][Vt], or NULL */
    const int32_t* faces_uv;  /* [3][F] texture-coordinate ids, or NULL */
    const float* mips;        /* pyramid written by gm_build_mipmaps, or NULL */
} gm_mesh;

/* ---------------------------------------------------------------------------
 * 1. gm_bin_triangles — vertex projection and 16x16 tile binning.
 * README "Mesh rasterizer", step 1 (triangles binned into 16x16 tiles) and the
 * near-plane rule (triangles with a vertex in front of the near plane are
 * skipped, no clipping).
 *
 * Writes vscreen [3][V] = (u, v, z_c) per vertex, evaluated in fp32 as
 *   x_c = ((R0 x + R1 y) + R2 z) + t0 (likewise y_c, z_c), u = (fx x_c)/z_c + cx.
 * A face is binned when its mask is non-zero, all three z_c >= near_z and its
 * fp64 signed area is non-zero; it goes to every tile that holds a pixel centre of
 * its pixel-centre bounding box.  tile_offsets [T+1] (exclusive prefix sums) and
 * tile_tris [n_pairs] list the face ids per tile (order inside a tile unspecified).
 * cap: capacity of tile_tris; n_pairs (device int64, out): number of (tile, face)
 * pairs; above cap, tile_tris is not written and tile_offsets is all zeros.
 * ws: device workspace of at least gm_bin_triangles_ws(...) bytes.
 * ------------------------------------------------------------------------- */
size_t gm_bin_triangles_ws(int32_t V, int32_t F, int32_t width, int32_t height);
gm_status gm_bin_triangles(const gm_camera* cam, const gm_mesh* mesh, float* vscreen,
                           int32_t* tile_offsets, int32_t* tile_tris, int64_t cap,
                           int64_t* n_pairs, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 2. gm_raster_zbuffer — nearest triangle at every pixel centre.
 * README "Mesh rasterizer", step 1 (a kernel finds the nearest triangle at each
 * pixel centre; this visibility decision is the only non-differentiable step).
 *
 * For pixel centre p the edge functions E_k(p) = (b.u-a.u)(p.v-a.v) -
 * (b.v-a.v)(p.u-a.u) of edges (v1,v2), (v2,v0), (v0,v1) are evaluated in fp64; p is
 * covered when E_k * sign(A) >= 0 for k = 0,1,2 (inclusive, no back-face culling).
 * Depth z = 1 / sum_k (E_k/A)/z_k in fp64.  The smallest z wins, an exact tie goes
 * to the smaller face id.  Outputs: face_id [H][W] (-1 = empty), depth [H][W] =
 * fp32 rounding of z (+inf = empty), tile_dmax [T] = max depth over the tile's
 * in-image pixels, +inf when any of them is empty (input of the occlusion cull).
 * Inputs: vscreen, tile_offsets [T+1] and tile_tris of call 1 for the same camera
 * and mesh.  ws: device scratch of at least gm_raster_zbuffer_ws(W, H) bytes, owned
 * by the caller (the tiles' launch order, largest bin first; it does not change the
 * result); too small or NULL is GM_ERR_ARG.
 * ------------------------------------------------------------------------- */
size_t gm_raster_zbuffer_ws(int32_t width, int32_t height);
gm_status gm_raster_zbuffer(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                            const int32_t* tile_offsets, const int32_t* tile_tris,
                            int32_t* face_id, float* depth, float* tile_dmax, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 3. gm_project_gaussians — EWA projection, conditional depth model, colour.
 * README "Hybrid rendering": z*(p) = z_c + g.(p - mean2d) with
 * g = (Sigma_uv + eps I)^-1 Sigma_uv,z and sigma^2 = Sigma_zz - Sigma_z,uv g, from
 * the projected 3D covariance; projection and spherical-harmonics colour as in
 * 3D Gaussian splatting.  eps = 0.3 px^2, also the 2D splat dilation.
 *
 * Inputs: means [3][N] world, quats [4][N] (w, x, y, z; normalised here), scales
 * [3][N] linear (exp of log-scales), opacity [N] in [0, 1] (sigmoid of logits),
 * sh [(d+1)^2][3][N] coefficients for sh_degree d in 0..3, or sh [1][3][N] plain
 * RGB when sh_degree = -1.  Colour = max(0, sum_lm Y_lm(dir) c_lm + 0.5) at
 * dir = normalize(mean - camera centre), real SH in the splatting sign convention.
 *
 * Output rec [N][GM_REC] floats per Gaussian (64-byte aligned records):
 *   0 u, 1 v (mean2d), 2 Q00, 3 Q01, 4 Q11 (conic = (Sigma_uv + eps I)^-1),
 *   5 opacity, 6..8 rgb, 9 z_c, 10 g0, 11 g1, 12 sigma,
 *   13 int32 tx0 | ty0 << 16, 14 int32 tx1 | ty1 << 16 (tile rect, exclusive),
 *   15 int32 number of tiles in the rect (0 = not listed).
 * The decision fields (0..5, 9..15) are evaluated in fp32 in a fixed order with no
 * fused multiply-add; the rect covers the box of the 3-sigma ellipse, half-widths
 * ceil(3 sqrt(Sigma2D_xx)) and ceil(3 sqrt(Sigma2D_yy)) pixels.  A Gaussian is
 * not listed when z_c < near_z, det <= 0 or its rect misses the image.
 * ------------------------------------------------------------------------- */
gm_status gm_project_gaussians(const gm_camera* cam, int32_t N, const float* means,
                               const float* quats, const float* scales, const float* opacity,
                               const float* sh, int32_t sh_degree, float* rec, hipStream_t stream);

/* gm_project_gaussians_multi — the projection of the same Gaussians into several
 * views in one pass.  README "Limitations and Todos": rendering a batch of camera
 * poses is listed as not yet supported; the world-space work (reading the parameters and colour
 * coefficients, normalising q, forming Sigma) does not depend on the view, so it is
 * done once per Gaussian and every view's record follows from it.
 *
 * cams: host array of nviews cameras.  Inputs as gm_project_gaussians.  Output rec
 * [nviews][N][GM_REC]: the records of view v start at rec + v N GM_REC and are
 * bitwise equal to those gm_project_gaussians writes for cams[v].  Views are
 * processed 16 to a launch.  GM_ERR_ARG on a NULL or invalid camera, negative N or
 * nviews, sh_degree outside -1..3 or misaligned rec; nviews = 0 or N = 0 does
 * nothing.  Asynchronous on stream.
 * ------------------------------------------------------------------------- */
gm_status gm_project_gaussians_multi(const gm_camera* cams, int32_t nviews, int32_t N, const float* means,
                                     const float* quats, const float* scales, const float* opacity,
                                     const float* sh, int32_t sh_degree, float* rec, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 4. gm_sort_tile_keys — occlusion cull, per-tile lists in depth order.
 * README "Hybrid rendering": Gaussians are composited "in the usual sorted 3DGS
 * order" (Limitations: sorted by centre depth); cull_occluded removes Gaussians
 * certainly hidden behind the mesh in fully covered 16x16 tiles without changing
 * the result.
 *
 * Lists every listed Gaussian i in every tile of its rect, ordered by (bits of
 * fp32 z_c, i).  With tile_dmax != NULL, pair (t, i) is dropped when t is fully
 * covered (tile_dmax[t] < inf) and
 *   min(0.99, o_i) Phi((Dmax_t + 1e-5 |Dmax_t| - zmin_ti) / (sigma_i softness))
 *     < (1/255)(1 - 1e-3),
 * zmin_ti = min of z*_i over the four corner pixel centres of the tile (softness 0:
 * dropped when zmin_ti >= Dmax_t + 1e-5 |Dmax_t|).  Such a pair falls under the
 * 1/255 skip rule at every pixel of the tile, so outputs are unchanged.
 * Outputs: tile_ranges [T][2] = [start, end) into sorted_ids [n_keys].
 * cap: capacity of sorted_ids; n_keys (device int64, out): number of listed pairs
 * (negative if list construction failed, which does not happen in correct use);
 * above cap, every tile range is [0, 0) and the contents of sorted_ids are
 * unspecified.  ws: at least gm_sort_tile_keys_ws(N, cap, W, H) bytes.
 * ------------------------------------------------------------------------- */
size_t gm_sort_tile_keys_ws(int32_t N, int64_t cap, int32_t width, int32_t height);
gm_status gm_sort_tile_keys(const gm_camera* cam, int32_t N, const float* rec,
                            const float* tile_dmax, float softness, int32_t* tile_ranges,
                            int32_t* sorted_ids, int64_t cap, int64_t* n_keys, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* The two halves of gm_sort_tile_keys, which is gm_sort_depth followed by
 * gm_sort_tiles with the same arguments.  gm_sort_depth orders the N Gaussians by
 * (bits of z_c, i) and keeps that order in ws; it reads rec only (not tile_dmax), so
 * a caller may run it on another stream than the mesh's z-buffer.  gm_sort_tiles
 * then culls, lists and sorts by tile; it must be ordered after gm_sort_depth on the
 * same ws, rec, N, cap and image size (same ws_bytes rule), and after whatever
 * wrote tile_dmax.  Between the two calls ws belongs to the pair: no other call may
 * use it.  Arguments, outputs and errors as for gm_sort_tile_keys. */
gm_status gm_sort_depth(const gm_camera* cam, int32_t N, const float* rec, int64_t cap, void* ws,
                        size_t ws_bytes, hipStream_t stream);
gm_status gm_sort_tiles(const gm_camera* cam, int32_t N, const float* rec, const float* tile_dmax,
                        float softness, int32_t* tile_ranges, int32_t* sorted_ids, int64_t cap,
                        int64_t* n_keys, void* ws, size_t ws_bytes, hipStream_t stream);

/* gm_project_gaussians followed by gm_sort_depth, in fewer launches: the projection
 * kernel also writes the depth sort's keys and ids into ws, so the sort does not
 * read them back from rec.  rec and ws end as after the two calls with the same
 * arguments (the records and the depth order bit for bit), and gm_sort_tiles follows
 * on the same ws as after gm_sort_depth.  Arguments as for those two calls (cap and
 * ws as for gm_sort_depth); errors as for either. */
gm_status gm_project_sort_depth(const gm_camera* cam, int32_t N, const float* means,
                                const float* quats, const float* scales, const float* opacity,
                                const float* sh, int32_t sh_degree, float* rec, int64_t cap,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 5. gm_composite_hybrid_fwd — depth-tested front-to-back composite.
 * README "Hybrid rendering": per pixel each Gaussian is split at the mesh surface,
 * f = Phi((D - z*(p)) / (sigma softness)); front parts alpha f and back parts
 * alpha (1 - f) form two layers, C = C_front + T_front (a_m c_m + (1 - a_m)(C_back +
 * T_back bg)).  Mesh coverage a_m is binary here (no edge antialiasing), so the
 * back layer never contributes and one front layer is evaluated:
 *   alpha_i = min(0.99, o exp(-q)), q = (Q00 dx^2 + 2 Q01 dx dy + Q11 dy^2)/2,
 *   alpha_F = alpha f (f = 1 off the mesh), entries with alpha_F < 1/255 skipped,
 *   the walk stops before an entry that would bring T below 1e-4;
 *   rgb = C_F + T_F (a_m c_m + (1 - a_m) bg), alpha = 1 - T_F (1 - a_m),
 *   depth = sum w_i z_c,i + T_F a_m D.
 * c_m: perspective-correct barycentrics from face_id; base colour from vertex
 * colours or the trilinear mip texture; Phong when `light` and normals are given:
 *   c_m = base (ka + kd max(0, n.l)) + ks [n.l > 0] max(0, r.e)^shininess.
 * Inputs: the outputs of calls 1-4; bg (host, 3 floats); softness >= 0.
 * Outputs: out_rgb [H][W][3], out_depth [H][W], out_alpha [H][W]; state for the
 * backward: state_T [H][W] (final transmittance), state_last [H][W] (index in the
 * tile list + 1 of the last included entry), state_cm [H][W][3] (the colour behind
 * the Gaussians: c_m on the mesh, bg elsewhere).  Deterministic.
 * ------------------------------------------------------------------------- */
gm_status gm_composite_hybrid_fwd(const gm_camera* cam, const float* rec,
                                  const int32_t* tile_ranges, const int32_t* sorted_ids,
                                  const int32_t* face_id, const float* depth, const gm_mesh* mesh,
                                  const float* vscreen, const gm_light* light, const float* bg,
                                  float softness, float* out_rgb, float* out_depth,
                                  float* out_alpha, float* state_T, int32_t* state_last,
                                  float* state_cm, hipStream_t stream);

/* The two halves of gm_composite_hybrid_fwd, which is gm_shade_surface followed by
 * gm_composite_hybrid_fwd_shaded with the same arguments.  gm_shade_surface writes
 * state_cm [H][W][3] (c_m where face_id >= 0, bg elsewhere); it reads the z-buffer's
 * face_id, the mesh, vscreen and light, not the lists, so a caller may run it on
 * another stream beside the tile sort.  gm_composite_hybrid_fwd_shaded takes that
 * state_cm as input (ordered after gm_shade_surface; bg enters only through it) and
 * writes the other outputs of gm_composite_hybrid_fwd, bit for bit the same.
 * Errors as for gm_composite_hybrid_fwd. */
gm_status gm_shade_surface(const gm_camera* cam, const int32_t* face_id, const gm_mesh* mesh,
                           const float* vscreen, const gm_light* light, const float* bg,
                           float* state_cm, hipStream_t stream);
gm_status gm_composite_hybrid_fwd_shaded(const gm_camera* cam, const float* rec,
                                         const int32_t* tile_ranges, const int32_t* sorted_ids,
                                         const int32_t* face_id, const float* depth, float softness,
                                         const float* state_cm, float* out_rgb, float* out_depth,
                                         float* out_alpha, float* state_T, int32_t* state_last,
                                         hipStream_t stream);

/* gm_composite_hybrid_fwd_stats — a measurement aid: gm_composite_hybrid_fwd_shaded
 * (same arguments, same outputs bit for bit) built with counters, which it ADDS to
 * stats (device int64 [3], zeroed by the caller): [0] included (pixel, entry) pairs
 * (the pairs the composite accumulates), [1] list entries evaluated wave-wide (one
 * per wave and entry: the unit of the kernel's per-entry instruction count), [2]
 * list entries staged into LDS.  Slower than the uncounted call; not part of the
 * rendering path. */
gm_status gm_composite_hybrid_fwd_stats(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                        const int32_t* sorted_ids, const int32_t* face_id, const float* depth,
                                        float softness, const float* state_cm, float* out_rgb, float* out_depth,
                                        float* out_alpha, float* state_T, int32_t* state_last, int64_t* stats,
                                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 6. gm_composite_hybrid_bwd — reverse mode of call 5.
 * README "Hybrid rendering": everything is differentiable, Gaussian parameters
 * also through the split, and the mesh through its depth and interpolated colour.
 *
 * Inputs: the camera, records, lists, z-buffer and softness given to call 5, its
 * three state buffers, and upstream gradients g_rgb [H][W][3], g_depth [H][W] (or
 * NULL = 0), g_alpha [H][W] (or NULL = 0).
 * Outputs (zero-filled by the call, then accumulated with float atomics):
 *   g_rec [N][GM_GRAD]: d/d(u, v, Q00, Q01, Q11, opacity, r, g, b, z_c, g0, g1, sigma);
 *   g_mesh_rgb [H][W][3] = dL/dc_m, g_mesh_depth [H][W] = dL/dD (either may be NULL).
 * Skipped and stopped entries get no gradient; the clamp at 0.99 has zero
 * derivative; the decisions are not differentiated.  The transmittance before each
 * entry is recovered from the final one by division (1 - alpha_F >= 0.01).
 * ws: at least gm_composite_hybrid_bwd_ws(W, H) bytes of device scratch (every tile's
 * walk length from the forward state and the order in which the tiles are taken,
 * longest first); its contents are not kept between calls.  The outputs do not
 * depend on that order beyond the summation order of the float atomics.
 * ------------------------------------------------------------------------- */
size_t gm_composite_hybrid_bwd_ws(int32_t width, int32_t height);
gm_status gm_composite_hybrid_bwd(const gm_camera* cam, int32_t N, const float* rec,
                                  const int32_t* tile_ranges, const int32_t* sorted_ids,
                                  const int32_t* face_id, const float* depth, float softness,
                                  const float* state_T, const int32_t* state_last,
                                  const float* state_cm, const float* g_rgb, const float* g_depth,
                                  const float* g_alpha, float* g_rec, float* g_mesh_rgb,
                                  float* g_mesh_depth, void* ws, size_t ws_bytes, hipStream_t stream);

/* gm_composite_hybrid_bwd_noalloc — call 6 for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and errors as gm_composite_hybrid_bwd
 * without ws / ws_bytes.  Its scratch (tile walk lengths and tile order) is a fixed
 * device array inside the library, GM_NOALLOC_MAX_TILES * 8 bytes (512 KiB), held
 * by every GPU the library runs on until the process ends; its address on a device
 * is looked up on the first call there.  The call allocates nothing (no hipMalloc,
 * no library allocation) and never clears that scratch with a memset (every entry
 * is written before it is read).  Images of more than GM_NOALLOC_MAX_TILES 16x16
 * tiles (above 4096 x 4096 pixels) are GM_ERR_ARG.  `stream` must belong to the
 * current device (GM_ERR_ARG otherwise).  All calls on one GPU share the one
 * scratch: calls that overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller. */
#define GM_NOALLOC_MAX_TILES 65536
gm_status gm_composite_hybrid_bwd_noalloc(const gm_camera* cam, int32_t N, const float* rec,
                                          const int32_t* tile_ranges, const int32_t* sorted_ids,
                                          const int32_t* face_id, const float* depth, float softness,
                                          const float* state_T, const int32_t* state_last, const float* state_cm,
                                          const float* g_rgb, const float* g_depth, const float* g_alpha,
                                          float* g_rec, float* g_mesh_rgb, float* g_mesh_depth, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 7. gm_project_gaussians_bwd — gradients of the Gaussians' own parameters.
 * README "Hybrid rendering": the renderer is differentiable end to end, through the
 * depth split as well, so means, rotations, scales, opacities and colour
 * coefficients get gradients through their projected records.
 *
 * Reverse mode of call 3 for every Gaussian: given g_rec [N][GM_GRAD] (the record
 * gradients of call 6: u, v, Q00, Q01, Q11, opacity, r, g, b, z_c, g0, g1, sigma),
 * writes g_means [3][N], g_quats [4][N] (raw quaternion, before normalisation),
 * g_scales [3][N] (linear scales), g_opacity [N] and g_sh [(d+1)^2][3][N] (or
 * [1][3][N] for sh_degree = -1).  Optional outputs (NULL to skip): g_log_scales
 * [3][N] = g_scales * scales and g_logit_opacity [N] = g_opacity * o (1 - o), the
 * gradients with respect to log-scales and opacity logits (opacity is then
 * required).  Inputs are those of call 3 plus its output rec; Gaussians that rec
 * does not list (word 15 = 0) get zeros.  A colour channel clamped at zero in the
 * forward passes no gradient.  Every output element is written (no accumulation).
 * ------------------------------------------------------------------------- */
gm_status gm_project_gaussians_bwd(const gm_camera* cam, int32_t N, const float* means,
                                   const float* quats, const float* scales, const float* opacity,
                                   const float* sh, int32_t sh_degree, const float* rec,
                                   const float* g_rec, float* g_means, float* g_quats,
                                   float* g_scales, float* g_opacity, float* g_sh,
                                   float* g_log_scales, float* g_logit_opacity, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 8. gm_mesh_bwd — gradients of the mesh's own parameters.
 * README "Design Details": the surface colour c_m comes from perspective-correct
 * barycentrics of the nearest triangle (vertex colours, or the trilinear mip-mapped
 * texture at the interpolated texture coordinate), lit per pixel by Phong shading of
 * interpolated normals (v1.1 notes); the mesh depth D enters the composite through
 * the split; the renderer is differentiable with respect to the mesh as well.
 *
 * Given g_mesh_rgb [H][W][3] = dL/dc_m and g_mesh_depth [H][W] = dL/dD (outputs of
 * call 6; either may be NULL) and the face_id buffer of call 2, writes the gradients
 * of the inputs of the surface colour and depth: g_verts [3][V] (world positions,
 * through the barycentrics, D and the lighting's view vectors), g_vcolor [3][V],
 * g_vnormal [3][V], g_uv [2][Vt], g_mips (gm_mipmaps_floats(S) floats; on return
 * its first S*S*3 floats hold dL/dtexture [S][S][3], the coarser levels hold the
 * intermediate sums of the pyramid's adjoint) and g_light [13] (pos[3], ambient[3],
 * diffuse[3], specular[3], shininess).  Outputs are zero-filled by the call; NULL
 * ones are skipped (g_vcolor needs vertex colours, g_vnormal and g_light a light and
 * normals, g_uv and g_mips a textured mesh).  Which face covers a pixel and the
 * texture's level of detail are taken as given (no gradient through them); a clamp
 * passes no gradient on its clamped side.  Vertex positions are taken in fp64
 * through the same camera as call 1.
 * ------------------------------------------------------------------------- */
gm_status gm_mesh_bwd(const gm_camera* cam, const gm_mesh* mesh, const gm_light* light,
                      const int32_t* face_id, const float* g_mesh_rgb, const float* g_mesh_depth,
                      float* g_verts, float* g_vcolor, float* g_vnormal, float* g_uv, float* g_mips,
                      float* g_light, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 9. Analytic edge antialiasing (README "Design Details > Mesh rasterizer", step 3,
 * and "Limitations and Todos": as in nvdiffrast, wherever two neighbouring pixels
 * see a silhouette, the point where the front surface's edge crosses between the
 * two pixel centres gives a fractional coverage and blends the colour over the
 * farther surface; internal edges of a connected surface are left alone; a
 * per-axis one-dimensional approximation, exact for straight edges away from
 * corners.  "Hybrid rendering": the mesh coverage a_m is then fractional at
 * silhouettes and the general two-layer composite
 * C = C_front + T_front (a_m c_m + (1 - a_m)(C_back + T_back bg)) applies).
 *
 * Readings (what the README leaves open):
 *  - Pairs: horizontally and vertically adjacent pixels whose z-buffer faces
 *    differ.  The front pixel a is the covered one, or the one with the smaller
 *    depth-buffer value (equal: smaller face id); b is the other.
 *  - The segment from a's centre to b's is followed over the front surface: it
 *    leaves a triangle through the edge whose inside-positive edge function falls
 *    to zero first, t = e(a) / (e(a) - e(b)) (edges with e(b) < e(a); ties: lower
 *    edge index); an internal edge passes it to the neighbouring face; the first
 *    silhouette edge gives the crossing t in [0, 1).  No effect when a triangle
 *    holds the rest of the segment or after 16 triangles.
 *  - Silhouette edge (edge k of face f runs from corner k+1 to corner k+2): no
 *    other face has its two vertex indices, several do, the one that does is not
 *    drawn in this view (masked, behind the near plane, zero area), or it faces
 *    the other way (opposite sign of the screen-space area).
 *  - Horizontal pairs take edges at least as steep as 45 degrees (|dv| >= |du|),
 *    vertical pairs the others.
 *  - 1D box filter: d = t - 1/2 < 0 moves the fraction -d of a to b's surface;
 *    d > 0 gives b the fraction d of a's surface.  A pixel's surface is its
 *    z-buffer colour c and depth D; an uncovered pixel has none.
 *  - Per pixel the pairs' effects add up into weights of its own and its four
 *    neighbours' surfaces: coverage a = sum of weights, premultiplied colour
 *    M = sum w c, depth M_D = sum w D.  a is clamped to [0, 1] with M and M_D
 *    scaled by (clamped / raw) (0 for raw <= 0).
 *  - The depth that splits the Gaussians: D on a covered pixel; on an uncovered
 *    pixel that receives coverage, the smallest D of the neighbours giving it;
 *    +inf otherwise.
 * Decisions and crossings are fp64 from the fp32 screen vertices (no contraction).
 *
 * gm_edge_adjacency: adj [3][F] int32, for edge k of face f the one other face with
 * the same two vertex indices, -1 if none, -2 if several; view independent, once
 * per mesh.  Workspace gm_edge_adjacency_ws(F) bytes (a hash table).
 *
 * gm_antialias: from the z-buffer of call 2 (face_id, depth), vscreen of call 1 and
 * adj, writes colour [H][W][3] (the shaded surface colour at covered pixels, 0
 * elsewhere; needed again by the reverse mode), the mesh layer [H][W][8] =
 * (M_r, M_g, M_b, M_D, a_m, D_split, 0, 0) and, when pairs is not NULL, the
 * per-pixel record of the pairs the reverse mode reads instead of repeating the
 * analysis, [H][W][12]: the five weights (own surface, left, right, up, down), the
 * clamp branch (int32: 0 unclamped, 1 scaled down from above 1, 2 zero) and the raw
 * coverage, then per direction an int32 code, -1 when that pair does not change the
 * pixel, else ((3 face + edge) << 2) | (screen area > 0) << 1 | (pixel is the front
 * one).  layer and pairs are 16-byte aligned.  When tile_dmax (the cull bound of
 * call 2) is given, every tile holding a covered pixel with a_m < 1 gets +inf, so
 * that call 4 culls only where the back layer is hidden.
 *
 * gm_composite_hybrid_fwd_aa / _bwd_aa: calls 5 and 6 with the mesh given by its
 * layer (bg: host, 3 floats, as in call 5).  Both layers follow the per-layer
 * rules of call 5; the back layer is composited where it is visible (a_m < 1 and a
 * finite D_split), and the pixel stops when its front layer stops (the 3DGS stop
 * is per pixel, and the back layer is seen only through T_F).  Outputs as call
 * 5: rgb = C_F + T_F (M + (1 - a_m)(C_B + T_B bg)), alpha = 1 - T_F (1 - a_m) T_B,
 * depth = Z_F + T_F (M_D + (1 - a_m) Z_B).  state [H][W][8] = (T_F, last_F as
 * int32, T_B, last_B as int32, C_B rgb, Z_B).  The reverse mode writes g_rec as
 * call 6 (zero-filled first) and g_layer [H][W][8] = dL/d(M_rgb, M_D, a_m,
 * D_split), 0, 0; its ws is call 6's (gm_composite_hybrid_bwd_ws bytes), the walk
 * length of a pixel being the longer of its two layers'.
 *
 * gm_antialias_bwd: reverse mode of gm_antialias, from its pairs record (the
 * crossings are recomputed from the recorded silhouette edges).  From g_layer it writes
 * g_mesh_rgb [H][W][3] and g_mesh_depth [H][W] (dL/dc and dL/dD at covered pixels'
 * own centres, 0 elsewhere: the inputs of call 8) and g_vscreen [2][V] (dL/du,
 * dL/dv of the screen vertices through the crossings; zero-filled first).  The
 * decisions (front pixel, edge, silhouette, axis, clamp branch, split neighbour)
 * carry no gradient.  Workspace gm_antialias_bwd_ws(width, height) bytes.
 *
 * gm_vscreen_bwd: adds to g_verts [3][V] the chain of g_vscreen through the
 * camera projection of call 1 (after call 8, which zero-fills g_verts).
 * ------------------------------------------------------------------------- */
size_t gm_edge_adjacency_ws(int32_t F);
gm_status gm_edge_adjacency(const gm_mesh* mesh, int32_t* adj, void* ws, size_t ws_bytes, hipStream_t stream);
gm_status gm_antialias(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen, const int32_t* adj,
                       const gm_light* light, const int32_t* face_id, const float* depth, float* colour,
                       float* layer, float* pairs, float* tile_dmax, hipStream_t stream);
gm_status gm_composite_hybrid_fwd_aa(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                     const int32_t* sorted_ids, const float* layer, const float* bg,
                                     float softness, float* out_rgb, float* out_depth, float* out_alpha,
                                     float* state, hipStream_t stream);
gm_status gm_composite_hybrid_bwd_aa(const gm_camera* cam, int32_t N, const float* rec,
                                     const int32_t* tile_ranges, const int32_t* sorted_ids, const float* layer,
                                     const float* bg, float softness, const float* state, const float* g_rgb,
                                     const float* g_depth, const float* g_alpha, float* g_rec, float* g_layer,
                                     void* ws, size_t ws_bytes, hipStream_t stream);
size_t gm_antialias_bwd_ws(int32_t width, int32_t height);
gm_status gm_antialias_bwd(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen, const float* pairs,
                           const int32_t* face_id, const float* depth, const float* colour,
                           const float* g_layer, float* g_mesh_rgb, float* g_mesh_depth, float* g_vscreen,
                           void* ws, size_t ws_bytes, hipStream_t stream);
gm_status gm_vscreen_bwd(const gm_camera* cam, const gm_mesh* mesh, const float* g_vscreen, float* g_verts,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Auxiliary.
 * gm_build_mipmaps: README v1.1 (trilinear mipmapping by default): box-filter
 * pyramid of a square power-of-two texture tex [S][S][3] (HWC, values in [0, 1]);
 * level l+1 texel = mean of the 2x2 block below it; levels stored back to back in
 * mips [gm_mipmaps_floats(S)].
 * ------------------------------------------------------------------------- */
size_t gm_mipmaps_floats(int32_t S);
gm_status gm_build_mipmaps(const float* tex, int32_t S, float* mips, hipStream_t stream);

/* Thread-local message for the last non-OK status of this thread ("" if none). */
const char* gm_last_error(void);
/* ABI version (major * 100 + minor). */
int32_t gm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GM_H */
