/*
 * CPU oracle for the hybrid mesh + 3D Gaussian tile rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library: it is a plain, slow, direct transcription
 * of what the method computes, so that a reader can check it against the gmesh
 * README ("A Lightweight and Differentiable Renderer for Joint Mesh and 3D Gaussian
 * Splat Scenes") by eye.
 *
 * Precision rules.
 *  - "Decision" arithmetic, whose result picks an integer (which triangle is
 *    nearest, which tiles a Gaussian touches, the depth order of Gaussians), is the
 *    kernel's precision: vertex and Gaussian projection in fp32 in the written
 *    evaluation order with no fused multiply-add (build with -ffp-contract=off), and
 *    edge functions / mesh depth in fp64.
 *  - Everything else (SH colour, shading, texture filtering, compositing and its
 *    reverse mode) is fp64, from the fp32 records and the fp32 depth buffer.
 *
 * Pins: every function here is checked in tests/ against closed forms, brute force
 * (exact rational coverage), invariants and finite differences.  Parts that the
 * pages leave unstated (the 0.3 px^2 dilation, 1/255, 1e-4, 0.99, the near plane,
 * the cull margin, SH signs beyond band 0, the Phong guard, LOD details, the depth
 * output) are readings; their pins check this spec, not the pages.
 *
 * Conventions (gmesh README, "Design Details": the mesh uses the same pinhole
 * camera and pixel convention as the Gaussians; the "Camera Coordinates" section is
 * empty in the page text, so the gsplat/OpenCV reading is taken):
 *   x_c = R x_w + t (R row-major), +x right, +y down, +z forward;
 *   u = fx x_c / z_c + cx, v = fy y_c / z_c + cy;
 *   pixel (i, j) = column i, row j, centre (i + 0.5, j + 0.5);
 *   tile (tx, ty) = pixels [16tx, 16tx+16) x [16ty, 16ty+16), id = ty*TX + tx.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OC_TILE 16
#define OC_NREC 13

typedef struct {
    int width, height;
    float fx, fy, cx, cy;
    float R[9], t[3];
    float near_z;
} oc_camera;

typedef struct {
    float pos[3], ambient[3], diffuse[3], specular[3], shininess;
} oc_light;

static int tiles_x(const oc_camera* c) { return (c->width + OC_TILE - 1) / OC_TILE; }
static int tiles_y(const oc_camera* c) { return (c->height + OC_TILE - 1) / OC_TILE; }

/* ------------------------------------------------------------------------- */
/* Mesh visibility (README, Design Details > Mesh rasterizer, step 1: triangles   */
/* binned into 16x16 tiles, nearest triangle at each pixel centre; "Triangles     */
/* with a vertex in front of the near plane are skipped").                        */
/* ------------------------------------------------------------------------- */

/* Vertex projection, fp32, written order. vscreen = [u][v][z_c] planes. */
void oc_project_vertices(const oc_camera* cam, int V, const float* verts, float* vscreen)
{
    const float* R = cam->R;
    for (int i = 0; i < V; ++i) {
        float x = verts[i], y = verts[V + i], z = verts[2 * V + i];
        float xc = ((R[0] * x + R[1] * y) + R[2] * z) + cam->t[0];
        float yc = ((R[3] * x + R[4] * y) + R[5] * z) + cam->t[1];
        float zc = ((R[6] * x + R[7] * y) + R[8] * z) + cam->t[2];
        float u = (cam->fx * xc) / zc + cam->cx;
        float v = (cam->fy * yc) / zc + cam->cy;
        vscreen[i] = u;
        vscreen[V + i] = v;
        vscreen[2 * V + i] = zc;
    }
}

/* Triangle setup shared by the raster and the shading below. */
typedef struct {
    double u[3], v[3], z[3];
    double A; /* twice the signed screen area */
    int valid;
} oc_tri;

static void tri_setup(const oc_camera* cam, int V, const float* vscreen, const int* faces,
                      const unsigned char* mask, int F, int f, oc_tri* t)
{
    t->valid = 0;
    if (mask && !mask[f]) return;
    for (int k = 0; k < 3; ++k) {
        int vi = faces[k * F + f];
        t->u[k] = (double)vscreen[vi];
        t->v[k] = (double)vscreen[V + vi];
        t->z[k] = (double)vscreen[2 * V + vi];
        if (!(vscreen[2 * V + vi] >= cam->near_z)) return; /* near plane: skip */
    }
    t->A = (t->u[1] - t->u[0]) * (t->v[2] - t->v[0]) - (t->v[1] - t->v[0]) * (t->u[2] - t->u[0]);
    t->valid = (t->A != 0.0);
}

/* Edge function of a->b at p: (b.u-a.u)(p.v-a.v) - (b.v-a.v)(p.u-a.u). */
static double edge(double au, double av, double bu, double bv, double pu, double pv)
{
    return (bu - au) * (pv - av) - (bv - av) * (pu - au);
}

/* Coverage of pixel centre (pu, pv): inclusive test E_k * sign(A) >= 0 for all k
 * (no fill rule, no back-face culling: triangle soups have arbitrary winding).
 * On success returns 1 with lambda[] = E_k / A and the perspective-correct depth. */
static int tri_cover(const oc_tri* t, double pu, double pv, double lam[3], double* zout)
{
    double E0 = edge(t->u[1], t->v[1], t->u[2], t->v[2], pu, pv);
    double E1 = edge(t->u[2], t->v[2], t->u[0], t->v[0], pu, pv);
    double E2 = edge(t->u[0], t->v[0], t->u[1], t->v[1], pu, pv);
    if (t->A > 0) {
        if (E0 < 0 || E1 < 0 || E2 < 0) return 0;
    } else {
        if (E0 > 0 || E1 > 0 || E2 > 0) return 0;
    }
    lam[0] = E0 / t->A;
    lam[1] = E1 / t->A;
    lam[2] = E2 / t->A;
    double inv = (lam[0] / t->z[0] + lam[1] / t->z[1]) + lam[2] / t->z[2];
    *zout = 1.0 / inv;
    return 1;
}

/* Pixel-centre bounding box of a valid triangle as a pixel-index range; returns 0
 * when no pixel centre of the image lies inside it. */
static int tri_pixel_box(const oc_camera* cam, const oc_tri* t, int* x0, int* x1, int* y0, int* y1)
{
    double umin = fmin(fmin(t->u[0], t->u[1]), t->u[2]);
    double umax = fmax(fmax(t->u[0], t->u[1]), t->u[2]);
    double vmin = fmin(fmin(t->v[0], t->v[1]), t->v[2]);
    double vmax = fmax(fmax(t->v[0], t->v[1]), t->v[2]);
    double a = ceil(umin - 0.5), b = floor(umax - 0.5);
    double c = ceil(vmin - 0.5), d = floor(vmax - 0.5);
    a = fmax(a, 0.0);
    c = fmax(c, 0.0);
    b = fmin(b, (double)(cam->width - 1));
    d = fmin(d, (double)(cam->height - 1));
    if (!(a <= b) || !(c <= d)) return 0;
    *x0 = (int)a; *x1 = (int)b; *y0 = (int)c; *y1 = (int)d;
    return 1;
}

/* Triangle bins: for every tile the ids of valid triangles whose pixel-centre box
 * meets the tile, in increasing id.  counts[T]; if tris != NULL also offsets[T+1]
 * (caller-computed) are used to write ids. */
void oc_tile_bins(const oc_camera* cam, int V, int F, const float* vscreen, const int* faces,
                  const unsigned char* mask, int* counts, const int* offsets, int* tris)
{
    int TX = tiles_x(cam), TY = tiles_y(cam), T = TX * TY;
    int* cursor = NULL;
    if (tris) {
        cursor = (int*)malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
        for (int i = 0; i < T; ++i) cursor[i] = offsets[i];
    }
    for (int i = 0; i < T; ++i) counts[i] = 0;
    for (int f = 0; f < F; ++f) {
        oc_tri t;
        tri_setup(cam, V, vscreen, faces, mask, F, f, &t);
        if (!t.valid) continue;
        int x0, x1, y0, y1;
        if (!tri_pixel_box(cam, &t, &x0, &x1, &y0, &y1)) continue;
        for (int ty = y0 / OC_TILE; ty <= y1 / OC_TILE; ++ty)
            for (int tx = x0 / OC_TILE; tx <= x1 / OC_TILE; ++tx) {
                int id = ty * TX + tx;
                counts[id]++;
                if (tris) tris[cursor[id]++] = f;
            }
    }
    free(cursor);
}

/* Nearest covering triangle at the pixel centres of the requested tiles.
 * The smaller fp64 depth wins; an exact tie keeps the smaller face id.
 * prefilter = 0: every pixel tests every face (the literal definition).
 * prefilter = 1: every pixel tests the faces of its tile's bin (same predicate,
 *                only skipping faces whose pixel-centre box misses the tile).
 * Outputs are full-image arrays; only pixels of requested tiles are written:
 * face_id (-1 empty), depth = (float)z (+inf empty), z1/z2 = nearest and second
 * nearest fp64 depth (+inf if absent), tile_dmax[tile] = max depth over the tile's
 * in-image pixels (+inf if any of them is empty). */
void oc_zbuffer(const oc_camera* cam, int V, int F, const float* vscreen, const int* faces,
                const unsigned char* mask, int ntiles, const int* tiles, int prefilter,
                int* face_id, float* depth, double* z1out, double* z2out, float* tile_dmax)
{
    int W = cam->width, H = cam->height, TX = tiles_x(cam);
    oc_tri* tri = (oc_tri*)malloc(sizeof(oc_tri) * (size_t)(F > 0 ? F : 1));
    for (int f = 0; f < F; ++f) tri_setup(cam, V, vscreen, faces, mask, F, f, &tri[f]);

#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < ntiles; ++k) {
        int tile = tiles[k];
        int tx = tile % TX, ty = tile / TX;
        int px0 = tx * OC_TILE, py0 = ty * OC_TILE;
        int px1 = px0 + OC_TILE < W ? px0 + OC_TILE : W;
        int py1 = py0 + OC_TILE < H ? py0 + OC_TILE : H;
        int* cand = NULL;
        int ncand = 0;
        if (prefilter) {
            cand = (int*)malloc(sizeof(int) * (size_t)(F > 0 ? F : 1));
            for (int f = 0; f < F; ++f) {
                int x0, x1, y0, y1;
                if (!tri[f].valid || !tri_pixel_box(cam, &tri[f], &x0, &x1, &y0, &y1)) continue;
                if (x1 < px0 || x0 >= px1 || y1 < py0 || y0 >= py1) continue;
                cand[ncand++] = f;
            }
        }
        float dmax = -INFINITY;
        int full = 1;
        for (int py = py0; py < py1; ++py)
            for (int px = px0; px < px1; ++px) {
                double pu = px + 0.5, pv = py + 0.5;
                double best = INFINITY, second = INFINITY;
                int bid = -1;
                int n = prefilter ? ncand : F;
                for (int c = 0; c < n; ++c) {
                    int f = prefilter ? cand[c] : c;
                    if (!tri[f].valid) continue;
                    double lam[3], z;
                    if (!tri_cover(&tri[f], pu, pv, lam, &z)) continue;
                    if (z < best) {
                        second = best;
                        best = z;
                        bid = f;
                    } else if (z < second) {
                        second = z;
                    }
                }
                int p = py * W + px;
                face_id[p] = bid;
                depth[p] = bid >= 0 ? (float)best : INFINITY;
                if (z1out) z1out[p] = best;
                if (z2out) z2out[p] = second;
                if (bid < 0) full = 0;
                else if (depth[p] > dmax) dmax = depth[p];
            }
        tile_dmax[tile] = full ? dmax : INFINITY;
        free(cand);
    }
    free(tri);
}

/* ------------------------------------------------------------------------- */
/* 3D Gaussian projection and the EWA conditional depth model (README, Design      */
/* Details > Hybrid rendering: z*(p) = z_c + g.(p - mean2d), g = (Sigma_uv + eps I)^-1*/
/* Sigma_uv,z, sigma^2 = Sigma_zz - Sigma_z,uv g; the same local affine             */
/* approximation as the 2D splat).  fp32, written order, no contraction.             */
/* Records: [N][13] = u, v, Q00, Q01, Q11, opacity, r, g, b, z_c, g0, g1, sigma.     */
/* rect: [N][4] = tx0, ty0, tx1, ty1 (exclusive); valid[N].  rgb64: fp64 colour.      */
/* ------------------------------------------------------------------------- */

static const float OC_EPS2D = 0.3f;   /* px^2 low-pass dilation (3DGS value; eps of the page) */

/* Real spherical harmonics up to degree 3 (the Gaussian-splatting sign and order
 * convention), evaluated in fp64 at the unit direction (x, y, z). The constants are
 * written as their closed forms. */
static void sh_basis(double x, double y, double z, double* Y)
{
    const double pi = 3.14159265358979323846;
    Y[0] = 0.5 * sqrt(1.0 / pi);
    double c1 = sqrt(3.0 / (4.0 * pi));
    Y[1] = -c1 * y;
    Y[2] = c1 * z;
    Y[3] = -c1 * x;
    double a = 0.5 * sqrt(15.0 / pi), b = 0.25 * sqrt(5.0 / pi), c = 0.25 * sqrt(15.0 / pi);
    Y[4] = a * x * y;
    Y[5] = -a * y * z;
    Y[6] = b * (2.0 * z * z - x * x - y * y);
    Y[7] = -a * x * z;
    Y[8] = c * (x * x - y * y);
    double d0 = 0.25 * sqrt(35.0 / (2.0 * pi)), d1 = 0.5 * sqrt(105.0 / pi);
    double d2 = 0.25 * sqrt(21.0 / (2.0 * pi)), d3 = 0.25 * sqrt(7.0 / pi);
    double d5 = 0.25 * sqrt(105.0 / pi);
    Y[9] = -d0 * y * (3.0 * x * x - y * y);
    Y[10] = d1 * x * y * z;
    Y[11] = -d2 * y * (4.0 * z * z - x * x - y * y);
    Y[12] = d3 * z * (2.0 * z * z - 3.0 * x * x - 3.0 * y * y);
    Y[13] = -d2 * x * (4.0 * z * z - x * x - y * y);
    Y[14] = d5 * z * (x * x - y * y);
    Y[15] = -d0 * x * (x * x - 3.0 * y * y);
}

void oc_sh_basis(double x, double y, double z, double* Y) { sh_basis(x, y, z, Y); }

void oc_project_gaussians(const oc_camera* cam, int N, const float* means, const float* quats,
                          const float* scales, const float* opacity, const float* sh, int sh_degree,
                          float* rec, int* rect, int* valid, double* rgb64)
{
    const float* W = cam->R;
    const float* tt = cam->t;
    const float fx = cam->fx, fy = cam->fy, cx = cam->cx, cy = cam->cy;
    int TX = tiles_x(cam), TY = tiles_y(cam);
    /* camera centre in world space, C = -R^T t (fp64, colour only) */
    double Cw[3];
    for (int j = 0; j < 3; ++j)
        Cw[j] = -((double)W[0 * 3 + j] * tt[0] + (double)W[1 * 3 + j] * tt[1] + (double)W[2 * 3 + j] * tt[2]);

#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        float mx = means[i], my = means[N + i], mz = means[2 * N + i];
        float xc = ((W[0] * mx + W[1] * my) + W[2] * mz) + tt[0];
        float yc = ((W[3] * mx + W[4] * my) + W[5] * mz) + tt[1];
        float zc = ((W[6] * mx + W[7] * my) + W[8] * mz) + tt[2];
        int ok = (zc >= cam->near_z);

        float qw = quats[i], qx = quats[N + i], qy = quats[2 * N + i], qz = quats[3 * N + i];
        float qq = ((qw * qw + qx * qx) + qy * qy) + qz * qz;
        if (!(qq > 0.0f)) ok = 0;
        float qn = sqrtf(qq);
        qw = qw / qn; qx = qx / qn; qy = qy / qn; qz = qz / qn;
        float Rq[9];
        Rq[0] = 1.0f - 2.0f * ((qy * qy) + (qz * qz));
        Rq[1] = 2.0f * ((qx * qy) - (qw * qz));
        Rq[2] = 2.0f * ((qx * qz) + (qw * qy));
        Rq[3] = 2.0f * ((qx * qy) + (qw * qz));
        Rq[4] = 1.0f - 2.0f * ((qx * qx) + (qz * qz));
        Rq[5] = 2.0f * ((qy * qz) - (qw * qx));
        Rq[6] = 2.0f * ((qx * qz) - (qw * qy));
        Rq[7] = 2.0f * ((qy * qz) + (qw * qx));
        Rq[8] = 1.0f - 2.0f * ((qx * qx) + (qy * qy));
        float s[3] = {scales[i], scales[N + i], scales[2 * N + i]};
        float M[9];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) M[r * 3 + c] = Rq[r * 3 + c] * s[c];
        /* Sigma = M M^T (world), upper triangle mirrored */
        float S[9];
        for (int r = 0; r < 3; ++r)
            for (int c = r; c < 3; ++c) {
                float v = (M[r * 3 + 0] * M[c * 3 + 0] + M[r * 3 + 1] * M[c * 3 + 1]) + M[r * 3 + 2] * M[c * 3 + 2];
                S[r * 3 + c] = v;
                S[c * 3 + r] = v;
            }
        /* Sigma_c = (W Sigma) W^T */
        float A[9], C[9];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c)
                A[r * 3 + c] = (W[r * 3 + 0] * S[0 * 3 + c] + W[r * 3 + 1] * S[1 * 3 + c]) + W[r * 3 + 2] * S[2 * 3 + c];
        for (int r = 0; r < 3; ++r)
            for (int c = r; c < 3; ++c) {
                float v = (A[r * 3 + 0] * W[c * 3 + 0] + A[r * 3 + 1] * W[c * 3 + 1]) + A[r * 3 + 2] * W[c * 3 + 2];
                C[r * 3 + c] = v;
                C[c * 3 + r] = v;
            }
        /* Jacobian of the pinhole projection at the mean (no frustum clamp) */
        float z2 = zc * zc;
        float J00 = fx / zc;
        float J02 = -(fx * xc) / z2;
        float J11 = fy / zc;
        float J12 = -(fy * yc) / z2;
        float T0[3], T1[3];
        for (int c = 0; c < 3; ++c) {
            T0[c] = J00 * C[0 * 3 + c] + J02 * C[2 * 3 + c];
            T1[c] = J11 * C[1 * 3 + c] + J12 * C[2 * 3 + c];
        }
        float S00 = T0[0] * J00 + T0[2] * J02;
        float S01 = T0[1] * J11 + T0[2] * J12;
        float S11 = T1[1] * J11 + T1[2] * J12;
        float k0 = T0[2], k1 = T1[2], Szz = C[8];
        float a = S00 + OC_EPS2D, b = S01, c = S11 + OC_EPS2D;
        float det = a * c - b * b;
        if (!(det > 0.0f)) ok = 0;
        float Q00 = c / det, Q01 = (-b) / det, Q11 = a / det;
        float g0 = Q00 * k0 + Q01 * k1;
        float g1 = Q01 * k0 + Q11 * k1;
        float var = Szz - (k0 * g0 + k1 * g1);
        float sig = sqrtf(var > 1e-12f ? var : 1e-12f);
        float u = (fx * xc) / zc + cx;
        float v = (fy * yc) / zc + cy;
        /* tile rect: the bounding box of the 3-sigma ellipse of the dilated 2D
         * covariance, half-widths ceil(3 sqrt(a)) and ceil(3 sqrt(c)) pixels along
         * x and y (the ellipse (d^T Sigma2D^-1 d) <= 9 reaches |dx| = 3 sqrt(a)) */
        float radx = ceilf(3.0f * sqrtf(a));
        float rady = ceilf(3.0f * sqrtf(c));
        int r4[4] = {0, 0, 0, 0};
        if (ok) {
            float fx0 = floorf((u - radx) / 16.0f), fx1 = ceilf((u + radx) / 16.0f);
            float fy0 = floorf((v - rady) / 16.0f), fy1 = ceilf((v + rady) / 16.0f);
            fx0 = fminf(fmaxf(fx0, 0.0f), (float)TX);
            fx1 = fminf(fmaxf(fx1, 0.0f), (float)TX);
            fy0 = fminf(fmaxf(fy0, 0.0f), (float)TY);
            fy1 = fminf(fmaxf(fy1, 0.0f), (float)TY);
            r4[0] = (int)fx0; r4[1] = (int)fy0; r4[2] = (int)fx1; r4[3] = (int)fy1;
            if (r4[0] >= r4[2] || r4[1] >= r4[3]) { r4[0] = r4[1] = r4[2] = r4[3] = 0; }
        }
        if (!ok) { r4[0] = r4[1] = r4[2] = r4[3] = 0; }
        valid[i] = ok && (r4[2] > r4[0]);
        for (int k = 0; k < 4; ++k) rect[i * 4 + k] = r4[k];

        /* colour: SH in fp64 at the view direction; degree -1 = plain RGB */
        double col[3];
        if (sh_degree < 0) {
            for (int ch = 0; ch < 3; ++ch) col[ch] = (double)sh[ch * N + i];
        } else {
            double dx = (double)mx - Cw[0], dy = (double)my - Cw[1], dz = (double)mz - Cw[2];
            double nrm = sqrt(dx * dx + dy * dy + dz * dz);
            dx /= nrm; dy /= nrm; dz /= nrm;
            double Y[16];
            sh_basis(dx, dy, dz, Y);
            int K = (sh_degree + 1) * (sh_degree + 1);
            for (int ch = 0; ch < 3; ++ch) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k) acc += Y[k] * (double)sh[((size_t)k * 3 + ch) * N + i];
                acc += 0.5;
                col[ch] = acc > 0.0 ? acc : 0.0;
            }
        }
        float* o = rec + (size_t)i * OC_NREC;
        o[0] = u; o[1] = v; o[2] = Q00; o[3] = Q01; o[4] = Q11; o[5] = opacity[i];
        o[6] = (float)col[0]; o[7] = (float)col[1]; o[8] = (float)col[2];
        o[9] = zc; o[10] = g0; o[11] = g1; o[12] = sig;
        rgb64[(size_t)i * 3 + 0] = col[0];
        rgb64[(size_t)i * 3 + 1] = col[1];
        rgb64[(size_t)i * 3 + 2] = col[2];
    }
}

/* ------------------------------------------------------------------------- */
/* Depth order and per-tile lists (README, Design Details > Hybrid rendering:       */
/* "in the usual sorted 3DGS order"; Limitations: Gaussians sorted by centre depth). */
/* ------------------------------------------------------------------------- */

typedef struct { uint32_t key; int id; } oc_kv;

static int kv_cmp(const void* a, const void* b)
{
    const oc_kv* x = (const oc_kv*)a;
    const oc_kv* y = (const oc_kv*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return x->id < y->id ? -1 : (x->id > y->id);
}

/* Valid Gaussians ordered by (bits of fp32 z_c, id); z_c > 0 so the bit pattern
 * orders like the value.  Returns the count. */
int oc_depth_order(int N, const float* rec, const int* valid, int* order)
{
    oc_kv* kv = (oc_kv*)malloc(sizeof(oc_kv) * (size_t)(N > 0 ? N : 1));
    int n = 0;
    for (int i = 0; i < N; ++i) {
        if (!valid[i]) continue;
        uint32_t bits;
        float z = rec[(size_t)i * OC_NREC + 9];
        memcpy(&bits, &z, 4);
        kv[n].key = bits;
        kv[n].id = i;
        ++n;
    }
    qsort(kv, (size_t)n, sizeof(oc_kv), kv_cmp);
    for (int k = 0; k < n; ++k) order[k] = kv[k].id;
    free(kv);
    return n;
}

static double Phi(double s) { return 0.5 * erfc(-s / sqrt(2.0)); }
static double phi(double s) { return exp(-0.5 * s * s) / sqrt(2.0 * 3.14159265358979323846); }

/* Occlusion cull quantity for Gaussian i in tile `tile` (README, Hybrid rendering:
 * Gaussians "certainly hidden behind the mesh in fully covered 16x16 tiles" are
 * removed without changing the result).  In a fully covered tile every pixel has
 * D <= Dmax, and the Gaussian's conditional depth is affine in p, so its minimum
 * over the tile is at a corner pixel centre; f is monotone in D - z*, alpha is at
 * most min(0.99, o).  The pair can be dropped when that bound is below the 1/255
 * skip threshold with margin: a depth slack of 1e-5 Dmax and a 1e-3 relative
 * margin on the threshold.  Returns bound / threshold (< 1 means culled), or +inf
 * when the tile is not fully covered. */
static double cull_ratio(const oc_camera* cam, const float* r, float dmax, int tile, double softness)
{
    if (!(dmax < INFINITY)) return INFINITY;
    int TX = tiles_x(cam);
    int tx = tile % TX, ty = tile / TX;
    double xa = tx * OC_TILE + 0.5, ya = ty * OC_TILE + 0.5;
    int xe = (tx + 1) * OC_TILE < cam->width ? (tx + 1) * OC_TILE : cam->width;
    int ye = (ty + 1) * OC_TILE < cam->height ? (ty + 1) * OC_TILE : cam->height;
    double xb = xe - 0.5, yb = ye - 0.5;
    double u = r[0], v = r[1], zc = r[9], g0 = r[10], g1 = r[11], sg = r[12], o = r[5];
    double xs[2] = {xa, xb}, ys[2] = {ya, yb};
    double zmin = INFINITY;
    for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b) {
            double z = zc + (g0 * (xs[a] - u) + g1 * (ys[b] - v));
            if (z < zmin) zmin = z;
        }
    double thr = (1.0 / 255.0) * (1.0 - 1e-3);
    double slack = 1e-5 * fabs((double)dmax);
    double amax = o < 0.99 ? o : 0.99;
    double bound;
    if (softness > 0.0) {
        bound = amax * Phi(((double)dmax + slack - zmin) / (sg * softness));
    } else {
        bound = (zmin < (double)dmax + slack) ? amax : 0.0;
    }
    return bound / thr;
}

/* The list of tile `tile`: every valid Gaussian whose rect holds the tile, in depth
 * order.  cullq[k] = cull ratio of the k-th entry (+inf when tile_dmax is NULL or the
 * tile is not fully covered).  Returns the list length (entries written up to cap). */
int oc_tile_list(const oc_camera* cam, const float* rec, const int* rect, const int* order,
                 int norder, const float* tile_dmax, double softness, int tile,
                 int* out, double* cullq, int cap)
{
    int TX = tiles_x(cam);
    int tx = tile % TX, ty = tile / TX;
    int n = 0;
    for (int k = 0; k < norder; ++k) {
        int i = order[k];
        const int* rc = rect + (size_t)i * 4;
        if (tx < rc[0] || tx >= rc[2] || ty < rc[1] || ty >= rc[3]) continue;
        if (n < cap) {
            out[n] = i;
            if (cullq)
                cullq[n] = tile_dmax ? cull_ratio(cam, rec + (size_t)i * OC_NREC, tile_dmax[tile], tile, softness)
                                     : INFINITY;
        }
        ++n;
    }
    return n;
}

/* All lists of the requested tiles at once (OpenMP over tiles).  counts[k] must be
 * computed first with oc_tile_counts; offsets[k] are the caller's prefix sums. */
void oc_tile_counts(const oc_camera* cam, const int* rect, const int* order, int norder,
                    int ntiles, const int* tiles, int* counts)
{
    int TX = tiles_x(cam);
#pragma omp parallel for schedule(dynamic, 4)
    for (int k = 0; k < ntiles; ++k) {
        int tx = tiles[k] % TX, ty = tiles[k] / TX, n = 0;
        for (int j = 0; j < norder; ++j) {
            const int* rc = rect + (size_t)order[j] * 4;
            if (tx >= rc[0] && tx < rc[2] && ty >= rc[1] && ty < rc[3]) ++n;
        }
        counts[k] = n;
    }
}

void oc_tile_lists(const oc_camera* cam, const float* rec, const int* rect, const int* order,
                   int norder, const float* tile_dmax, double softness, int ntiles, const int* tiles,
                   const long long* offsets, int* ids, double* cullq)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int k = 0; k < ntiles; ++k) {
        long long o = offsets[k];
        int cap = (int)(offsets[k + 1] - o);
        oc_tile_list(cam, rec, rect, order, norder, tile_dmax, softness, tiles[k], ids + o,
                     cullq ? cullq + o : NULL, cap);
    }
}

/* ------------------------------------------------------------------------- */
/* Mesh surface: perspective-correct barycentrics, base colour, Phong, trilinear  */
/* texture (README, Design Details > Mesh rasterizer step 2; v1.1 notes: texture   */
/* with per-corner coordinates, trilinear mipmapping by default, Phong with         */
/* interpolated vertex normals and the specular highlight following the camera;    */
/* Limitations: coordinates outside [0, 1] are clamped, isotropic filtering).      */
/* ------------------------------------------------------------------------- */

/* Box-filter pyramid of a square power-of-two texture [S][S][3]: level l+1 texel is
 * the mean of the 2x2 block of level l.  mips holds the levels back to back (fp64). */
void oc_build_mips(const float* tex, int S, double* mips)
{
    size_t n0 = (size_t)S * S * 3;
    for (size_t i = 0; i < n0; ++i) mips[i] = tex[i];
    double* prev = mips;
    int s = S;
    while (s > 1) {
        int h = s / 2;
        double* cur = prev + (size_t)s * s * 3;
        for (int y = 0; y < h; ++y)
            for (int x = 0; x < h; ++x)
                for (int c = 0; c < 3; ++c) {
                    double a = prev[((size_t)(2 * y) * s + 2 * x) * 3 + c];
                    double b = prev[((size_t)(2 * y) * s + 2 * x + 1) * 3 + c];
                    double d = prev[((size_t)(2 * y + 1) * s + 2 * x) * 3 + c];
                    double e = prev[((size_t)(2 * y + 1) * s + 2 * x + 1) * 3 + c];
                    cur[((size_t)y * h + x) * 3 + c] = 0.25 * (a + b + d + e);
                }
        prev = cur;
        s = h;
    }
}

static void bilinear(const double* lvl, int s, double u, double v, double* out)
{
    u = u < 0 ? 0 : (u > 1 ? 1 : u);
    v = v < 0 ? 0 : (v > 1 ? 1 : v);
    double x = u * s - 0.5, y = v * s - 0.5;
    double x0 = floor(x), y0 = floor(y);
    double ax = x - x0, ay = y - y0;
    int ix0 = (int)x0, iy0 = (int)y0;
    int ix1 = ix0 + 1, iy1 = iy0 + 1;
    ix0 = ix0 < 0 ? 0 : (ix0 > s - 1 ? s - 1 : ix0);
    ix1 = ix1 < 0 ? 0 : (ix1 > s - 1 ? s - 1 : ix1);
    iy0 = iy0 < 0 ? 0 : (iy0 > s - 1 ? s - 1 : iy0);
    iy1 = iy1 < 0 ? 0 : (iy1 > s - 1 ? s - 1 : iy1);
    for (int c = 0; c < 3; ++c) {
        double t00 = lvl[((size_t)iy0 * s + ix0) * 3 + c], t01 = lvl[((size_t)iy0 * s + ix1) * 3 + c];
        double t10 = lvl[((size_t)iy1 * s + ix0) * 3 + c], t11 = lvl[((size_t)iy1 * s + ix1) * 3 + c];
        double top = t00 + (t01 - t00) * ax, bot = t10 + (t11 - t10) * ax;
        out[c] = top + (bot - top) * ay;
    }
}

typedef struct {
    const oc_camera* cam;
    int V, F;
    const float* vscreen; /* [3][V] */
    const int* faces;     /* [3][F] */
    const float* vcolor;  /* [3][V] or NULL */
    const float* vnormal; /* [3][V] or NULL (then unlit) */
    const float* verts;   /* [3][V] world (unused by shading) */
    const float* uv;      /* [2][Vt] or NULL */
    const int* faces_uv;  /* [3][F] */
    int Vt;
    const double* mips;   /* oc_build_mips output or NULL */
    int tex_size;
    const oc_light* light; /* NULL: unlit */
} oc_mesh;

/* Surface colour c_m at pixel (px, py) covered by face f; also returns the lod. */
static void shade(const oc_mesh* m, int f, int px, int py, double* cm, double* lod_out)
{
    const oc_camera* cam = m->cam;
    oc_tri t;
    tri_setup(cam, m->V, m->vscreen, m->faces, NULL, m->F, f, &t);
    double pu = px + 0.5, pv = py + 0.5, lam[3], z;
    if (!tri_cover(&t, pu, pv, lam, &z)) { /* caller guarantees coverage */
        lam[0] = lam[1] = lam[2] = 1.0 / 3.0;
        z = (t.z[0] + t.z[1] + t.z[2]) / 3.0;
    }
    double b[3];
    for (int k = 0; k < 3; ++k) b[k] = lam[k] / t.z[k] * z;
    double base[3] = {0, 0, 0};
    if (m->mips && m->uv) {
        double uvk[3][2];
        for (int k = 0; k < 3; ++k) {
            int ti = m->faces_uv[k * m->F + f];
            uvk[k][0] = m->uv[ti];
            uvk[k][1] = m->uv[m->Vt + ti];
        }
        double uu = 0, vv = 0;
        for (int k = 0; k < 3; ++k) { uu += b[k] * uvk[k][0]; vv += b[k] * uvk[k][1]; }
        /* analytic screen derivatives of the perspective-correct uv */
        double w[3], W = 0, dwx[3], dwy[3];
        /* dE_k/dpu = -(b.v - a.v), dE_k/dpv = (b.u - a.u), edges (1,2), (2,0), (0,1) */
        int ea[3] = {1, 2, 0}, eb[3] = {2, 0, 1};
        for (int k = 0; k < 3; ++k) {
            w[k] = lam[k] / t.z[k];
            W += w[k];
            dwx[k] = (-(t.v[eb[k]] - t.v[ea[k]]) / t.A) / t.z[k];
            dwy[k] = ((t.u[eb[k]] - t.u[ea[k]]) / t.A) / t.z[k];
        }
        double dux = 0, dvx = 0, duy = 0, dvy = 0;
        for (int k = 0; k < 3; ++k) {
            dux += dwx[k] * (uvk[k][0] - uu) / W;
            dvx += dwx[k] * (uvk[k][1] - vv) / W;
            duy += dwy[k] * (uvk[k][0] - uu) / W;
            dvy += dwy[k] * (uvk[k][1] - vv) / W;
        }
        double S0 = m->tex_size;
        double lx = sqrt((S0 * dux) * (S0 * dux) + (S0 * dvx) * (S0 * dvx));
        double ly = sqrt((S0 * duy) * (S0 * duy) + (S0 * dvy) * (S0 * dvy));
        double rho = lx > ly ? lx : ly;
        int nlev = 0;
        for (int s = m->tex_size; s >= 1; s >>= 1) ++nlev;
        double lmax = nlev - 1;
        double lod = rho > 0 ? log2(rho) : 0.0;
        lod = lod < 0 ? 0 : (lod > lmax ? lmax : lod);
        if (lod_out) *lod_out = lod;
        int l0 = (int)floor(lod);
        int l1 = l0 + 1 < (int)lmax ? l0 + 1 : (int)lmax;
        double tl = lod - l0;
        const double* lv = m->mips;
        const double *p0 = NULL, *p1 = NULL;
        int s = m->tex_size;
        for (int l = 0; l <= (int)lmax; ++l) {
            if (l == l0) p0 = lv;
            if (l == l1) p1 = lv;
            lv += (size_t)(s >> l) * (s >> l) * 3;
        }
        double c0[3], c1[3];
        bilinear(p0, s >> l0, uu, vv, c0);
        bilinear(p1, s >> l1, uu, vv, c1);
        for (int c = 0; c < 3; ++c) base[c] = c0[c] + (c1[c] - c0[c]) * tl;
    } else if (m->vcolor) {
        for (int c = 0; c < 3; ++c)
            for (int k = 0; k < 3; ++k) base[c] += b[k] * m->vcolor[c * m->V + m->faces[k * m->F + f]];
    }
    if (m->light && m->vnormal) {
        const float* R = cam->R;
        double nw[3] = {0, 0, 0};
        for (int c = 0; c < 3; ++c)
            for (int k = 0; k < 3; ++k) nw[c] += b[k] * m->vnormal[c * m->V + m->faces[k * m->F + f]];
        double n[3], L[3], x[3];
        for (int r = 0; r < 3; ++r) {
            n[r] = R[r * 3 + 0] * nw[0] + R[r * 3 + 1] * nw[1] + R[r * 3 + 2] * nw[2];
            L[r] = R[r * 3 + 0] * (double)m->light->pos[0] + R[r * 3 + 1] * (double)m->light->pos[1] +
                   R[r * 3 + 2] * (double)m->light->pos[2] + cam->t[r];
        }
        x[0] = (pu - cam->cx) / cam->fx * z;
        x[1] = (pv - cam->cy) / cam->fy * z;
        x[2] = z;
        double nn = sqrt(n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);
        double l[3] = {L[0] - x[0], L[1] - x[1], L[2] - x[2]};
        double ln = sqrt(l[0] * l[0] + l[1] * l[1] + l[2] * l[2]);
        double e[3] = {-x[0], -x[1], -x[2]};
        double en = sqrt(e[0] * e[0] + e[1] * e[1] + e[2] * e[2]);
        for (int r = 0; r < 3; ++r) { n[r] /= nn; l[r] /= ln; e[r] /= en; }
        double ndl = n[0] * l[0] + n[1] * l[1] + n[2] * l[2];
        double rv[3];
        for (int r = 0; r < 3; ++r) rv[r] = 2.0 * ndl * n[r] - l[r];
        double rde = rv[0] * e[0] + rv[1] * e[1] + rv[2] * e[2];
        double diff = ndl > 0 ? ndl : 0.0;
        double spec = (ndl > 0 && rde > 0) ? pow(rde, (double)m->light->shininess) : 0.0;
        for (int c = 0; c < 3; ++c)
            cm[c] = base[c] * ((double)m->light->ambient[c] + (double)m->light->diffuse[c] * diff) +
                    (double)m->light->specular[c] * spec;
    } else {
        for (int c = 0; c < 3; ++c) cm[c] = base[c];
    }
}

void oc_shade_pixels(const oc_mesh* m, int npix, const int* pix, const int* face_id, double* cm,
                     double* lod)
{
#pragma omp parallel for schedule(static)
    for (int k = 0; k < npix; ++k) {
        int p = pix[k], f = face_id[k];
        double c[3] = {0, 0, 0}, l = 0;
        if (f >= 0) shade(m, f, p % m->cam->width, p / m->cam->width, c, &l);
        cm[k * 3 + 0] = c[0]; cm[k * 3 + 1] = c[1]; cm[k * 3 + 2] = c[2];
        if (lod) lod[k] = l;
    }
}

/* ------------------------------------------------------------------------- */
/* Hybrid compositing, forward and reverse mode (README, Design Details > Hybrid    */
/* rendering: f = Phi((D - z*(p)) / (sigma softness)); front parts alpha f and back */
/* parts alpha (1 - f) composited into two layers in sorted order; C = C_front +    */
/* T_front (a_m c_m + (1 - a_m)(C_back + T_back bg)); differentiable w.r.t. the      */
/* Gaussians also through the split, and the mesh depth and colour).                */
/* Layer rules (3DGS): alpha = min(0.99, o exp(-q)); an entry with alpha_L < 1/255   */
/* is skipped; a layer stops before an entry that would bring T below 1e-4.          */
/* ------------------------------------------------------------------------- */

typedef struct {
    /* inputs */
    const oc_camera* cam;
    const oc_mesh* mesh;        /* for c_m; may have no colour source (then c_m = 0) */
    int N;
    const double* rec;          /* [N][13] fp64 copy of the records */
    int ntiles;
    const int* tiles;           /* requested tile ids */
    const long long* offsets;   /* [ntiles+1] into ids */
    const int* ids;             /* per-tile lists, depth order */
    const int* face_id;         /* [H][W] */
    const double* depth;        /* [H][W]: the fp32 depth buffer, upcast */
    double bg[3];
    double softness;
    const float* g_rgb;         /* [H][W][3] or NULL (then no backward) */
    const float* g_depth;       /* [H][W] or NULL */
    const float* g_alpha;       /* [H][W] or NULL */
    /* outputs, full-image arrays (only requested tiles written) */
    double* rgb;                /* [H][W][3] reduced (one-layer) form */
    double* out_depth;          /* [H][W] */
    double* alpha;              /* [H][W] */
    double* rgb2;               /* [H][W][3] general two-layer form (may be NULL) */
    double* depth2;
    double* alpha2;
    double* T_final;            /* [H][W] */
    int* n_last;                /* [H][W] index + 1 of the last included entry in the tile list */
    int* n_incl;                /* [H][W] number of included entries */
    double* margin;             /* [H][W] min relative distance of a skip/stop decision to its threshold */
    double* clamp_margin;       /* [H][W] min relative distance of o exp(-q) to 0.99 (included entries) */
    double* grad;               /* [N][13] accumulated (atomic) */
    double* g_mesh_rgb;         /* [H][W][3] */
    double* g_mesh_depth;       /* [H][W] */
    long long* pairs_evaluated; /* scalar */
    /* antialiased mesh layer (NULL: binary coverage from face_id / depth / mesh) */
    const double* layer;        /* [H][W][6]: M_rgb, M_D (premultiplied), a_m, D_split */
    double* g_layer;            /* [H][W][6] dL/d(layer) (written when g_rgb is given) */
    double* T_back;             /* [H][W] back-layer transmittance (may be NULL) */
    int* n_last_back;           /* [H][W] index + 1 of the back layer's last included entry */
} oc_comp;

typedef struct {
    int idx;
    double T, aF, alpha, ao, G, f, s, dx, dy;
} oc_entry;

static void eval_pair(const double* r, double px, double py, int on_mesh, double D, double softness,
                      double* alpha, double* ao, double* G, double* f, double* s, double* dx, double* dy)
{
    double ddx = px - r[0], ddy = py - r[1];
    double q = 0.5 * (r[2] * ddx * ddx + 2.0 * r[3] * ddx * ddy + r[4] * ddy * ddy);
    double g = exp(-q);
    double a0 = r[5] * g;
    *G = g;
    *ao = a0;
    *alpha = a0 < 0.99 ? a0 : 0.99;
    *dx = ddx;
    *dy = ddy;
    *s = 0.0;
    if (!on_mesh) {
        *f = 1.0;
        return;
    }
    double num = (D - r[9]) - (r[10] * ddx + r[11] * ddy);
    if (softness > 0.0) {
        *s = num / (r[12] * softness);
        *f = Phi(*s);
    } else {
        *f = num > 0.0 ? 1.0 : 0.0;
    }
}

static double reld(double x, double thr) { return fabs(x - thr) / thr; }

/* One pixel with an antialiased mesh layer: the general two-layer form
 * C = C_F + T_F (M + (1 - a_m)(C_B + T_B bg)), alpha = 1 - T_F (1 - a_m) T_B,
 * depth = Z_F + T_F (M_D + (1 - a_m) Z_B), with M, M_D the premultiplied mesh colour
 * and depth.  Both layers follow the 3DGS rules on their own (skip below 1/255,
 * stop before T < 1e-4), and the pixel stops when its front layer stops: the back
 * layer is seen only through T_front, and the 3DGS stop is per pixel (nothing after
 * it counts), so neither layer takes that entry or any later one.  The back layer
 * is composited only where it is visible (a_m < 1 and a finite split depth);
 * elsewhere it is empty (C_B = 0, Z_B = 0, T_B = 1).  The reverse mode is exact for both layers: the back layer sees the
 * upstream gradients scaled by k = T_F (1 - a_m), with behind it bg (depth 0) and
 * the alpha term; per entry dL/dalpha = f dL/dalpha_F + (1 - f) dL/dalpha_B and
 * dL/df = alpha (dL/dalpha_F - dL/dalpha_B). */
static void composite_pixel_aa(const oc_comp* a, int p, double pu, double pv, long long o0, int n,
                               oc_entry* entF, oc_entry* entB, double* daFj, double* daBj,
                               long long* pairs_total)
{
    const double thr_skip = 1.0 / 255.0, thr_stop = 1e-4;
    const double* L = a->layer + 6 * (size_t)p;
    double Mc[3] = {L[0], L[1], L[2]}, MD = L[3], am = L[4], D = L[5];
    int on = isfinite(D);
    double TF = 1.0, TB = 1.0, CF[3] = {0, 0, 0}, CB[3] = {0, 0, 0}, ZF = 0, ZB = 0;
    int aliveF = 1, aliveB = on && am < 1.0, lastF = 0, lastB = 0, nF = 0, nB = 0;
    double mg = INFINITY, cmg = INFINITY;
    for (int j = 0; j < n && (aliveF || aliveB); ++j) {
        const double* r = a->rec + (size_t)a->ids[o0 + j] * OC_NREC;
        double al, ao, G, f, s, dx, dy;
        eval_pair(r, pu, pv, on, D, a->softness, &al, &ao, &G, &f, &s, &dx, &dy);
        ++*pairs_total;
        for (int layer = 0; layer < 2; ++layer) {
            int* alive = layer == 0 ? &aliveF : &aliveB;
            if (!*alive) continue;
            double aL = layer == 0 ? al * f : al * (1.0 - f);
            double* T = layer == 0 ? &TF : &TB;
            double m1 = reld(aL, thr_skip);
            if (m1 < mg) mg = m1;
            if (!(aL >= thr_skip)) continue;
            double Tn = *T * (1.0 - aL);
            double m2 = reld(Tn, thr_stop);
            if (m2 < mg) mg = m2;
            if (Tn < thr_stop) {
                *alive = 0;
                if (layer == 0) aliveB = 0; /* the pixel stops with its front layer */
                continue;
            }
            double w = aL * *T;
            oc_entry* e = layer == 0 ? &entF[nF++] : &entB[nB++];
            e->idx = j; e->T = *T; e->aF = aL; e->alpha = al; e->ao = ao; e->G = G; e->f = f; e->s = s;
            e->dx = dx; e->dy = dy;
            double m3 = reld(ao, 0.99);
            if (m3 < cmg) cmg = m3;
            double* Cc = layer == 0 ? CF : CB;
            for (int c = 0; c < 3; ++c) Cc[c] += w * r[6 + c];
            if (layer == 0) ZF += w * r[9]; else ZB += w * r[9];
            *T = Tn;
            if (layer == 0) lastF = j + 1; else lastB = j + 1;
        }
    }
    double Y[3];
    for (int c = 0; c < 3; ++c) {
        Y[c] = CB[c] + TB * a->bg[c];
        double v = CF[c] + TF * (Mc[c] + (1.0 - am) * Y[c]);
        a->rgb[p * 3 + c] = v;
        if (a->rgb2) a->rgb2[p * 3 + c] = v;
    }
    a->alpha[p] = 1.0 - TF * (1.0 - am) * TB;
    a->out_depth[p] = ZF + TF * (MD + (1.0 - am) * ZB);
    if (a->alpha2) a->alpha2[p] = a->alpha[p];
    if (a->depth2) a->depth2[p] = a->out_depth[p];
    a->T_final[p] = TF;
    a->n_last[p] = lastF;
    if (a->T_back) a->T_back[p] = TB;
    if (a->n_last_back) a->n_last_back[p] = lastB;
    if (a->n_incl) a->n_incl[p] = nF;
    if (a->margin) a->margin[p] = mg;
    if (a->clamp_margin) a->clamp_margin[p] = cmg;
    if (!a->g_rgb) return;

    /* ---- reverse mode ---- */
    double GC[3] = {a->g_rgb[p * 3 + 0], a->g_rgb[p * 3 + 1], a->g_rgb[p * 3 + 2]};
    double GZ = a->g_depth ? a->g_depth[p] : 0.0;
    double GA = a->g_alpha ? a->g_alpha[p] : 0.0;
    double k = TF * (1.0 - am);
    /* dL/dT_F: everything behind the front layer */
    double BF = GZ * (MD + (1.0 - am) * ZB) - GA * (1.0 - am) * TB;
    for (int c = 0; c < 3; ++c) BF += GC[c] * (Mc[c] + (1.0 - am) * Y[c]);
    /* dL/dT_B, scaled: the background behind the back layer */
    double BB = -GA * k;
    for (int c = 0; c < 3; ++c) BB += GC[c] * k * a->bg[c];
    for (int j = 0; j < n; ++j) daFj[j] = daBj[j] = 0.0;
    double acc = TF * BF;
    for (int e = nF - 1; e >= 0; --e) {
        const oc_entry* en = &entF[e];
        const double* r = a->rec + (size_t)a->ids[o0 + en->idx] * OC_NREC;
        double Vv = GC[0] * r[6] + GC[1] * r[7] + GC[2] * r[8] + GZ * r[9];
        daFj[en->idx] = en->T * Vv - acc / (1.0 - en->aF);
        acc += en->aF * en->T * Vv;
    }
    acc = TB * BB;
    for (int e = nB - 1; e >= 0; --e) {
        const oc_entry* en = &entB[e];
        const double* r = a->rec + (size_t)a->ids[o0 + en->idx] * OC_NREC;
        double Vv = k * (GC[0] * r[6] + GC[1] * r[7] + GC[2] * r[8] + GZ * r[9]);
        daBj[en->idx] = en->T * Vv - acc / (1.0 - en->aF);
        acc += en->aF * en->T * Vv;
    }
    double gD = 0.0;
    int iF = 0, iB = 0;
    for (int j = 0; j < n; ++j) {
        const oc_entry* eF = (iF < nF && entF[iF].idx == j) ? &entF[iF++] : NULL;
        const oc_entry* eB = (iB < nB && entB[iB].idx == j) ? &entB[iB++] : NULL;
        if (!eF && !eB) continue;
        const oc_entry* en = eF ? eF : eB; /* alpha, G, f, s, dx, dy are the same in both */
        int id = a->ids[o0 + j];
        const double* r = a->rec + (size_t)id * OC_NREC;
        double wF = eF ? eF->aF * eF->T : 0.0, wB = eB ? eB->aF * eB->T : 0.0;
        double gr[OC_NREC];
        memset(gr, 0, sizeof(gr));
        for (int c = 0; c < 3; ++c) gr[6 + c] = (wF + k * wB) * GC[c];
        gr[9] = (wF + k * wB) * GZ;
        double daF = daFj[j], daB = daBj[j];
        double da = en->f * daF + (1.0 - en->f) * daB;
        if (en->ao <= 0.99) {
            gr[5] = en->G * da;
            double Hh = r[5] * en->G * da;
            gr[2] = -0.5 * en->dx * en->dx * Hh;
            gr[3] = -en->dx * en->dy * Hh;
            gr[4] = -0.5 * en->dy * en->dy * Hh;
            gr[0] = Hh * (r[2] * en->dx + r[3] * en->dy);
            gr[1] = Hh * (r[3] * en->dx + r[4] * en->dy);
        }
        if (on && a->softness > 0.0) {
            double ds = en->alpha * phi(en->s) * (daF - daB);
            double kap = 1.0 / (r[12] * a->softness);
            gr[9] -= kap * ds;
            gr[10] -= kap * ds * en->dx;
            gr[11] -= kap * ds * en->dy;
            gr[0] += kap * ds * r[10];
            gr[1] += kap * ds * r[11];
            gr[12] -= ds * en->s / r[12];
            gD += kap * ds;
        }
        double* dst = a->grad + (size_t)id * OC_NREC;
        for (int c = 0; c < OC_NREC; ++c) {
#pragma omp atomic
            dst[c] += gr[c];
        }
    }
    double* gl = a->g_layer + 6 * (size_t)p;
    for (int c = 0; c < 3; ++c) gl[c] = TF * GC[c];
    gl[3] = TF * GZ;
    gl[4] = TF * (GA * TB - (GC[0] * Y[0] + GC[1] * Y[1] + GC[2] * Y[2]) - GZ * ZB);
    gl[5] = gD;
}

void oc_composite(oc_comp* a)
{
    const oc_camera* cam = a->cam;
    int W = cam->width, H = cam->height, TX = tiles_x(cam);
    const double thr_skip = 1.0 / 255.0, thr_stop = 1e-4;
    long long pairs_total = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : pairs_total)
    for (int k = 0; k < a->ntiles; ++k) {
        int tile = a->tiles[k];
        int tx = tile % TX, ty = tile / TX;
        long long o0 = a->offsets[k], o1 = a->offsets[k + 1];
        int n = (int)(o1 - o0);
        oc_entry* ent = (oc_entry*)malloc(sizeof(oc_entry) * (size_t)(n > 0 ? n : 1));
        oc_entry* entB = NULL;
        double *daF = NULL, *daB = NULL;
        if (a->layer) {
            entB = (oc_entry*)malloc(sizeof(oc_entry) * (size_t)(n > 0 ? n : 1));
            daF = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            daB = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        }
        for (int py = ty * OC_TILE; py < ty * OC_TILE + OC_TILE && py < H; ++py)
            for (int px = tx * OC_TILE; px < tx * OC_TILE + OC_TILE && px < W; ++px) {
                int p = py * W + px;
                double pu = px + 0.5, pv = py + 0.5;
                if (a->layer) {
                    composite_pixel_aa(a, p, pu, pv, o0, n, ent, entB, daF, daB, &pairs_total);
                    continue;
                }
                int fid = a->face_id[p];
                int on = fid >= 0;
                double am = on ? 1.0 : 0.0;
                double D = on ? a->depth[p] : INFINITY;
                double cm[3] = {0, 0, 0};
                if (on && a->mesh) shade(a->mesh, fid, px, py, cm, NULL);

                /* ---- forward, both layers ---- */
                double TF = 1.0, TB = 1.0, CF[3] = {0, 0, 0}, CB[3] = {0, 0, 0}, ZF = 0, ZB = 0;
                int aliveF = 1, aliveB = 1, last = 0, nin = 0;
                double mg = INFINITY, cmg = INFINITY;
                for (int j = 0; j < n && (aliveF || aliveB); ++j) {
                    const double* r = a->rec + (size_t)a->ids[o0 + j] * OC_NREC;
                    double al, ao, G, f, s, dx, dy;
                    eval_pair(r, pu, pv, on, D, a->softness, &al, &ao, &G, &f, &s, &dx, &dy);
                    ++pairs_total;
                    if (aliveF) {
                        double aF = al * f;
                        double m1 = reld(aF, thr_skip);
                        if (m1 < mg) mg = m1;
                        if (aF >= thr_skip) {
                            double Tn = TF * (1.0 - aF);
                            double m2 = reld(Tn, thr_stop);
                            if (m2 < mg) mg = m2;
                            if (Tn < thr_stop) {
                                aliveF = 0;
                            } else {
                                double w = aF * TF;
                                ent[nin].idx = j; ent[nin].T = TF; ent[nin].aF = aF; ent[nin].alpha = al;
                                ent[nin].ao = ao; ent[nin].G = G; ent[nin].f = f; ent[nin].s = s;
                                ent[nin].dx = dx; ent[nin].dy = dy;
                                ++nin;
                                double m3 = reld(ao, 0.99);
                                if (m3 < cmg) cmg = m3;
                                for (int c = 0; c < 3; ++c) CF[c] += w * r[6 + c];
                                ZF += w * r[9];
                                TF = Tn;
                                last = j + 1;
                            }
                        }
                    }
                    if (aliveB) {
                        double aB = al * (1.0 - f);
                        if (aB >= thr_skip) {
                            double Tn = TB * (1.0 - aB);
                            if (Tn < thr_stop) {
                                aliveB = 0;
                            } else {
                                double w = aB * TB;
                                for (int c = 0; c < 3; ++c) CB[c] += w * r[6 + c];
                                ZB += w * r[9];
                                TB = Tn;
                            }
                        }
                    }
                }
                for (int c = 0; c < 3; ++c) {
                    a->rgb[p * 3 + c] = CF[c] + TF * (am * cm[c] + (1.0 - am) * a->bg[c]);
                    if (a->rgb2)
                        a->rgb2[p * 3 + c] = CF[c] + TF * (am * cm[c] + (1.0 - am) * (CB[c] + TB * a->bg[c]));
                }
                a->alpha[p] = 1.0 - TF * (1.0 - am);
                a->out_depth[p] = ZF + TF * am * (on ? D : 0.0);
                if (a->alpha2) a->alpha2[p] = 1.0 - TF * (1.0 - am) * TB;
                if (a->depth2) {
                    double Dm = on ? D : 0.0; /* background depth is 0 */
                    a->depth2[p] = ZF + TF * (am * Dm + (1.0 - am) * ZB);
                }
                a->T_final[p] = TF;
                a->n_last[p] = last;
                if (a->n_incl) a->n_incl[p] = nin;
                if (a->margin) a->margin[p] = mg;
                if (a->clamp_margin) a->clamp_margin[p] = cmg;

                /* ---- reverse mode of the one-layer form (exact, stored T) ---- */
                if (!a->g_rgb) continue;
                double GC[3] = {a->g_rgb[p * 3 + 0], a->g_rgb[p * 3 + 1], a->g_rgb[p * 3 + 2]};
                double GZ = a->g_depth ? a->g_depth[p] : 0.0;
                double GA = a->g_alpha ? a->g_alpha[p] : 0.0;
                double B = GZ * am * (on ? D : 0.0) - GA * (1.0 - am);
                for (int c = 0; c < 3; ++c) B += GC[c] * (am * cm[c] + (1.0 - am) * a->bg[c]);
                double acc = TF * B;
                double gD = 0.0;
                for (int e = nin - 1; e >= 0; --e) {
                    const oc_entry* en = &ent[e];
                    int id = a->ids[o0 + en->idx];
                    const double* r = a->rec + (size_t)id * OC_NREC;
                    double w = en->aF * en->T;
                    double Vv = GC[0] * r[6] + GC[1] * r[7] + GC[2] * r[8] + GZ * r[9];
                    double daF = en->T * Vv - acc / (1.0 - en->aF);
                    acc += w * Vv;
                    double gr[OC_NREC];
                    memset(gr, 0, sizeof(gr));
                    for (int c = 0; c < 3; ++c) gr[6 + c] = w * GC[c];
                    gr[9] = w * GZ;
                    double da = en->f * daF;
                    if (en->ao <= 0.99) {
                        gr[5] = en->G * da;
                        double Hh = r[5] * en->G * da;
                        gr[2] = -0.5 * en->dx * en->dx * Hh;
                        gr[3] = -en->dx * en->dy * Hh;
                        gr[4] = -0.5 * en->dy * en->dy * Hh;
                        gr[0] = Hh * (r[2] * en->dx + r[3] * en->dy);
                        gr[1] = Hh * (r[3] * en->dx + r[4] * en->dy);
                    }
                    if (on && a->softness > 0.0) {
                        double ds = en->alpha * phi(en->s) * daF;
                        double kap = 1.0 / (r[12] * a->softness);
                        gr[9] -= kap * ds;
                        gr[10] -= kap * ds * en->dx;
                        gr[11] -= kap * ds * en->dy;
                        gr[0] += kap * ds * r[10];
                        gr[1] += kap * ds * r[11];
                        gr[12] -= ds * en->s / r[12];
                        gD += kap * ds;
                    }
                    double* dst = a->grad + (size_t)id * OC_NREC;
                    for (int c = 0; c < OC_NREC; ++c) {
#pragma omp atomic
                        dst[c] += gr[c];
                    }
                }
                for (int c = 0; c < 3; ++c) a->g_mesh_rgb[p * 3 + c] = TF * am * GC[c];
                a->g_mesh_depth[p] = TF * am * GZ + gD;
            }
        free(ent);
        free(entB);
        free(daF);
        free(daB);
    }
    if (a->pairs_evaluated) *a->pairs_evaluated = pairs_total;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the OpenMP loops of this library use. */
int oc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Erf-based normal CDF, exported so that tests can pin it against closed values. */
double oc_Phi(double s) { return Phi(s); }
