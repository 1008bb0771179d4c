/*
 * CPU oracle of the analytic edge antialiasing of the mesh and of its reverse mode.
 *
 * TEST INFRASTRUCTURE ONLY (see gm_oracle.c): loaded by the test suite, the package
 * smoke check and the benchmark's CPU-baseline leg; it shares no code with the HIP
 * library.
 *
 * What is computed (gmesh README, "Design Details > Mesh rasterizer", step 3, and
 * "Limitations and Todos": edges are antialiased analytically as in nvdiffrast; for
 * every pair of neighbouring pixels that sees a silhouette, the point where the front
 * triangle's edge crosses between the two pixel centres gives a fractional coverage
 * and blends the colour over the farther surface; internal edges of a connected
 * surface are left alone; the approximation is per axis and one-dimensional, exact
 * for straight edges away from corners; "Hybrid rendering": with antialiasing the
 * mesh coverage a_m is fractional at silhouettes).
 *
 * Readings (the pages give no more than the above):
 *  - Pairs are the horizontally and the vertically adjacent pixel pairs of the image
 *    whose z-buffer faces differ.  The front pixel is the covered one, or, when both
 *    are covered, the one with the smaller depth-buffer value (equal values: the
 *    smaller face id).
 *  - The segment from the front pixel's centre a to the other centre b is followed
 *    over the front surface: it leaves a triangle through the edge whose
 *    (inside-positive) edge function falls to zero first, at t = e(a) / (e(a) - e(b))
 *    (over the edges with e(b) < e(a); equal t: the lower edge index).  If that
 *    edge is internal, the segment continues in the neighbouring face from there;
 *    the first silhouette edge it leaves through gives the crossing t in [0, 1).
 *    It stops with no effect when a triangle holds the rest of the segment (t >= 1:
 *    the other centre is on the same connected surface) or after 16 triangles.
 *    (Near an outline the triangle seen at a is often not the one that carries the
 *    outline: thin, foreshortened triangles between it and the outline cover no
 *    pixel centre.)
 *  - An edge is a silhouette edge in this view when no other face shares its two
 *    vertex indices, more than one does, the one that does is not drawn in this
 *    view (masked, behind the near plane, zero area), or that face faces the other
 *    way (opposite sign of the screen-space area).  Otherwise it is an internal edge
 *    of a connected surface.
 *  - Per axis: a horizontal pair takes edges at least as steep as 45 degrees
 *    (|dv| >= |du|), a vertical pair the others, so every edge is handled along one
 *    axis only.
 *  - One-dimensional box filter along the pair's axis: the front surface covers
 *    the segment up to the crossing.  With d = t - 1/2: d < 0 moves the fraction -d
 *    of the front pixel to the other pixel's surface; d > 0 gives the other pixel
 *    the fraction d of the front pixel's surface; d = 0 changes nothing.  "The
 *    surface" of a pixel is its z-buffer colour c and depth D at its centre; an
 *    uncovered pixel contributes nothing (coverage goes to whatever lies behind the
 *    mesh).
 *  - The effects of all pairs add up as per-pixel weights: w_self (1 on a covered
 *    pixel, 0 elsewhere, then changed) and w_d for the four neighbours d (left,
 *    right, up, down).  Raw coverage a = w_self + sum_d w_d; premultiplied mesh
 *    colour M = w_self c(x) + sum_d w_d c(n_d) and depth M_D likewise with D.
 *  - Where silhouettes meet in one pixel the sum can leave [0, 1]; the coverage used
 *    is clamped to [0, 1] and M, M_D are scaled by (clamped / raw) (0 when raw <= 0),
 *    which keeps the mesh colour M / a.
 *  - The depth that splits the Gaussians at a pixel: its own D when covered; on an
 *    uncovered pixel that receives coverage, the smallest D of the neighbours that
 *    give it coverage; +inf otherwise.
 *
 * Precision: the crossing and the decisions are fp64 from the (upcast) fp32 screen
 * vertices, as in the raster; weights and sums fp64.
 *
 * Layout: the layer output is [H][W][6] = (M_r, M_g, M_b, M_D, a, D_split).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int width, height;
    float fx, fy, cx, cy;
    float R[9], t[3];
    float near_z;
} aa_camera; /* the same layout as the oracle's camera */

/* ------------------------------------------------------------------------- */
/* Edge adjacency: for edge k of face f (the edge opposite corner k, from corner   */
/* k+1 to corner k+2), the one other face with the same two vertex indices, -1 if  */
/* none, -2 if more than one.  View independent.                                   */
/* ------------------------------------------------------------------------- */
typedef struct {
    int lo, hi, face, k;
} aa_edge;

static int edge_cmp(const void* x, const void* y)
{
    const aa_edge* a = (const aa_edge*)x;
    const aa_edge* b = (const aa_edge*)y;
    if (a->lo != b->lo) return a->lo < b->lo ? -1 : 1;
    if (a->hi != b->hi) return a->hi < b->hi ? -1 : 1;
    if (a->face != b->face) return a->face < b->face ? -1 : 1;
    return a->k < b->k ? -1 : (a->k > b->k);
}

void oc_edge_adjacency(int F, const int* faces, int* adj)
{
    aa_edge* e = (aa_edge*)malloc(sizeof(aa_edge) * (size_t)(3 * F > 0 ? 3 * F : 1));
    for (int f = 0; f < F; ++f)
        for (int k = 0; k < 3; ++k) {
            int a = faces[((k + 1) % 3) * F + f], b = faces[((k + 2) % 3) * F + f];
            aa_edge* x = &e[3 * f + k];
            x->lo = a < b ? a : b;
            x->hi = a < b ? b : a;
            x->face = f;
            x->k = k;
        }
    qsort(e, (size_t)(3 * F), sizeof(aa_edge), edge_cmp);
    for (int i = 0; i < 3 * F;) {
        int j = i;
        while (j < 3 * F && e[j].lo == e[i].lo && e[j].hi == e[i].hi) ++j;
        int n = j - i; /* face-edges sharing this vertex pair */
        for (int m = i; m < j; ++m) {
            int other = -1;
            if (n == 2) other = e[m == i ? i + 1 : i].face;
            else if (n > 2) other = -2;
            adj[e[m].k * F + e[m].face] = other;
        }
        i = j;
    }
    free(e);
}

/* ------------------------------------------------------------------------- */
/* Pair analysis                                                               */
/* ------------------------------------------------------------------------- */
typedef struct {
    const aa_camera* cam;
    int V, F;
    const double* vs;          /* [3][V] screen u, v, z (upcast fp32, or perturbed) */
    const int* faces;          /* [3][F] */
    const unsigned char* mask; /* [F] or NULL */
    const int* adj;            /* [3][F] */
    const int* face_id;        /* [H][W] */
    const float* depth;        /* [H][W] */
} aa_in;

typedef struct {
    double u[3], v[3];
    double sgn; /* sign of the screen-space area */
    int valid;
} aa_tri;

static void tri_of(const aa_in* in, int f, aa_tri* t)
{
    t->valid = 0;
    if (in->mask && !in->mask[f]) return;
    for (int k = 0; k < 3; ++k) {
        int vi = in->faces[k * in->F + f];
        t->u[k] = in->vs[vi];
        t->v[k] = in->vs[in->V + vi];
        if (!(in->vs[2 * in->V + vi] >= (double)in->cam->near_z)) return;
    }
    double A = (t->u[1] - t->u[0]) * (t->v[2] - t->v[0]) - (t->v[1] - t->v[0]) * (t->u[2] - t->u[0]);
    if (A == 0.0) return;
    t->sgn = A > 0.0 ? 1.0 : -1.0;
    t->valid = 1;
}

/* inside-positive edge function of edge k (corner k+1 -> corner k+2) at (pu, pv) */
static double edge_fn(const aa_tri* t, int k, double pu, double pv)
{
    int i = (k + 1) % 3, j = (k + 2) % 3;
    return t->sgn * ((t->u[j] - t->u[i]) * (pv - t->v[i]) - (t->v[j] - t->v[i]) * (pu - t->u[i]));
}

#define AA_MAX_WALK 16 /* triangles followed from the front pixel's */

typedef struct {
    int a, b;      /* front pixel, other pixel */
    int face, k;   /* the face whose silhouette edge k is crossed */
    aa_tri tri;
    double ea, eb; /* edge function at the two centres */
    double t;      /* crossing, from a's centre (0) to b's (1) */
} aa_pair;

/* Pixel q is the right (axis 0) or the lower (axis 1) neighbour of p.  Returns 1
 * when the pair changes a coverage (t != 1/2), filling *r. */
static int analyse(const aa_in* in, int p, int q, int axis, aa_pair* r)
{
    int W = in->cam->width;
    int fp = in->face_id[p], fq = in->face_id[q];
    if (fp == fq) return 0;
    int a;
    if (fq < 0) a = p;
    else if (fp < 0) a = q;
    else if (in->depth[p] < in->depth[q]) a = p;
    else if (in->depth[q] < in->depth[p]) a = q;
    else a = fp < fq ? p : q;
    int b = a == p ? q : p;
    int F = in->face_id[a];
    aa_tri t;
    tri_of(in, F, &t);
    if (!t.valid) return 0; /* cannot happen for a z-buffer face */
    double au = (a % W) + 0.5, av = (a / W) + 0.5, bu = (b % W) + 0.5, bv = (b / W) + 0.5;
    int G = F, kx = -1;
    double tx = 0.0, eax = 0.0, ebx = 0.0;
    for (int step = 0; step < AA_MAX_WALK; ++step) {
        /* exit of the segment from triangle G */
        int ke = -1;
        double te = INFINITY, ea_e = 0.0, eb_e = 0.0;
        for (int k = 0; k < 3; ++k) {
            double ea = edge_fn(&t, k, au, av), eb = edge_fn(&t, k, bu, bv);
            if (!(eb < ea)) continue;
            double tk = ea / (ea - eb);
            if (tk < te) {
                te = tk;
                ke = k;
                ea_e = ea;
                eb_e = eb;
            }
        }
        if (ke < 0 || !(te < 1.0)) return 0; /* G holds the rest of the segment */
        int g = in->adj[ke * in->F + G];
        aa_tri tg;
        int internal = 0;
        if (g >= 0) {
            tri_of(in, g, &tg);
            internal = tg.valid && tg.sgn == t.sgn;
        }
        if (!internal) {
            kx = ke;
            tx = te;
            eax = ea_e;
            ebx = eb_e;
            break;
        }
        G = g;
        t = tg;
    }
    if (kx < 0) return 0;
    F = G;
    /* axis test */
    int i = (kx + 1) % 3, j = (kx + 2) % 3;
    double du = fabs(t.u[j] - t.u[i]), dv = fabs(t.v[j] - t.v[i]);
    if (axis == 0 ? !(dv >= du) : !(du > dv)) return 0;
    if (tx == 0.5) return 0;
    r->a = a;
    r->b = b;
    r->face = F;
    r->k = kx;
    r->tri = t;
    r->ea = eax;
    r->eb = ebx;
    r->t = tx;
    return 1;
}

/* direction index of neighbour n seen from x: 0 left, 1 right, 2 up, 3 down */
static int dir_of(int x, int n, int W)
{
    if (n == x - 1) return 0;
    if (n == x + 1) return 1;
    if (n == x - W) return 2;
    return 3;
}

static int neighbour(int x, int d, int W)
{
    return d == 0 ? x - 1 : d == 1 ? x + 1 : d == 2 ? x - W : x + W;
}

/* Per-pixel weights from every pair: wself [HW], wn [HW][4]. */
static void weights(const aa_in* in, double* wself, double* wn)
{
    int W = in->cam->width, H = in->cam->height;
    for (int x = 0; x < W * H; ++x) {
        wself[x] = in->face_id[x] >= 0 ? 1.0 : 0.0;
        for (int d = 0; d < 4; ++d) wn[4 * x + d] = 0.0;
    }
    for (int axis = 0; axis < 2; ++axis)
        for (int y = 0; y < H - axis; ++y)
            for (int x = 0; x < W - (1 - axis); ++x) {
                int p = y * W + x, q = axis == 0 ? p + 1 : p + W;
                aa_pair r;
                if (!analyse(in, p, q, axis, &r)) continue;
                int bcov = in->face_id[r.b] >= 0;
                if (r.t < 0.5) {
                    double lost = 0.5 - r.t;
                    wself[r.a] -= lost;
                    if (bcov) wn[4 * r.a + dir_of(r.a, r.b, W)] += lost;
                } else {
                    double gained = r.t - 0.5;
                    wn[4 * r.b + dir_of(r.b, r.a, W)] += gained;
                    if (bcov) wself[r.b] -= gained;
                }
            }
}

/* Forward: colour [H][W][3] = the z-buffer surface colour at covered pixels (other
 * entries unused).  layer [H][W][6]; raw [H][W][6] (w_self, w_left, w_right, w_up,
 * w_down, raw coverage) or NULL. */
void oc_antialias(const aa_camera* cam, int V, int F, const double* vs, const int* faces,
                  const unsigned char* mask, const int* adj, const int* face_id, const float* depth,
                  const double* colour, double* layer, double* raw)
{
    aa_in in = {cam, V, F, vs, faces, mask, adj, face_id, depth};
    int W = cam->width, H = cam->height, HW = W * H;
    double* wself = (double*)malloc(sizeof(double) * (size_t)(HW > 0 ? HW : 1));
    double* wn = (double*)malloc(sizeof(double) * 4 * (size_t)(HW > 0 ? HW : 1));
    weights(&in, wself, wn);
    for (int x = 0; x < HW; ++x) {
        int cov = face_id[x] >= 0;
        double a = wself[x], M[3] = {0, 0, 0}, MD = 0.0, Ds = cov ? (double)depth[x] : INFINITY;
        if (cov) {
            for (int c = 0; c < 3; ++c) M[c] = wself[x] * colour[3 * x + c];
            MD = wself[x] * (double)depth[x];
        }
        for (int d = 0; d < 4; ++d) {
            double w = wn[4 * x + d];
            if (w == 0.0) continue;
            int n = neighbour(x, d, W);
            a += w;
            for (int c = 0; c < 3; ++c) M[c] += w * colour[3 * n + c];
            MD += w * (double)depth[n];
            if (!cov && w > 0.0 && (double)depth[n] < Ds) Ds = (double)depth[n];
        }
        double s = a > 1.0 ? 1.0 / a : (a < 0.0 ? 0.0 : 1.0);
        double ac = a > 1.0 ? 1.0 : (a < 0.0 ? 0.0 : a);
        double* o = layer + 6 * (size_t)x;
        for (int c = 0; c < 3; ++c) o[c] = s * M[c];
        o[3] = s * MD;
        o[4] = ac;
        o[5] = Ds;
        if (raw) {
            raw[6 * (size_t)x] = wself[x];
            for (int d = 0; d < 4; ++d) raw[6 * (size_t)x + 1 + d] = wn[4 * x + d];
            raw[6 * (size_t)x + 5] = a;
        }
    }
    free(wself);
    free(wn);
}

/* Reverse mode.  g_layer [H][W][6] = dL/d(M_r, M_g, M_b, M_D, a, D_split) of the
 * clamped layer.  Outputs (accumulated, caller zeroes): g_colour [H][W][3] and
 * g_depth [H][W] (dL/dc and dL/dD at the covered pixels' own centres), g_vs [2][V]
 * (dL/du, dL/dv of the screen vertices through the crossings).  The decisions
 * (front pixel, crossed edge, silhouette, axis, sign of t - 1/2, the clamp branch,
 * the neighbour giving D_split) are not differentiated. */
void oc_antialias_bwd(const aa_camera* cam, int V, int F, const double* vs, const int* faces,
                      const unsigned char* mask, const int* adj, const int* face_id, const float* depth,
                      const double* colour, const double* g_layer, double* g_colour, double* g_depth,
                      double* g_vs)
{
    aa_in in = {cam, V, F, vs, faces, mask, adj, face_id, depth};
    int W = cam->width, H = cam->height, HW = W * H;
    size_t n1 = (size_t)(HW > 0 ? HW : 1);
    double* wself = (double*)malloc(sizeof(double) * n1);
    double* wn = (double*)malloc(sizeof(double) * 4 * n1);
    double* gws = (double*)calloc(n1, sizeof(double));    /* dL/dw_self */
    double* gwn = (double*)calloc(4 * n1, sizeof(double)); /* dL/dw_d */
    weights(&in, wself, wn);

    for (int x = 0; x < HW; ++x) {
        int cov = face_id[x] >= 0;
        const double* g = g_layer + 6 * (size_t)x;
        /* raw sums again */
        double a = wself[x], M[3] = {0, 0, 0}, MD = 0.0;
        if (cov) {
            for (int c = 0; c < 3; ++c) M[c] = wself[x] * colour[3 * x + c];
            MD = wself[x] * (double)depth[x];
        }
        int dsel = -1;
        double Ds = cov ? (double)depth[x] : INFINITY;
        for (int d = 0; d < 4; ++d) {
            double w = wn[4 * x + d];
            if (w == 0.0) continue;
            int n = neighbour(x, d, W);
            a += w;
            for (int c = 0; c < 3; ++c) M[c] += w * colour[3 * n + c];
            MD += w * (double)depth[n];
            if (!cov && w > 0.0 && (double)depth[n] < Ds) {
                Ds = (double)depth[n];
                dsel = d;
            }
        }
        /* clamp */
        double gMx[4] = {0, 0, 0, 0}, gax = 0.0;
        if (a > 1.0) {
            double s = 1.0 / a;
            for (int c = 0; c < 4; ++c) gMx[c] = s * g[c];
            gax = -s * s * (g[0] * M[0] + g[1] * M[1] + g[2] * M[2] + g[3] * MD);
        } else if (a >= 0.0) {
            for (int c = 0; c < 4; ++c) gMx[c] = g[c];
            gax = g[4];
        }
        /* colour and depth of the surfaces that make up M */
        if (cov) {
            for (int c = 0; c < 3; ++c) g_colour[3 * x + c] += wself[x] * gMx[c];
            g_depth[x] += wself[x] * gMx[3] + g[5]; /* own D also splits the Gaussians */
            gws[x] = gMx[0] * colour[3 * x] + gMx[1] * colour[3 * x + 1] + gMx[2] * colour[3 * x + 2] +
                     gMx[3] * (double)depth[x] + gax;
        }
        for (int d = 0; d < 4; ++d) {
            double w = wn[4 * x + d];
            int n = neighbour(x, d, W);
            if (w != 0.0) {
                for (int c = 0; c < 3; ++c) g_colour[3 * n + c] += w * gMx[c];
                g_depth[n] += w * gMx[3];
            }
            if (n >= 0 && n < HW && face_id[n] >= 0 && ((d < 2 && n / W == x / W) || d >= 2))
                gwn[4 * x + d] = gMx[0] * colour[3 * n] + gMx[1] * colour[3 * n + 1] +
                                 gMx[2] * colour[3 * n + 2] + gMx[3] * (double)depth[n] + gax;
        }
        if (dsel >= 0) g_depth[neighbour(x, dsel, W)] += g[5];
    }

    /* crossings */
    for (int axis = 0; axis < 2; ++axis)
        for (int y = 0; y < H - axis; ++y)
            for (int x = 0; x < W - (1 - axis); ++x) {
                int p = y * W + x, q = axis == 0 ? p + 1 : p + W;
                aa_pair r;
                if (!analyse(&in, p, q, axis, &r)) continue;
                int bcov = face_id[r.b] >= 0;
                double gt;
                if (r.t < 0.5) {
                    gt = gws[r.a] - (bcov ? gwn[4 * r.a + dir_of(r.a, r.b, W)] : 0.0);
                } else {
                    gt = gwn[4 * r.b + dir_of(r.b, r.a, W)] - (bcov ? gws[r.b] : 0.0);
                }
                if (gt == 0.0) continue;
                double den = r.ea - r.eb;
                double dt_dea = -r.eb / (den * den), dt_deb = r.ea / (den * den);
                int i = (r.k + 1) % 3, j = (r.k + 2) % 3;
                int vi = faces[i * F + r.face], vj = faces[j * F + r.face];
                const aa_tri* t = &r.tri;
                double au = (r.a % W) + 0.5, av = (r.a / W) + 0.5, bu = (r.b % W) + 0.5, bv = (r.b / W) + 0.5;
                /* e(p) = sgn((u_j - u_i)(p_v - v_i) - (v_j - v_i)(p_u - u_i)) */
                double s = t->sgn;
                double dui = dt_dea * s * (t->v[j] - av) + dt_deb * s * (t->v[j] - bv);
                double dvi = dt_dea * s * (au - t->u[j]) + dt_deb * s * (bu - t->u[j]);
                double duj = dt_dea * s * (av - t->v[i]) + dt_deb * s * (bv - t->v[i]);
                double dvj = dt_dea * s * (t->u[i] - au) + dt_deb * s * (t->u[i] - bu);
                g_vs[vi] += gt * dui;
                g_vs[V + vi] += gt * dvi;
                g_vs[vj] += gt * duj;
                g_vs[V + vj] += gt * dvj;
            }
    free(wself);
    free(wn);
    free(gws);
    free(gwn);
}
