/*
 * CPU oracle, part 3: the mesh side of the backward (test infrastructure only;
 * loaded into liboracle.so with gm_oracle.c, sharing nothing with the HIP library).
 *
 * gmesh README, "Design Details": the mesh colour at a pixel comes from
 * perspective-correct barycentrics of the nearest triangle (vertex colours, or a
 * trilinear mip-mapped texture at the interpolated texture coordinate), lit per
 * pixel with Phong shading of interpolated normals by a point light (v1.1 notes),
 * and the mesh depth D enters the hybrid composite through the split; the renderer
 * is differentiable with respect to the mesh as well.  Given dL/dc_m and dL/dD per
 * pixel (outputs of the composite's reverse mode), this file computes the
 * gradients of the vertex positions, vertex colours, vertex normals, texture
 * coordinates, texture texels and light parameters.
 *
 * Readings: visibility (which face covers a pixel) is taken as given and carries
 * no gradient; the texture level of detail is taken as given (no gradient through
 * the screen-space derivatives that select it); the gradient of a clamp or of
 * max(0, .) is zero on the clamped side.
 *
 * Everything is fp64, from fp64 inputs: vertex positions are projected here in
 * fp64 (the continuous map the fp32 vertex projection rounds).  Pins (tests/):
 * central finite differences of oc_mesh_fwd64 for every input, the constant
 * texture closed form (dL/dtexel summed over texels = coverage-weighted sum of the
 * pixel gradients), and vertex-colour closed forms.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

typedef struct {
    int width, height;
    float fx, fy, cx, cy;
    float R[9], t[3];
    float near_z;
} mb_camera; /* same layout as oc_camera in gm_oracle.c */

typedef struct {
    int V, F, Vt, S;       /* S: square texture side, 0 when untextured */
    const double* verts;   /* [3][V] world positions */
    const int* faces;      /* [3][F] */
    const double* vcolor;  /* [3][V] or NULL */
    const double* vnormal; /* [3][V] or NULL (unlit) */
    const double* uv;      /* [2][Vt] or NULL */
    const int* faces_uv;   /* [3][F] or NULL */
    const double* tex;     /* [S][S][3] or NULL */
    const double* light;   /* pos[3], ambient[3], diffuse[3], specular[3], shininess; NULL = unlit */
} mb_mesh;

static int mb_levels(int S)
{
    int n = 0;
    for (int s = S; s >= 1; s >>= 1) ++n;
    return n;
}

/* Box-filter pyramid (level l+1 texel = mean of its 2x2 block of level l), levels
 * back to back, fp64. */
static double* mb_pyramid(const double* tex, int S)
{
    size_t total = 0;
    for (int s = S; s >= 1; s >>= 1) total += (size_t)s * s * 3;
    double* m = (double*)malloc(sizeof(double) * total);
    for (size_t i = 0; i < (size_t)S * S * 3; ++i) m[i] = tex[i];
    double* prev = m;
    for (int s = S; s > 1; s >>= 1) {
        const int h = s / 2;
        double* cur = prev + (size_t)s * s * 3;
        for (int y = 0; y < h; ++y)
            for (int x = 0; x < h; ++x)
                for (int c = 0; c < 3; ++c)
                    cur[((size_t)y * h + x) * 3 + c] =
                        0.25 * (prev[((size_t)(2 * y) * s + 2 * x) * 3 + c] + prev[((size_t)(2 * y) * s + 2 * x + 1) * 3 + c] +
                                prev[((size_t)(2 * y + 1) * s + 2 * x) * 3 + c] +
                                prev[((size_t)(2 * y + 1) * s + 2 * x + 1) * 3 + c]);
        prev = cur;
    }
    return m;
}

static size_t mb_level_offset(int S, int l)
{
    size_t o = 0;
    for (int k = 0; k < l; ++k) o += (size_t)(S >> k) * (S >> k) * 3;
    return o;
}

/* Bilinear lookup with clamp-to-edge addressing at (u, v) in [0, 1] (clamped).
 * Returns the colour, the four texel indices and weights, and d colour / d(u, v). */
typedef struct {
    size_t idx[4];
    double wgt[4];
    double col[3], du[3], dv[3];
} mb_bilin;

static void mb_bilinear(const double* lvl, int s, double u, double v, mb_bilin* b)
{
    const double cu = u < 0 ? 0 : (u > 1 ? 1 : u), cv = v < 0 ? 0 : (v > 1 ? 1 : v);
    const double su = (u > 0 && u < 1) ? 1.0 : 0.0, sv = (v > 0 && v < 1) ? 1.0 : 0.0;
    const double x = cu * s - 0.5, y = cv * s - 0.5;
    const double x0 = floor(x), y0 = floor(y);
    const double ax = x - x0, ay = y - y0;
    int ix0 = (int)x0, iy0 = (int)y0, ix1 = ix0 + 1, iy1 = iy0 + 1;
    ix0 = ix0 < 0 ? 0 : (ix0 > s - 1 ? s - 1 : ix0);
    ix1 = ix1 < 0 ? 0 : (ix1 > s - 1 ? s - 1 : ix1);
    iy0 = iy0 < 0 ? 0 : (iy0 > s - 1 ? s - 1 : iy0);
    iy1 = iy1 < 0 ? 0 : (iy1 > s - 1 ? s - 1 : iy1);
    b->idx[0] = ((size_t)iy0 * s + ix0) * 3;
    b->idx[1] = ((size_t)iy0 * s + ix1) * 3;
    b->idx[2] = ((size_t)iy1 * s + ix0) * 3;
    b->idx[3] = ((size_t)iy1 * s + ix1) * 3;
    b->wgt[0] = (1 - ax) * (1 - ay);
    b->wgt[1] = ax * (1 - ay);
    b->wgt[2] = (1 - ax) * ay;
    b->wgt[3] = ax * ay;
    for (int c = 0; c < 3; ++c) {
        const double t00 = lvl[b->idx[0] + c], t01 = lvl[b->idx[1] + c];
        const double t10 = lvl[b->idx[2] + c], t11 = lvl[b->idx[3] + c];
        const double top = t00 + (t01 - t00) * ax, bot = t10 + (t11 - t10) * ax;
        b->col[c] = top + (bot - top) * ay;
        b->du[c] = ((t01 - t00) * (1 - ay) + (t11 - t10) * ay) * s * su;
        b->dv[c] = (bot - top) * s * sv;
    }
}

/* Forward state of one pixel. */
typedef struct {
    int vi[3], ti[3];
    double X[3][3], xc[3][3];        /* world and camera positions of the corners */
    double u[3], v[3], z[3];         /* screen positions and depths */
    double E[3], A, lam[3], w[3], W, zz, b[3];
    /* texture */
    int textured, l0, l1;
    double tl, uu, vv, uvk[3][2];
    mb_bilin B0, B1;
    double base[3];
    /* lighting */
    int lit;
    double nw[3], nt[3], nn, n[3], L[3], x[3], lt[3], ln, l[3], et[3], en, e[3], ndl, r[3], rde, diff, spec;
    double cm[3];
} mb_px;

static void mb_forward(const mb_camera* cam, const mb_mesh* m, const double* mips, int px, int py, int f, mb_px* s)
{
    double R[9], t[3];
    for (int i = 0; i < 9; ++i) R[i] = cam->R[i];
    for (int i = 0; i < 3; ++i) t[i] = cam->t[i];
    const double fx = cam->fx, fy = cam->fy, cx = cam->cx, cy = cam->cy;
    for (int k = 0; k < 3; ++k) {
        s->vi[k] = m->faces[k * m->F + f];
        for (int j = 0; j < 3; ++j) s->X[k][j] = m->verts[(size_t)j * m->V + s->vi[k]];
        for (int r = 0; r < 3; ++r)
            s->xc[k][r] = R[r * 3 + 0] * s->X[k][0] + R[r * 3 + 1] * s->X[k][1] + R[r * 3 + 2] * s->X[k][2] + t[r];
        s->u[k] = fx * s->xc[k][0] / s->xc[k][2] + cx;
        s->v[k] = fy * s->xc[k][1] / s->xc[k][2] + cy;
        s->z[k] = s->xc[k][2];
    }
    const double pu = px + 0.5, pv = py + 0.5;
    /* edge (a -> b) opposite corner k: (1,2), (2,0), (0,1) */
    const int ea[3] = {1, 2, 0}, eb[3] = {2, 0, 1};
    for (int k = 0; k < 3; ++k) {
        const int a = ea[k], b = eb[k];
        s->E[k] = (s->u[b] - s->u[a]) * (pv - s->v[a]) - (s->v[b] - s->v[a]) * (pu - s->u[a]);
    }
    s->A = (s->u[1] - s->u[0]) * (s->v[2] - s->v[0]) - (s->v[1] - s->v[0]) * (s->u[2] - s->u[0]);
    s->W = 0;
    for (int k = 0; k < 3; ++k) {
        s->lam[k] = s->E[k] / s->A;
        s->w[k] = s->lam[k] / s->z[k];
        s->W += s->w[k];
    }
    s->zz = 1.0 / s->W;
    for (int k = 0; k < 3; ++k) s->b[k] = s->w[k] * s->zz;

    for (int c = 0; c < 3; ++c) s->base[c] = 0;
    s->textured = m->tex && m->uv && m->faces_uv;
    if (s->textured) {
        for (int k = 0; k < 3; ++k) {
            s->ti[k] = m->faces_uv[k * m->F + f];
            s->uvk[k][0] = m->uv[s->ti[k]];
            s->uvk[k][1] = m->uv[m->Vt + s->ti[k]];
        }
        s->uu = s->vv = 0;
        for (int k = 0; k < 3; ++k) {
            s->uu += s->b[k] * s->uvk[k][0];
            s->vv += s->b[k] * s->uvk[k][1];
        }
        /* level of detail from the analytic screen derivatives (taken as given below) */
        double dux = 0, dvx = 0, duy = 0, dvy = 0;
        for (int k = 0; k < 3; ++k) {
            const double dwx = (-(s->v[eb[k]] - s->v[ea[k]]) / s->A) / s->z[k];
            const double dwy = ((s->u[eb[k]] - s->u[ea[k]]) / s->A) / s->z[k];
            dux += dwx * (s->uvk[k][0] - s->uu) / s->W;
            dvx += dwx * (s->uvk[k][1] - s->vv) / s->W;
            duy += dwy * (s->uvk[k][0] - s->uu) / s->W;
            dvy += dwy * (s->uvk[k][1] - s->vv) / s->W;
        }
        const double S0 = m->S;
        const double lx = sqrt(S0 * dux * S0 * dux + S0 * dvx * S0 * dvx);
        const double ly = sqrt(S0 * duy * S0 * duy + S0 * dvy * S0 * dvy);
        const double rho = lx > ly ? lx : ly;
        const int lmax = mb_levels(m->S) - 1;
        double lod = rho > 0 ? log2(rho) : 0.0;
        lod = lod < 0 ? 0 : (lod > lmax ? lmax : lod);
        s->l0 = (int)floor(lod);
        s->l1 = s->l0 + 1 < lmax ? s->l0 + 1 : lmax;
        s->tl = lod - s->l0;
        mb_bilinear(mips + mb_level_offset(m->S, s->l0), m->S >> s->l0, s->uu, s->vv, &s->B0);
        mb_bilinear(mips + mb_level_offset(m->S, s->l1), m->S >> s->l1, s->uu, s->vv, &s->B1);
        for (int c = 0; c < 3; ++c) s->base[c] = s->B0.col[c] + (s->B1.col[c] - s->B0.col[c]) * s->tl;
    } else if (m->vcolor) {
        for (int c = 0; c < 3; ++c)
            for (int k = 0; k < 3; ++k) s->base[c] += s->b[k] * m->vcolor[(size_t)c * m->V + s->vi[k]];
    }
    s->lit = m->light && m->vnormal;
    if (s->lit) {
        const double* lp = m->light;
        for (int c = 0; c < 3; ++c) {
            s->nw[c] = 0;
            for (int k = 0; k < 3; ++k) s->nw[c] += s->b[k] * m->vnormal[(size_t)c * m->V + s->vi[k]];
        }
        for (int r = 0; r < 3; ++r) {
            s->nt[r] = R[r * 3 + 0] * s->nw[0] + R[r * 3 + 1] * s->nw[1] + R[r * 3 + 2] * s->nw[2];
            s->L[r] = R[r * 3 + 0] * lp[0] + R[r * 3 + 1] * lp[1] + R[r * 3 + 2] * lp[2] + t[r];
        }
        s->x[0] = (pu - cx) / fx * s->zz;
        s->x[1] = (pv - cy) / fy * s->zz;
        s->x[2] = s->zz;
        s->nn = sqrt(s->nt[0] * s->nt[0] + s->nt[1] * s->nt[1] + s->nt[2] * s->nt[2]);
        for (int r = 0; r < 3; ++r) {
            s->lt[r] = s->L[r] - s->x[r];
            s->et[r] = -s->x[r];
        }
        s->ln = sqrt(s->lt[0] * s->lt[0] + s->lt[1] * s->lt[1] + s->lt[2] * s->lt[2]);
        s->en = sqrt(s->et[0] * s->et[0] + s->et[1] * s->et[1] + s->et[2] * s->et[2]);
        for (int r = 0; r < 3; ++r) {
            s->n[r] = s->nt[r] / s->nn;
            s->l[r] = s->lt[r] / s->ln;
            s->e[r] = s->et[r] / s->en;
        }
        s->ndl = s->n[0] * s->l[0] + s->n[1] * s->l[1] + s->n[2] * s->l[2];
        for (int r = 0; r < 3; ++r) s->r[r] = 2.0 * s->ndl * s->n[r] - s->l[r];
        s->rde = s->r[0] * s->e[0] + s->r[1] * s->e[1] + s->r[2] * s->e[2];
        s->diff = s->ndl > 0 ? s->ndl : 0.0;
        s->spec = (s->ndl > 0 && s->rde > 0) ? pow(s->rde, lp[12]) : 0.0;
        for (int c = 0; c < 3; ++c) s->cm[c] = s->base[c] * (lp[3 + c] + lp[6 + c] * s->diff) + lp[9 + c] * s->spec;
    } else {
        for (int c = 0; c < 3; ++c) s->cm[c] = s->base[c];
    }
}

/* c_m [npix][3] and D [npix] of the given pixels and faces (fp64). */
void oc_mesh_fwd64(const mb_camera* cam, const mb_mesh* m, int npix, const int* pix, const int* face, double* cm,
                   double* D)
{
    double* mips = m->tex ? mb_pyramid(m->tex, m->S) : NULL;
#pragma omp parallel for schedule(static)
    for (int k = 0; k < npix; ++k) {
        mb_px s;
        mb_forward(cam, m, mips, pix[k] % cam->width, pix[k] / cam->width, face[k], &s);
        for (int c = 0; c < 3; ++c) cm[k * 3 + c] = s.cm[c];
        D[k] = s.zz;
    }
    free(mips);
}

#define MB_ADD(ptr, val)       \
    do {                       \
        double v_ = (val);     \
        _Pragma("omp atomic")  \
        *(ptr) += v_;          \
    } while (0)

/* Reverse mode.  g_cm [npix][3] = dL/dc_m, g_D [npix] = dL/dD (either may be NULL).
 * Outputs are accumulated (the caller zero-fills): g_verts [3][V], g_vcolor [3][V],
 * g_vnormal [3][V], g_uv [2][Vt], g_tex [S][S][3], g_light [13] (pos, ambient,
 * diffuse, specular, shininess).  Unused outputs may be NULL. */
void oc_mesh_bwd(const mb_camera* cam, const mb_mesh* m, int npix, const int* pix, const int* face,
                 const double* g_cm, const double* g_D, double* g_verts, double* g_vcolor, double* g_vnormal,
                 double* g_uv, double* g_tex, double* g_light)
{
    double* mips = m->tex ? mb_pyramid(m->tex, m->S) : NULL;
    size_t ptotal = 0;
    for (int s = m->S; s >= 1; s >>= 1) ptotal += (size_t)s * s * 3;
    double* gmips = m->tex ? (double*)calloc(ptotal, sizeof(double)) : NULL;
    double R[9];
    for (int i = 0; i < 9; ++i) R[i] = cam->R[i];
    const double fx = cam->fx, fy = cam->fy, cx = cam->cx, cy = cam->cy;
#pragma omp parallel for schedule(dynamic, 64)
    for (int k = 0; k < npix; ++k) {
        const int px = pix[k] % cam->width, py = pix[k] / cam->width;
        mb_px s;
        mb_forward(cam, m, mips, px, py, face[k], &s);
        double gc[3] = {0, 0, 0};
        if (g_cm)
            for (int c = 0; c < 3; ++c) gc[c] = g_cm[k * 3 + c];
        double gz = g_D ? g_D[k] : 0.0;
        double gb[3] = {0, 0, 0}, gbase[3];
        /* lighting */
        if (s.lit) {
            const double* lp = m->light;
            double gdiff = 0, gspec = 0;
            for (int c = 0; c < 3; ++c) {
                gbase[c] = gc[c] * (lp[3 + c] + lp[6 + c] * s.diff);
                if (g_light) {
                    MB_ADD(&g_light[3 + c], gc[c] * s.base[c]);
                    MB_ADD(&g_light[6 + c], gc[c] * s.base[c] * s.diff);
                    MB_ADD(&g_light[9 + c], gc[c] * s.spec);
                }
                gdiff += gc[c] * s.base[c] * lp[6 + c];
                gspec += gc[c] * lp[9 + c];
            }
            double gndl = s.ndl > 0 ? gdiff : 0.0, grde = 0;
            if (s.ndl > 0 && s.rde > 0) {
                grde = gspec * lp[12] * pow(s.rde, lp[12] - 1.0);
                if (g_light) MB_ADD(&g_light[12], gspec * s.spec * log(s.rde));
            }
            double gn[3], gl[3], ge[3];
            /* rde = r . e, r = 2 ndl n - l */
            double rn = 0;
            for (int r = 0; r < 3; ++r) {
                const double grr = grde * s.e[r];
                ge[r] = grde * s.r[r];
                rn += grr * s.n[r];
                gn[r] = 2.0 * s.ndl * grr;
                gl[r] = -grr;
            }
            gndl += 2.0 * rn;
            for (int r = 0; r < 3; ++r) {  /* ndl = n . l */
                gn[r] += gndl * s.l[r];
                gl[r] += gndl * s.n[r];
            }
            /* normalisations */
            double dn = 0, dl = 0, de = 0;
            for (int r = 0; r < 3; ++r) {
                dn += s.n[r] * gn[r];
                dl += s.l[r] * gl[r];
                de += s.e[r] * ge[r];
            }
            double gnt[3], glt[3], get[3];
            for (int r = 0; r < 3; ++r) {
                gnt[r] = (gn[r] - s.n[r] * dn) / s.nn;
                glt[r] = (gl[r] - s.l[r] * dl) / s.ln;
                get[r] = (ge[r] - s.e[r] * de) / s.en;
            }
            /* nt = R nw, nw = sum b_k normal_k; lt = L - x, et = -x, L = R pos + t */
            double gnw[3], gx[3];
            for (int j = 0; j < 3; ++j) {
                gnw[j] = R[0 * 3 + j] * gnt[0] + R[1 * 3 + j] * gnt[1] + R[2 * 3 + j] * gnt[2];
                if (g_light) MB_ADD(&g_light[j], R[0 * 3 + j] * glt[0] + R[1 * 3 + j] * glt[1] + R[2 * 3 + j] * glt[2]);
            }
            for (int r = 0; r < 3; ++r) gx[r] = -glt[r] - get[r];
            for (int kk = 0; kk < 3; ++kk) {
                double acc = 0;
                for (int c = 0; c < 3; ++c) {
                    acc += m->vnormal[(size_t)c * m->V + s.vi[kk]] * gnw[c];
                    if (g_vnormal) MB_ADD(&g_vnormal[(size_t)c * m->V + s.vi[kk]], s.b[kk] * gnw[c]);
                }
                gb[kk] += acc;
            }
            /* x = ((pu - cx)/fx z, (pv - cy)/fy z, z) */
            gz += gx[0] * (px + 0.5 - cx) / fx + gx[1] * (py + 0.5 - cy) / fy + gx[2];
        } else {
            for (int c = 0; c < 3; ++c) gbase[c] = gc[c];
        }
        /* base colour */
        if (s.textured) {
            double guu = 0, gvv = 0;
            for (int c = 0; c < 3; ++c) {
                const double g0 = gbase[c] * (1.0 - s.tl), g1 = gbase[c] * s.tl;
                guu += g0 * s.B0.du[c] + g1 * s.B1.du[c];
                gvv += g0 * s.B0.dv[c] + g1 * s.B1.dv[c];
                const size_t o0 = mb_level_offset(m->S, s.l0), o1 = mb_level_offset(m->S, s.l1);
                for (int q = 0; q < 4; ++q) {
                    MB_ADD(&gmips[o0 + s.B0.idx[q] + c], g0 * s.B0.wgt[q]);
                    MB_ADD(&gmips[o1 + s.B1.idx[q] + c], g1 * s.B1.wgt[q]);
                }
            }
            for (int kk = 0; kk < 3; ++kk) {
                gb[kk] += s.uvk[kk][0] * guu + s.uvk[kk][1] * gvv;
                if (g_uv) {
                    MB_ADD(&g_uv[s.ti[kk]], s.b[kk] * guu);
                    MB_ADD(&g_uv[m->Vt + s.ti[kk]], s.b[kk] * gvv);
                }
            }
        } else if (m->vcolor) {
            for (int kk = 0; kk < 3; ++kk)
                for (int c = 0; c < 3; ++c) {
                    gb[kk] += m->vcolor[(size_t)c * m->V + s.vi[kk]] * gbase[c];
                    if (g_vcolor) MB_ADD(&g_vcolor[(size_t)c * m->V + s.vi[kk]], s.b[kk] * gbase[c]);
                }
        }
        if (!g_verts) continue;
        /* b_k = w_k z, z = 1 / W, W = sum w_k, w_k = lam_k / z_k, lam_k = E_k / A */
        double gw[3];
        for (int kk = 0; kk < 3; ++kk) {
            gw[kk] = gb[kk] * s.zz;
            gz += gb[kk] * s.w[kk];
        }
        const double gW = -gz * s.zz * s.zz;
        double glam[3], gzk[3], gu[3] = {0, 0, 0}, gv[3] = {0, 0, 0};
        for (int kk = 0; kk < 3; ++kk) {
            gw[kk] += gW;
            glam[kk] = gw[kk] / s.z[kk];
            gzk[kk] = -gw[kk] * s.lam[kk] / (s.z[kk] * s.z[kk]);
        }
        double gA = 0;
        const int ea[3] = {1, 2, 0}, eb[3] = {2, 0, 1};
        const double pu = px + 0.5, pv = py + 0.5;
        for (int kk = 0; kk < 3; ++kk) {
            const double gE = glam[kk] / s.A;
            gA -= glam[kk] * s.lam[kk] / s.A;
            const int a = ea[kk], b = eb[kk];
            /* E = (u_b - u_a)(pv - v_a) - (v_b - v_a)(pu - u_a) */
            gu[a] += gE * (s.v[b] - pv);
            gu[b] += gE * (pv - s.v[a]);
            gv[a] += gE * (pu - s.u[b]);
            gv[b] += gE * (s.u[a] - pu);
        }
        /* A = (u1 - u0)(v2 - v0) - (v1 - v0)(u2 - u0) */
        gu[0] += gA * (s.v[1] - s.v[2]);
        gu[1] += gA * (s.v[2] - s.v[0]);
        gu[2] += gA * (s.v[0] - s.v[1]);
        gv[0] += gA * (s.u[2] - s.u[1]);
        gv[1] += gA * (s.u[0] - s.u[2]);
        gv[2] += gA * (s.u[1] - s.u[0]);
        /* u = fx x/z + cx, v = fy y/z + cy, z; x_c = R X + t */
        for (int kk = 0; kk < 3; ++kk) {
            const double zc = s.xc[kk][2];
            const double gxc = gu[kk] * fx / zc, gyc = gv[kk] * fy / zc;
            const double gzc = gzk[kk] - gu[kk] * fx * s.xc[kk][0] / (zc * zc) - gv[kk] * fy * s.xc[kk][1] / (zc * zc);
            for (int j = 0; j < 3; ++j)
                MB_ADD(&g_verts[(size_t)j * m->V + s.vi[kk]], R[0 * 3 + j] * gxc + R[1 * 3 + j] * gyc + R[2 * 3 + j] * gzc);
        }
    }
    /* pyramid adjoint: each coarse texel's gradient goes 1/4 to each of its children */
    if (gmips) {
        const int nl = mb_levels(m->S);
        for (int l = nl - 1; l >= 1; --l) {
            const int s = m->S >> l, sf = m->S >> (l - 1);
            const double* gc = gmips + mb_level_offset(m->S, l);
            double* gf = gmips + mb_level_offset(m->S, l - 1);
            for (int y = 0; y < s; ++y)
                for (int x = 0; x < s; ++x)
                    for (int c = 0; c < 3; ++c) {
                        const double g = 0.25 * gc[((size_t)y * s + x) * 3 + c];
                        gf[((size_t)(2 * y) * sf + 2 * x) * 3 + c] += g;
                        gf[((size_t)(2 * y) * sf + 2 * x + 1) * 3 + c] += g;
                        gf[((size_t)(2 * y + 1) * sf + 2 * x) * 3 + c] += g;
                        gf[((size_t)(2 * y + 1) * sf + 2 * x + 1) * 3 + c] += g;
                    }
        }
        if (g_tex)
            for (size_t i = 0; i < (size_t)m->S * m->S * 3; ++i) g_tex[i] += gmips[i];
    }
    free(gmips);
    free(mips);
}

/* Gradients of the screen positions of the vertices (dL/du, dL/dv per vertex, [2][V],
 * e.g. from the antialiased silhouettes) carried to the world positions through the
 * fp64 pinhole projection u = fx x_c / z_c + cx, v = fy y_c / z_c + cy, x_c = R X + t.
 * Accumulated into g_verts [3][V]. */
void oc_vscreen_bwd(const mb_camera* cam, const mb_mesh* m, const double* g_vs, double* g_verts)
{
    const int V = m->V;
    for (int i = 0; i < V; ++i) {
        const double gu = g_vs[i], gv = g_vs[V + i];
        if (gu == 0.0 && gv == 0.0) continue;
        double xc[3];
        for (int r = 0; r < 3; ++r)
            xc[r] = (double)cam->R[3 * r] * m->verts[i] + (double)cam->R[3 * r + 1] * m->verts[V + i] +
                    (double)cam->R[3 * r + 2] * m->verts[2 * V + i] + (double)cam->t[r];
        const double z = xc[2];
        const double gx = gu * cam->fx / z, gy = gv * cam->fy / z;
        const double gzc = -gu * cam->fx * xc[0] / (z * z) - gv * cam->fy * xc[1] / (z * z);
        for (int j = 0; j < 3; ++j)
            g_verts[(size_t)j * V + i] += (double)cam->R[j] * gx + (double)cam->R[3 + j] * gy + (double)cam->R[6 + j] * gzc;
    }
}
