/*
 * CPU oracle, part 2: the projection's backward (test infrastructure only; loaded
 * into the same liboracle.so as gm_oracle.c and, like it, sharing nothing with the
 * HIP library).
 *
 * gmesh README, "Design Details > Hybrid rendering" states that the whole renderer
 * is differentiable, through the depth split as well, so the Gaussians' own
 * parameters (means, rotations, scales, opacities, SH colour coefficients) receive
 * gradients through their projected 2D records.  The records are those of the
 * forward projection in gm_oracle.c (EWA splatting: Sigma = R S S^T R^T, Sigma_c =
 * W Sigma W^T, the pinhole Jacobian J, Sigma_2D = J Sigma_c J^T + 0.3 I, conic =
 * Sigma_2D^-1, the conditional depth model g = conic (J Sigma_c e_z), sigma^2 =
 * Sigma_c,zz - (J Sigma_c e_z) . g, SH colour at the view direction).
 *
 * Here that forward is re-evaluated in fp64 from fp64 inputs (value arithmetic: the
 * same formulas, no decisions) and differentiated by hand in reverse mode, one
 * step of the forward at a time, in reverse order.  Pins (tests/): central finite
 * differences of oc_project_f64, closed forms for an axis-aligned Gaussian on the
 * optical axis, and the invariance of the records under scaling of the quaternion.
 */
#include <math.h>
#include <stddef.h>

typedef struct {
    int width, height;
    float fx, fy, cx, cy;
    float R[9], t[3];
    float near_z;
} oc_camera_pb; /* same layout as oc_camera in gm_oracle.c */

#define PB_EPS2D 0.3
#define PB_NREC 13

typedef struct {
    double W[9], t[3], fx, fy, cx, cy, Cw[3];
} cam64;

static void cam64_of(const oc_camera_pb* c, cam64* k)
{
    for (int i = 0; i < 9; ++i) k->W[i] = c->R[i];
    for (int i = 0; i < 3; ++i) k->t[i] = c->t[i];
    k->fx = c->fx;
    k->fy = c->fy;
    k->cx = c->cx;
    k->cy = c->cy;
    /* camera centre C = -W^T t */
    for (int j = 0; j < 3; ++j) k->Cw[j] = -(k->W[0 * 3 + j] * k->t[0] + k->W[1 * 3 + j] * k->t[1] + k->W[2 * 3 + j] * k->t[2]);
}

/* Real SH basis (same closed forms as gm_oracle.c) and its gradient with respect to
 * the direction components, each polynomial differentiated term by term. */
static void sh_basis_grad(double x, double y, double z, double* Y, double (*dY)[3])
{
    const double pi = 3.14159265358979323846;
    const double c0 = 0.5 * sqrt(1.0 / pi), c1 = sqrt(3.0 / (4.0 * pi));
    const double a = 0.5 * sqrt(15.0 / pi), b = 0.25 * sqrt(5.0 / pi), c = 0.25 * sqrt(15.0 / pi);
    const double d0 = 0.25 * sqrt(35.0 / (2.0 * pi)), d1 = 0.5 * sqrt(105.0 / pi);
    const double d2 = 0.25 * sqrt(21.0 / (2.0 * pi)), d3 = 0.25 * sqrt(7.0 / pi);
    const double d5 = 0.25 * sqrt(105.0 / pi);
    const double xx = x * x, yy = y * y, zz = z * z;
    Y[0] = c0;                                   dY[0][0] = 0;             dY[0][1] = 0;             dY[0][2] = 0;
    Y[1] = -c1 * y;                              dY[1][0] = 0;             dY[1][1] = -c1;           dY[1][2] = 0;
    Y[2] = c1 * z;                               dY[2][0] = 0;             dY[2][1] = 0;             dY[2][2] = c1;
    Y[3] = -c1 * x;                              dY[3][0] = -c1;           dY[3][1] = 0;             dY[3][2] = 0;
    Y[4] = a * x * y;                            dY[4][0] = a * y;         dY[4][1] = a * x;         dY[4][2] = 0;
    Y[5] = -a * y * z;                           dY[5][0] = 0;             dY[5][1] = -a * z;        dY[5][2] = -a * y;
    Y[6] = b * (2.0 * zz - xx - yy);             dY[6][0] = -2.0 * b * x;  dY[6][1] = -2.0 * b * y;  dY[6][2] = 4.0 * b * z;
    Y[7] = -a * x * z;                           dY[7][0] = -a * z;        dY[7][1] = 0;             dY[7][2] = -a * x;
    Y[8] = c * (xx - yy);                        dY[8][0] = 2.0 * c * x;   dY[8][1] = -2.0 * c * y;  dY[8][2] = 0;
    /* -d0 (3 x^2 y - y^3) */
    Y[9] = -d0 * y * (3.0 * xx - yy);
    dY[9][0] = -6.0 * d0 * x * y;  dY[9][1] = -d0 * (3.0 * xx - 3.0 * yy);  dY[9][2] = 0;
    Y[10] = d1 * x * y * z;
    dY[10][0] = d1 * y * z;  dY[10][1] = d1 * x * z;  dY[10][2] = d1 * x * y;
    /* -d2 (4 y z^2 - x^2 y - y^3) */
    Y[11] = -d2 * y * (4.0 * zz - xx - yy);
    dY[11][0] = 2.0 * d2 * x * y;  dY[11][1] = -d2 * (4.0 * zz - xx - 3.0 * yy);  dY[11][2] = -8.0 * d2 * y * z;
    /* d3 (2 z^3 - 3 x^2 z - 3 y^2 z) */
    Y[12] = d3 * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
    dY[12][0] = -6.0 * d3 * x * z;  dY[12][1] = -6.0 * d3 * y * z;  dY[12][2] = d3 * (6.0 * zz - 3.0 * xx - 3.0 * yy);
    /* -d2 (4 x z^2 - x^3 - x y^2) */
    Y[13] = -d2 * x * (4.0 * zz - xx - yy);
    dY[13][0] = -d2 * (4.0 * zz - 3.0 * xx - yy);  dY[13][1] = 2.0 * d2 * x * y;  dY[13][2] = -8.0 * d2 * x * z;
    /* d5 (x^2 z - y^2 z) */
    Y[14] = d5 * z * (xx - yy);
    dY[14][0] = 2.0 * d5 * x * z;  dY[14][1] = -2.0 * d5 * y * z;  dY[14][2] = d5 * (xx - yy);
    /* -d0 (x^3 - 3 x y^2) */
    Y[15] = -d0 * x * (xx - 3.0 * yy);
    dY[15][0] = -d0 * (3.0 * xx - 3.0 * yy);  dY[15][1] = 6.0 * d0 * x * y;  dY[15][2] = 0;
}

/* Forward values of one Gaussian (fp64). */
typedef struct {
    double x[3];          /* camera-space mean */
    double qn, qh[4];     /* |q|, q / |q| (w, x, y, z) */
    double Rq[9], s[3], M[9], C[9];
    double J0[3], J1[3];  /* rows of the pinhole Jacobian: (fx/z, 0, -fx x/z^2), (0, fy/z, -fy y/z^2) */
    double S00, S01, S11, k0, k1, Szz;
    double a, b, c, det, Q00, Q01, Q11, g0, g1, var, sig, u, v;
    int clamp;            /* var <= 1e-12: sigma = 1e-6, flat */
    double dir[3], nrm, Y[16], dY[16][3], acc[3], col[3];
} g64;

/* shc[k * 3 + ch]: this Gaussian's colour coefficients ((d+1)^2 x 3), or RGB when
 * sh_degree < 0. */
static void proj64(const cam64* k, const double* mu, const double* q, const double* s, const double* shc,
                   int sh_degree, g64* g)
{
    const double* W = k->W;
    for (int r = 0; r < 3; ++r) g->x[r] = W[r * 3 + 0] * mu[0] + W[r * 3 + 1] * mu[1] + W[r * 3 + 2] * mu[2] + k->t[r];
    g->qn = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
    for (int i = 0; i < 4; ++i) g->qh[i] = q[i] / g->qn;
    const double w = g->qh[0], x = g->qh[1], y = g->qh[2], z = g->qh[3];
    double* R = g->Rq;
    R[0] = 1.0 - 2.0 * (y * y + z * z);
    R[1] = 2.0 * (x * y - w * z);
    R[2] = 2.0 * (x * z + w * y);
    R[3] = 2.0 * (x * y + w * z);
    R[4] = 1.0 - 2.0 * (x * x + z * z);
    R[5] = 2.0 * (y * z - w * x);
    R[6] = 2.0 * (x * z - w * y);
    R[7] = 2.0 * (y * z + w * x);
    R[8] = 1.0 - 2.0 * (x * x + y * y);
    for (int c = 0; c < 3; ++c) g->s[c] = s[c];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) g->M[r * 3 + c] = R[r * 3 + c] * s[c];
    double S[9], A[9];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            double v = 0.0;
            for (int j = 0; j < 3; ++j) v += g->M[r * 3 + j] * g->M[c * 3 + j];
            S[r * 3 + c] = v;
        }
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            double v = 0.0;
            for (int j = 0; j < 3; ++j) v += W[r * 3 + j] * S[j * 3 + c];
            A[r * 3 + c] = v;
        }
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            double v = 0.0;
            for (int j = 0; j < 3; ++j) v += A[r * 3 + j] * W[c * 3 + j];
            g->C[r * 3 + c] = v;
        }
    const double xc = g->x[0], yc = g->x[1], zc = g->x[2];
    g->J0[0] = k->fx / zc; g->J0[1] = 0.0; g->J0[2] = -k->fx * xc / (zc * zc);
    g->J1[0] = 0.0; g->J1[1] = k->fy / zc; g->J1[2] = -k->fy * yc / (zc * zc);
    double CJ0[3], CJ1[3];
    for (int r = 0; r < 3; ++r) {
        CJ0[r] = g->C[r * 3 + 0] * g->J0[0] + g->C[r * 3 + 1] * g->J0[1] + g->C[r * 3 + 2] * g->J0[2];
        CJ1[r] = g->C[r * 3 + 0] * g->J1[0] + g->C[r * 3 + 1] * g->J1[1] + g->C[r * 3 + 2] * g->J1[2];
    }
    g->S00 = g->J0[0] * CJ0[0] + g->J0[1] * CJ0[1] + g->J0[2] * CJ0[2];
    g->S01 = g->J0[0] * CJ1[0] + g->J0[1] * CJ1[1] + g->J0[2] * CJ1[2];
    g->S11 = g->J1[0] * CJ1[0] + g->J1[1] * CJ1[1] + g->J1[2] * CJ1[2];
    g->k0 = g->J0[0] * g->C[0 * 3 + 2] + g->J0[1] * g->C[1 * 3 + 2] + g->J0[2] * g->C[2 * 3 + 2];
    g->k1 = g->J1[0] * g->C[0 * 3 + 2] + g->J1[1] * g->C[1 * 3 + 2] + g->J1[2] * g->C[2 * 3 + 2];
    g->Szz = g->C[8];
    g->a = g->S00 + PB_EPS2D;
    g->b = g->S01;
    g->c = g->S11 + PB_EPS2D;
    g->det = g->a * g->c - g->b * g->b;
    g->Q00 = g->c / g->det;
    g->Q01 = -g->b / g->det;
    g->Q11 = g->a / g->det;
    g->g0 = g->Q00 * g->k0 + g->Q01 * g->k1;
    g->g1 = g->Q01 * g->k0 + g->Q11 * g->k1;
    g->var = g->Szz - (g->k0 * g->g0 + g->k1 * g->g1);
    g->clamp = !(g->var > 1e-12);
    g->sig = sqrt(g->clamp ? 1e-12 : g->var);
    g->u = k->fx * xc / zc + k->cx;
    g->v = k->fy * yc / zc + k->cy;
    if (sh_degree < 0) {
        for (int ch = 0; ch < 3; ++ch) g->col[ch] = shc[ch];
    } else {
        double d[3];
        for (int j = 0; j < 3; ++j) d[j] = mu[j] - k->Cw[j];
        g->nrm = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
        for (int j = 0; j < 3; ++j) g->dir[j] = d[j] / g->nrm;
        sh_basis_grad(g->dir[0], g->dir[1], g->dir[2], g->Y, g->dY);
        const int K = (sh_degree + 1) * (sh_degree + 1);
        for (int ch = 0; ch < 3; ++ch) {
            double acc = 0.0;
            for (int kk = 0; kk < K; ++kk) acc += g->Y[kk] * shc[kk * 3 + ch];
            g->acc[ch] = acc + 0.5;
            g->col[ch] = g->acc[ch] > 0.0 ? g->acc[ch] : 0.0;
        }
    }
}

/* Reverse mode through proj64.  gr: the 13 record gradients (u, v, Q00, Q01, Q11,
 * opacity, r, g, b, z_c, g0, g1, sigma).  Outputs: d/dmean (3), d/dq (4, raw
 * quaternion), d/dscale (3), d/dcoefficients (K x 3, or 3 for RGB). */
static void proj64_bwd(const cam64* k, const g64* g, const double* shc, int sh_degree, const double* gr,
                       double* gmu, double* gq, double* gs, double* gsh)
{
    for (int j = 0; j < 3; ++j) gmu[j] = 0.0;
    /* colour */
    if (sh_degree < 0) {
        for (int ch = 0; ch < 3; ++ch) gsh[ch] = gr[6 + ch];
    } else {
        const int K = (sh_degree + 1) * (sh_degree + 1);
        double gacc[3], gdir[3] = {0.0, 0.0, 0.0};
        for (int ch = 0; ch < 3; ++ch) gacc[ch] = g->acc[ch] > 0.0 ? gr[6 + ch] : 0.0;
        for (int kk = 0; kk < K; ++kk) {
            double gY = 0.0;
            for (int ch = 0; ch < 3; ++ch) {
                gsh[kk * 3 + ch] = g->Y[kk] * gacc[ch];
                gY += shc[kk * 3 + ch] * gacc[ch];
            }
            for (int j = 0; j < 3; ++j) gdir[j] += gY * g->dY[kk][j];
        }
        /* dir = d / |d|, d = mean - camera centre: d dir / d d = (I - dir dir^T) / |d| */
        const double dd = g->dir[0] * gdir[0] + g->dir[1] * gdir[1] + g->dir[2] * gdir[2];
        for (int j = 0; j < 3; ++j) gmu[j] += (gdir[j] - g->dir[j] * dd) / g->nrm;
    }
    /* sigma = sqrt(var) */
    const double gvar = g->clamp ? 0.0 : gr[12] / (2.0 * g->sig);
    /* var = Szz - (k0 g0 + k1 g1) */
    double gg0 = gr[10] - g->k0 * gvar, gg1 = gr[11] - g->k1 * gvar;
    double gk0 = -g->g0 * gvar, gk1 = -g->g1 * gvar, gSzz = gvar;
    /* g0 = Q00 k0 + Q01 k1, g1 = Q01 k0 + Q11 k1 */
    const double gQ00 = gr[2] + gg0 * g->k0;
    const double gQ01 = gr[3] + gg0 * g->k1 + gg1 * g->k0;
    const double gQ11 = gr[4] + gg1 * g->k1;
    gk0 += g->Q00 * gg0 + g->Q01 * gg1;
    gk1 += g->Q01 * gg0 + g->Q11 * gg1;
    /* (Q00, Q01, Q11) = (c, -b, a) / det, det = a c - b^2 */
    const double a = g->a, b = g->b, c = g->c, det = g->det, d2 = det * det;
    const double ga = gQ00 * (-c * c / d2) + gQ01 * (b * c / d2) + gQ11 * (-b * b / d2);
    const double gb = gQ00 * (2.0 * b * c / d2) + gQ01 * (-1.0 / det - 2.0 * b * b / d2) + gQ11 * (2.0 * a * b / d2);
    const double gc = gQ00 * (-b * b / d2) + gQ01 * (a * b / d2) + gQ11 * (-a * a / d2);
    const double gS00 = ga, gS01 = gb, gS11 = gc;
    /* S00 = J0 C J0^T, S01 = J0 C J1^T, S11 = J1 C J1^T, k0 = J0 C e_z, k1 = J1 C e_z,
     * Szz = C_zz: gradient with respect to C (as a general matrix) and to J0, J1 */
    const double* J0 = g->J0;
    const double* J1 = g->J1;
    double gC[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            gC[i * 3 + j] = gS00 * J0[i] * J0[j] + gS01 * J0[i] * J1[j] + gS11 * J1[i] * J1[j];
    for (int i = 0; i < 3; ++i) gC[i * 3 + 2] += gk0 * J0[i] + gk1 * J1[i];
    gC[8] += gSzz;
    double gJ0[3], gJ1[3];
    for (int i = 0; i < 3; ++i) {
        double cj0 = 0.0, cj1 = 0.0;
        for (int j = 0; j < 3; ++j) {
            cj0 += g->C[i * 3 + j] * J0[j];
            cj1 += g->C[i * 3 + j] * J1[j];
        }
        gJ0[i] = 2.0 * gS00 * cj0 + gS01 * cj1 + gk0 * g->C[i * 3 + 2];
        gJ1[i] = gS01 * cj0 + 2.0 * gS11 * cj1 + gk1 * g->C[i * 3 + 2];
    }
    /* J0 = (fx/z, 0, -fx x/z^2), J1 = (0, fy/z, -fy y/z^2); u, v; z_c */
    const double xc = g->x[0], yc = g->x[1], zc = g->x[2], fx = k->fx, fy = k->fy;
    double gx = 0.0, gy = 0.0, gz = 0.0;
    gz += -gJ0[0] * fx / (zc * zc);
    gx += -gJ0[2] * fx / (zc * zc);
    gz += gJ0[2] * 2.0 * fx * xc / (zc * zc * zc);
    gz += -gJ1[1] * fy / (zc * zc);
    gy += -gJ1[2] * fy / (zc * zc);
    gz += gJ1[2] * 2.0 * fy * yc / (zc * zc * zc);
    gx += gr[0] * fx / zc;
    gz += -gr[0] * fx * xc / (zc * zc);
    gy += gr[1] * fy / zc;
    gz += -gr[1] * fy * yc / (zc * zc);
    gz += gr[9];
    /* x_c = W mean + t */
    const double* W = k->W;
    for (int j = 0; j < 3; ++j) gmu[j] += W[0 * 3 + j] * gx + W[1 * 3 + j] * gy + W[2 * 3 + j] * gz;
    /* C = W Sigma W^T: gSigma = W^T gC W */
    double T[9], gS[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double v = 0.0;
            for (int l = 0; l < 3; ++l) v += W[l * 3 + i] * gC[l * 3 + j];
            T[i * 3 + j] = v;
        }
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double v = 0.0;
            for (int l = 0; l < 3; ++l) v += T[i * 3 + l] * W[l * 3 + j];
            gS[i * 3 + j] = v;
        }
    /* Sigma = M M^T: gM = (gSigma + gSigma^T) M */
    double gM[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double v = 0.0;
            for (int l = 0; l < 3; ++l) v += (gS[i * 3 + l] + gS[l * 3 + i]) * g->M[l * 3 + j];
            gM[i * 3 + j] = v;
        }
    /* M = R diag(s) */
    double gR[9];
    for (int c2 = 0; c2 < 3; ++c2) {
        gs[c2] = 0.0;
        for (int r = 0; r < 3; ++r) {
            gR[r * 3 + c2] = gM[r * 3 + c2] * g->s[c2];
            gs[c2] += gM[r * 3 + c2] * g->Rq[r * 3 + c2];
        }
    }
    /* R(w, x, y, z) of the unit quaternion */
    const double w = g->qh[0], x = g->qh[1], y = g->qh[2], z = g->qh[3];
    double gqh[4];
    gqh[0] = 2.0 * (-z * gR[1] + y * gR[2] + z * gR[3] - x * gR[5] - y * gR[6] + x * gR[7]);
    gqh[1] = 2.0 * (y * gR[1] + z * gR[2] + y * gR[3] - 2.0 * x * gR[4] - w * gR[5] + z * gR[6] + w * gR[7] -
                    2.0 * x * gR[8]);
    gqh[2] = 2.0 * (-2.0 * y * gR[0] + x * gR[1] + w * gR[2] + x * gR[3] + z * gR[5] - w * gR[6] + z * gR[7] -
                    2.0 * y * gR[8]);
    gqh[3] = 2.0 * (-2.0 * z * gR[0] - w * gR[1] + x * gR[2] + w * gR[3] - 2.0 * z * gR[4] + y * gR[5] +
                    x * gR[6] + y * gR[7]);
    /* qh = q / |q| */
    const double dq = g->qh[0] * gqh[0] + g->qh[1] * gqh[1] + g->qh[2] * gqh[2] + g->qh[3] * gqh[3];
    for (int i = 0; i < 4; ++i) gq[i] = (gqh[i] - g->qh[i] * dq) / g->qn;
}

static void gather(int N, int i, const double* means, const double* quats, const double* scales, const double* sh,
                   int sh_degree, double* mu, double* q, double* s, double* shc)
{
    for (int j = 0; j < 3; ++j) mu[j] = means[(size_t)j * N + i];
    for (int j = 0; j < 4; ++j) q[j] = quats[(size_t)j * N + i];
    for (int j = 0; j < 3; ++j) s[j] = scales[(size_t)j * N + i];
    const int K = sh_degree < 0 ? 1 : (sh_degree + 1) * (sh_degree + 1);
    for (int kk = 0; kk < K; ++kk)
        for (int ch = 0; ch < 3; ++ch) shc[kk * 3 + ch] = sh[((size_t)kk * 3 + ch) * N + i];
}

/* fp64 records [N][13] of every Gaussian (no validity decisions). */
void oc_project_f64(const oc_camera_pb* cam, int N, const double* means, const double* quats,
                    const double* scales, const double* opacity, const double* sh, int sh_degree, double* rec)
{
    cam64 k;
    cam64_of(cam, &k);
#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        double mu[3], q[4], s[3], shc[48];
        gather(N, i, means, quats, scales, sh, sh_degree, mu, q, s, shc);
        g64 g;
        proj64(&k, mu, q, s, shc, sh_degree, &g);
        double* o = rec + (size_t)i * PB_NREC;
        o[0] = g.u; o[1] = g.v; o[2] = g.Q00; o[3] = g.Q01; o[4] = g.Q11; o[5] = opacity[i];
        o[6] = g.col[0]; o[7] = g.col[1]; o[8] = g.col[2];
        o[9] = g.x[2]; o[10] = g.g0; o[11] = g.g1; o[12] = g.sig;
    }
}

/* Gradients of sum_i g_rec[i] . record_i with respect to every input plane.  Gaussians
 * with listed[i] == 0 (not on any tile) get zeros.  Outputs: g_means [3][N],
 * g_quats [4][N], g_scales [3][N], g_opacity [N], g_sh [K][3][N] (K = 1 for RGB). */
void oc_project_bwd(const oc_camera_pb* cam, int N, const double* means, const double* quats,
                    const double* scales, const double* sh, int sh_degree, const int* listed, const double* g_rec,
                    double* g_means, double* g_quats, double* g_scales, double* g_opacity, double* g_sh)
{
    cam64 k;
    cam64_of(cam, &k);
    const int K = sh_degree < 0 ? 1 : (sh_degree + 1) * (sh_degree + 1);
#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        double mu[3], q[4], s[3], shc[48];
        double gmu[3] = {0, 0, 0}, gq[4] = {0, 0, 0, 0}, gs[3] = {0, 0, 0}, gsh[48], go = 0.0;
        for (int j = 0; j < 48; ++j) gsh[j] = 0.0;
        if (listed[i]) {
            gather(N, i, means, quats, scales, sh, sh_degree, mu, q, s, shc);
            g64 g;
            proj64(&k, mu, q, s, shc, sh_degree, &g);
            proj64_bwd(&k, &g, shc, sh_degree, g_rec + (size_t)i * PB_NREC, gmu, gq, gs, gsh);
            go = g_rec[(size_t)i * PB_NREC + 5];
        }
        for (int j = 0; j < 3; ++j) g_means[(size_t)j * N + i] = gmu[j];
        for (int j = 0; j < 4; ++j) g_quats[(size_t)j * N + i] = gq[j];
        for (int j = 0; j < 3; ++j) g_scales[(size_t)j * N + i] = gs[j];
        g_opacity[i] = go;
        for (int kk = 0; kk < K; ++kk)
            for (int ch = 0; ch < 3; ++ch) g_sh[((size_t)kk * 3 + ch) * N + i] = gsh[kk * 3 + ch];
    }
}
