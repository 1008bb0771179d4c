// Backward of the Gaussian projection: from the 13 record gradients to the
// Gaussians' means, quaternions, scales, opacities and SH coefficients (gmesh
// README, "Design Details > Hybrid rendering": the renderer is differentiable end to
// end, through the depth split as well, so the Gaussian parameters receive
// gradients through their projected records).
//
// One thread per Gaussian.  The forward (EWA covariance, pinhole Jacobian, conic,
// depth model, SH colour) is re-evaluated and differentiated in reverse order.
// The covariance chain runs in fp64: for long, thin Gaussians the 2D covariance is
// nearly singular and the depth model's variance is a small difference of large
// terms, so fp32 would lose most of its digits there; fp64 costs little in a kernel
// bound by its memory traffic.  The SH colour part is well conditioned and stays
// fp32.  Value arithmetic only: no decision depends on it, so contraction is on.
#include "gm_internal.h"
#include "gm_sh.h"

namespace gm {

constexpr double BWD_EPS2D = 0.3;  // the forward's low-pass dilation

__global__ void __launch_bounds__(256)
k_project_bwd(DevCamera cam, int N, const float* __restrict__ means, const float* __restrict__ quats,
              const float* __restrict__ scales, const float* __restrict__ opacity, const float* __restrict__ sh,
              int sh_degree, const float* __restrict__ rec, const float* __restrict__ g_rec,
              float* __restrict__ g_means, float* __restrict__ g_quats, float* __restrict__ g_scales,
              float* __restrict__ g_opacity, float* __restrict__ g_sh, float* __restrict__ g_log_scales,
              float* __restrict__ g_logit)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int K = sh_degree < 0 ? 1 : (sh_degree + 1) * (sh_degree + 1);
    // An unlisted Gaussian (no record gradient) gets zero gradients.  It runs the same
    // arithmetic, with its outputs replaced by zeros at the stores (its forward values
    // may be infinite), so that every load is issued at once, none behind the test.
    // unrolled over the 16 coefficients (K of them live), issued with every other load
    float shv[48];
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) shv[k * 3 + ch] = k < K ? sh[((size_t)k * 3 + ch) * N + i] : 0.0f;
    const bool listed = __float_as_int(rec[(size_t)i * GM_REC + 15]) > 0;
    float gr[GM_GRAD];
#pragma unroll
    for (int k = 0; k < GM_GRAD; ++k) gr[k] = g_rec[(size_t)i * GM_GRAD + k];
    const int keep = listed ? -1 : 0;  // a mask rather than a select, which the compiler
                                       // would turn back into loads behind the test
#pragma unroll
    for (int k = 0; k < GM_GRAD; ++k) gr[k] = __int_as_float(__float_as_int(gr[k]) & keep);
    double W[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) W[k] = cam.R[k];
    const double mu[3] = {means[i], means[N + i], means[2 * N + i]};
    const double qr[4] = {quats[i], quats[N + i], quats[2 * N + i], quats[3 * N + i]};
    const double s[3] = {scales[i], scales[N + i], scales[2 * N + i]};

    // ---- forward values (fp64) ------------------------------------------------------
    double xc[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) xc[r] = W[3 * r] * mu[0] + W[3 * r + 1] * mu[1] + W[3 * r + 2] * mu[2] + (double)cam.t[r];
    const double qn = sqrt(qr[0] * qr[0] + qr[1] * qr[1] + qr[2] * qr[2] + qr[3] * qr[3]);
    const double iqn = 1.0 / qn;
    const double w = qr[0] * iqn, x = qr[1] * iqn, y = qr[2] * iqn, z = qr[3] * iqn;
    double R[9];
    R[0] = 1.0 - 2.0 * (y * y + z * z);
    R[1] = 2.0 * (x * y - w * z);
    R[2] = 2.0 * (x * z + w * y);
    R[3] = 2.0 * (x * y + w * z);
    R[4] = 1.0 - 2.0 * (x * x + z * z);
    R[5] = 2.0 * (y * z - w * x);
    R[6] = 2.0 * (x * z - w * y);
    R[7] = 2.0 * (y * z + w * x);
    R[8] = 1.0 - 2.0 * (x * x + y * y);
    double M[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) M[3 * r + c] = R[3 * r + c] * s[c];
    // camera-space covariance C = (W M)(W M)^T
    double WM[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) WM[3 * r + c] = W[3 * r] * M[c] + W[3 * r + 1] * M[3 + c] + W[3 * r + 2] * M[6 + c];
    double C[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = r; c < 3; ++c) {
            const double v = WM[3 * r] * WM[3 * c] + WM[3 * r + 1] * WM[3 * c + 1] + WM[3 * r + 2] * WM[3 * c + 2];
            C[3 * r + c] = v;
            C[3 * c + r] = v;
        }
    const double fx = cam.fx, fy = cam.fy;
    const double iz = 1.0 / xc[2];
    const double j00 = fx * iz, j02 = -fx * xc[0] * iz * iz;
    const double j11 = fy * iz, j12 = -fy * xc[1] * iz * iz;
    const double J0[3] = {j00, 0.0, j02}, J1[3] = {0.0, j11, j12};
    double CJ0[3], CJ1[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        CJ0[r] = C[3 * r] * j00 + C[3 * r + 2] * j02;
        CJ1[r] = C[3 * r + 1] * j11 + C[3 * r + 2] * j12;
    }
    const double a = j00 * CJ0[0] + j02 * CJ0[2] + BWD_EPS2D;
    const double b = j00 * CJ1[0] + j02 * CJ1[2];
    const double c = j11 * CJ1[1] + j12 * CJ1[2] + BWD_EPS2D;
    const double k0 = CJ0[2], k1 = CJ1[2];
    const double det = a * c - b * b, idet = 1.0 / det;
    const double Q00 = c * idet, Q01 = -b * idet, Q11 = a * idet;
    const double g0 = Q00 * k0 + Q01 * k1, g1 = Q01 * k0 + Q11 * k1;
    const double var = C[8] - (k0 * g0 + k1 * g1);
    const bool clamp = !(var > 1e-12);
    const double sig = sqrt(clamp ? 1e-12 : var);

    // ---- colour (fp32) ---------------------------------------------------------------
    double gmu[3] = {0.0, 0.0, 0.0};
    if (sh_degree < 0) {
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) g_sh[(size_t)ch * N + i] = gr[6 + ch];  // zero when unlisted
    } else {
        const float* Wf = cam.R;
        float cw[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) cw[j] = -(Wf[j] * cam.t[0] + Wf[3 + j] * cam.t[1] + Wf[6 + j] * cam.t[2]);
        const float d0 = means[i] - cw[0], d1 = means[N + i] - cw[1], d2 = means[2 * N + i] - cw[2];
        const float nrm = sqrtf(d0 * d0 + d1 * d1 + d2 * d2), inrm = 1.0f / nrm;
        const float dx = d0 * inrm, dy = d1 * inrm, dz = d2 * inrm;
        float Y[16];
        sh_basis_f(dx, dy, dz, Y);
        // colour = max(0, sum_k Y_k c_k + 1/2): a clamped channel passes nothing.  The
        // forward record holds the clamped colour, so "> 0" reads the clamp off it.
        const float4 rb = reinterpret_cast<const float4*>(rec + (size_t)i * GM_REC)[1];
        const float rc = rec[(size_t)i * GM_REC + 8];
        const float gacc[3] = {rb.z > 0.0f ? gr[6] : 0.0f, rb.w > 0.0f ? gr[7] : 0.0f, rc > 0.0f ? gr[8] : 0.0f};
        float gdx = 0.0f, gdy = 0.0f, gdz = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (k < K) {  // K is the same for every thread
                float gY = 0.0f;
#pragma unroll
                for (int ch = 0; ch < 3; ++ch) {
                    g_sh[((size_t)k * 3 + ch) * N + i] = listed ? Y[k] * gacc[ch] : 0.0f;
                    gY += shv[k * 3 + ch] * gacc[ch];
                }
                float ex, ey, ez;
                sh_basis_grad_f(k, dx, dy, dz, ex, ey, ez);
                gdx += gY * ex;
                gdy += gY * ey;
                gdz += gY * ez;
            }
        }
        // dir = d / |d|: d dir / d d = (I - dir dir^T) / |d|
        const float dd = dx * gdx + dy * gdy + dz * gdz;
        gmu[0] = (gdx - dx * dd) * inrm;
        gmu[1] = (gdy - dy * dd) * inrm;
        gmu[2] = (gdz - dz * dd) * inrm;
    }

    // ---- depth model and conic (fp64) -------------------------------------------------
    double gd[GM_GRAD];
#pragma unroll
    for (int k = 0; k < GM_GRAD; ++k) gd[k] = gr[k];
    const double gvar = clamp ? 0.0 : gd[12] / (2.0 * sig);
    const double gg0 = gd[10] - k0 * gvar, gg1 = gd[11] - k1 * gvar;
    const double gQ00 = gd[2] + gg0 * k0;
    const double gQ01 = gd[3] + gg0 * k1 + gg1 * k0;
    const double gQ11 = gd[4] + gg1 * k1;
    const double gk0 = -g0 * gvar + Q00 * gg0 + Q01 * gg1;
    const double gk1 = -g1 * gvar + Q01 * gg0 + Q11 * gg1;
    const double gSzz = gvar;
    // (Q00, Q01, Q11) = (c, -b, a) / det, det = a c - b^2
    const double id2 = idet * idet;
    const double ga = (-c * c * gQ00 + b * c * gQ01 - b * b * gQ11) * id2;
    const double gb = (2.0 * b * c * gQ00 - (det + 2.0 * b * b) * gQ01 + 2.0 * a * b * gQ11) * id2;
    const double gc = (-b * b * gQ00 + a * b * gQ01 - a * a * gQ11) * id2;

    // ---- Sigma_2D = J C J^T (+ eps), k = J C e_z, Szz = C_zz ---------------------------
    // H = gC + gC^T, the symmetric part of the gradient with respect to C
    double H[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int q = 0; q < 3; ++q)
            H[3 * r + q] = 2.0 * ga * J0[r] * J0[q] + gb * (J0[r] * J1[q] + J1[r] * J0[q]) + 2.0 * gc * J1[r] * J1[q];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const double e = gk0 * J0[r] + gk1 * J1[r];
        H[3 * r + 2] += e;
        H[6 + r] += e;
    }
    H[8] += 2.0 * gSzz;
    // Jacobian entries that vary: J00, J02 (row 0) and J11, J12 (row 1)
    const double gJ00 = 2.0 * ga * CJ0[0] + gb * CJ1[0] + gk0 * C[2];
    const double gJ02 = 2.0 * ga * CJ0[2] + gb * CJ1[2] + gk0 * C[8];
    const double gJ11 = gb * CJ0[1] + 2.0 * gc * CJ1[1] + gk1 * C[5];
    const double gJ12 = gb * CJ0[2] + 2.0 * gc * CJ1[2] + gk1 * C[8];
    const double iz2 = iz * iz, iz3 = iz2 * iz;
    const double gx = -gJ02 * fx * iz2 + gd[0] * fx * iz;
    const double gy = -gJ12 * fy * iz2 + gd[1] * fy * iz;
    const double gz = -gJ00 * fx * iz2 + 2.0 * gJ02 * fx * xc[0] * iz3 - gJ11 * fy * iz2 +
                      2.0 * gJ12 * fy * xc[1] * iz3 - gd[0] * fx * xc[0] * iz2 - gd[1] * fy * xc[1] * iz2 + gd[9];
    // x_c = W mean + t
#pragma unroll
    for (int j = 0; j < 3; ++j) gmu[j] += W[j] * gx + W[3 + j] * gy + W[6 + j] * gz;

    // ---- C = W M M^T W^T: gradient with respect to M is W^T H W M ---------------------
    double HW[9];  // H (W M)
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int q = 0; q < 3; ++q) HW[3 * r + q] = H[3 * r] * WM[q] + H[3 * r + 1] * WM[3 + q] + H[3 * r + 2] * WM[6 + q];
    double gM[9];  // W^T (H W M)
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int q = 0; q < 3; ++q) gM[3 * r + q] = W[r] * HW[q] + W[3 + r] * HW[3 + q] + W[6 + r] * HW[6 + q];
    // M = R diag(s)
    double gR[9], gs[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        gs[q] = gM[q] * R[q] + gM[3 + q] * R[3 + q] + gM[6 + q] * R[6 + q];
#pragma unroll
        for (int r = 0; r < 3; ++r) gR[3 * r + q] = gM[3 * r + q] * s[q];
    }
    // R of the unit quaternion (w, x, y, z), then the normalisation
    double gqh[4];
    gqh[0] = 2.0 * (-z * gR[1] + y * gR[2] + z * gR[3] - x * gR[5] - y * gR[6] + x * gR[7]);
    gqh[1] = 2.0 * (y * gR[1] + z * gR[2] + y * gR[3] - 2.0 * x * gR[4] - w * gR[5] + z * gR[6] + w * gR[7] -
                    2.0 * x * gR[8]);
    gqh[2] = 2.0 * (-2.0 * y * gR[0] + x * gR[1] + w * gR[2] + x * gR[3] + z * gR[5] - w * gR[6] + z * gR[7] -
                    2.0 * y * gR[8]);
    gqh[3] = 2.0 * (-2.0 * z * gR[0] - w * gR[1] + x * gR[2] + w * gR[3] - 2.0 * z * gR[4] + y * gR[5] +
                    x * gR[6] + y * gR[7]);
    const double dq = w * gqh[0] + x * gqh[1] + y * gqh[2] + z * gqh[3];
    const double qh[4] = {w, x, y, z};

#pragma unroll
    for (int j = 0; j < 3; ++j) g_means[(size_t)j * N + i] = listed ? (float)gmu[j] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) g_quats[(size_t)j * N + i] = listed ? (float)((gqh[j] - qh[j] * dq) * iqn) : 0.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) g_scales[(size_t)j * N + i] = listed ? (float)gs[j] : 0.0f;
    g_opacity[i] = gr[5];
    if (g_log_scales)  // scale = exp(log scale)
#pragma unroll
        for (int j = 0; j < 3; ++j) g_log_scales[(size_t)j * N + i] = listed ? (float)(gs[j] * s[j]) : 0.0f;
    if (g_logit) {  // opacity = sigmoid(logit)
        const float o = opacity[i];
        g_logit[i] = gr[5] * o * (1.0f - o);
    }
}

}  // namespace gm

using namespace gm;

extern "C" gm_status gm_project_gaussians_bwd(const gm_camera* cam, int32_t N, const float* means,
                                              const float* quats, const float* scales, const float* opacity,
                                              const float* sh, int32_t sh_degree, const float* rec,
                                              const float* g_rec, float* g_means, float* g_quats, float* g_scales,
                                              float* g_opacity, float* g_sh, float* g_log_scales,
                                              float* g_logit_opacity, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(sh_degree >= -1 && sh_degree <= 3, "sh_degree %d outside -1..3", sh_degree);
    if (N == 0) return GM_OK;
    GM_ARG_CHECK(means && quats && scales && sh && rec && g_rec, "an input is NULL");
    GM_ARG_CHECK(g_means && g_quats && g_scales && g_opacity && g_sh, "an output is NULL");
    GM_ARG_CHECK(opacity || !g_logit_opacity, "g_logit_opacity needs opacity");
    GM_ARG_CHECK(((uintptr_t)rec & 15) == 0, "rec must be 16-byte aligned");
    const DevCamera dc = dev_camera(*cam);
    k_project_bwd<<<(unsigned)div_up(N, 256), 256, 0, stream>>>(dc, N, means, quats, scales, opacity, sh, sh_degree,
                                                                rec, g_rec, g_means, g_quats, g_scales, g_opacity,
                                                                g_sh, g_log_scales, g_logit_opacity);
    GM_LAUNCH_CHECK();
    return GM_OK;
}
