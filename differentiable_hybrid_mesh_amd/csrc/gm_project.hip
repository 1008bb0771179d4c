// 3D Gaussian projection with the EWA conditional depth model and SH colour
// (gmesh README, "Design Details > Hybrid rendering": z*(p) = z_c + g.(p - mean2d),
// g = (Sigma_uv + eps I)^-1 Sigma_uv,z, sigma^2 = Sigma_zz - Sigma_z,uv g).
//
// The record fields that decide tile membership and order are evaluated in fp32 in
// a fixed order with no fused multiply-add and correctly rounded / and sqrt, so
// that every implementation of the same order gets the same bits.
#pragma clang fp contract(off)

#include <algorithm>

#include "gm_internal.h"
#include "gm_sh.h"

namespace gm {

constexpr float EPS2D = 0.3f;  // px^2: low-pass dilation, also the eps of the depth model

// World covariance Sigma = M M^T, M = R(q / |q|) diag(s): view independent.
struct WorldGauss {
    float mx, my, mz;
    float S[9];
    bool ok;  // |q| > 0
};

__device__ inline WorldGauss world_gaussian(int N, int i, const float* __restrict__ means,
                                            const float* __restrict__ quats, const float* __restrict__ scales)
{
    WorldGauss g;
    g.mx = means[i];
    g.my = means[N + i];
    g.mz = means[2 * N + i];
    float qw = quats[i], qx = quats[N + i], qy = quats[2 * N + i], qz = quats[3 * N + i];
    const float qq = ((qw * qw + qx * qx) + qy * qy) + qz * qz;
    g.ok = qq > 0.0f;
    const float qn = sqrtf(qq);
    qw = qw / qn;
    qx = qx / qn;
    qy = qy / qn;
    qz = qz / qn;
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
    const float s[3] = {scales[i], scales[N + i], scales[2 * N + i]};
    float M[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) M[r * 3 + c] = Rq[r * 3 + c] * s[c];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = r; c < 3; ++c) {
            const float v = (M[r * 3 + 0] * M[c * 3 + 0] + M[r * 3 + 1] * M[c * 3 + 1]) + M[r * 3 + 2] * M[c * 3 + 2];
            g.S[r * 3 + c] = v;
            g.S[c * 3 + r] = v;
        }
    return g;
}

// The record of Gaussian i in one view.  shc: its colour coefficients, read once by
// the caller ([k][3] for degree d >= 0, RGB for d = -1).
// Writes the record; returns its key for the depth sort: the bits of z_c when the
// Gaussian is listed (z_c > 0, so the bits order like the values), all ones otherwise.
__device__ inline uint32_t project_view(const DevCamera& cam, const WorldGauss& g, float opacity, const float* shc,
                                        int sh_degree, float* __restrict__ rec_i)
{
    const float* W = cam.R;
    const float mx = g.mx, my = g.my, mz = g.mz;
    const float xc = ((W[0] * mx + W[1] * my) + W[2] * mz) + cam.t[0];
    const float yc = ((W[3] * mx + W[4] * my) + W[5] * mz) + cam.t[1];
    const float zc = ((W[6] * mx + W[7] * my) + W[8] * mz) + cam.t[2];
    bool ok = zc >= cam.near_z && g.ok;
    const float* S = g.S;
    float A[9], C[9];  // Sigma_c = (W Sigma) W^T
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c)
            A[r * 3 + c] = (W[r * 3 + 0] * S[0 * 3 + c] + W[r * 3 + 1] * S[1 * 3 + c]) + W[r * 3 + 2] * S[2 * 3 + c];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = r; c < 3; ++c) {
            const float v = (A[r * 3 + 0] * W[c * 3 + 0] + A[r * 3 + 1] * W[c * 3 + 1]) + A[r * 3 + 2] * W[c * 3 + 2];
            C[r * 3 + c] = v;
            C[c * 3 + r] = v;
        }
    // pinhole Jacobian at the mean (no frustum clamp)
    const float z2 = zc * zc;
    const float J00 = cam.fx / zc;
    const float J02 = -(cam.fx * xc) / z2;
    const float J11 = cam.fy / zc;
    const float J12 = -(cam.fy * yc) / z2;
    float T0[3], T1[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        T0[c] = J00 * C[0 * 3 + c] + J02 * C[2 * 3 + c];
        T1[c] = J11 * C[1 * 3 + c] + J12 * C[2 * 3 + c];
    }
    const float S00 = T0[0] * J00 + T0[2] * J02;
    const float S01 = T0[1] * J11 + T0[2] * J12;
    const float S11 = T1[1] * J11 + T1[2] * J12;
    const float k0 = T0[2], k1 = T1[2], Szz = C[8];
    const float a = S00 + EPS2D, b = S01, c = S11 + EPS2D;
    const float det = a * c - b * b;
    if (!(det > 0.0f)) ok = false;
    const float Q00 = c / det, Q01 = (-b) / det, Q11 = a / det;
    const float g0 = Q00 * k0 + Q01 * k1;
    const float g1 = Q01 * k0 + Q11 * k1;
    const float var = Szz - (k0 * g0 + k1 * g1);
    const float sig = sqrtf(var > 1e-12f ? var : 1e-12f);
    const float u = (cam.fx * xc) / zc + cam.cx;
    const float v = (cam.fy * yc) / zc + cam.cy;
    // tile rect: the box of the 3-sigma ellipse of the dilated 2D covariance, whose
    // half-widths along x and y are 3 sqrt(a) and 3 sqrt(c), rounded up to pixels
    const float radx = ceilf(3.0f * sqrtf(a));
    const float rady = ceilf(3.0f * sqrtf(c));
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    if (ok) {
        float fx0 = floorf((u - radx) / 16.0f), fx1 = ceilf((u + radx) / 16.0f);
        float fy0 = floorf((v - rady) / 16.0f), fy1 = ceilf((v + rady) / 16.0f);
        fx0 = fminf(fmaxf(fx0, 0.0f), (float)cam.tx);
        fx1 = fminf(fmaxf(fx1, 0.0f), (float)cam.tx);
        fy0 = fminf(fmaxf(fy0, 0.0f), (float)cam.ty);
        fy1 = fminf(fmaxf(fy1, 0.0f), (float)cam.ty);
        r0 = (int)fx0;
        r1 = (int)fy0;
        r2 = (int)fx1;
        r3 = (int)fy1;
        if (r0 >= r2 || r1 >= r3) r0 = r1 = r2 = r3 = 0;
    }
    const int ntiles = (r2 - r0) * (r3 - r1);

    // colour (value arithmetic, fp32)
    float col[3];
    if (sh_degree < 0) {
        col[0] = shc[0];
        col[1] = shc[1];
        col[2] = shc[2];
    } else {
        float cw[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) cw[j] = -(W[j] * cam.t[0] + W[3 + j] * cam.t[1] + W[6 + j] * cam.t[2]);
        float dx = mx - cw[0], dy = my - cw[1], dz = mz - cw[2];
        const float nrm = sqrtf(dx * dx + dy * dy + dz * dz);
        dx /= nrm;
        dy /= nrm;
        dz /= nrm;
        float Y[16];
        sh_basis_f(dx, dy, dz, Y);
        const int K = (sh_degree + 1) * (sh_degree + 1);
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (k < K) acc += Y[k] * shc[k * 3 + ch];
            acc += 0.5f;
            col[ch] = acc > 0.0f ? acc : 0.0f;
        }
    }
    float4* o = reinterpret_cast<float4*>(rec_i);
    o[0] = make_float4(u, v, Q00, Q01);
    o[1] = make_float4(Q11, opacity, col[0], col[1]);
    o[2] = make_float4(col[2], zc, g0, g1);
    o[3] = make_float4(sig, __int_as_float(r0 | (r1 << 16)), __int_as_float(r2 | (r3 << 16)),
                       __int_as_float(ntiles));
    return ntiles > 0 ? __float_as_uint(zc) : 0xffffffffu;
}

__device__ inline void load_colour(int N, int i, const float* __restrict__ sh, int sh_degree, float* shc)
{
    const int K = sh_degree < 0 ? 1 : (sh_degree + 1) * (sh_degree + 1);
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) shc[k * 3 + ch] = k < K ? sh[((size_t)k * 3 + ch) * N + i] : 0.0f;
}

// KEYS: also the depth sort's input (key and id of every Gaussian, and the key
// count), which the sort otherwise extracts from the records in a kernel of its own.
template <bool KEYS>
__global__ void __launch_bounds__(256)
k_project_gaussians(DevCamera cam, int N, const float* __restrict__ means,
                    const float* __restrict__ quats, const float* __restrict__ scales,
                    const float* __restrict__ opacity, const float* __restrict__ sh, int sh_degree,
                    float* __restrict__ rec, uint32_t* __restrict__ keys = nullptr, int32_t* __restrict__ ids = nullptr,
                    long long* __restrict__ d_n = nullptr)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (KEYS && i == 0) *d_n = N;
    if (i >= N) return;
    const WorldGauss g = world_gaussian(N, i, means, quats, scales);
    float shc[48];
    load_colour(N, i, sh, sh_degree, shc);
    const uint32_t key = project_view(cam, g, opacity[i], shc, sh_degree, rec + (size_t)i * GM_REC);
    if constexpr (KEYS) {
        keys[i] = key;
        ids[i] = i;
    }
}

gm_status check_project_args(const gm_camera* cam, int32_t N, const float* means, const float* quats,
                             const float* scales, const float* opacity, const float* sh, int32_t sh_degree,
                             const float* rec)
{
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(sh_degree >= -1 && sh_degree <= 3, "sh_degree %d outside -1..3", sh_degree);
    if (N == 0) return GM_OK;
    GM_ARG_CHECK(means && quats && scales && opacity && sh && rec, "an input or rec is NULL");
    GM_ARG_CHECK(((uintptr_t)rec & 15) == 0, "rec must be 16-byte aligned");
    return GM_OK;
}

gm_status launch_project_keys(const DevCamera& dc, int32_t N, const float* means, const float* quats,
                              const float* scales, const float* opacity, const float* sh, int32_t sh_degree,
                              float* rec, uint32_t* keys, int32_t* ids, long long* d_n, hipStream_t stream)
{
    k_project_gaussians<true><<<(unsigned)div_up(N, 256), 256, 0, stream>>>(dc, N, means, quats, scales, opacity, sh,
                                                                            sh_degree, rec, keys, ids, d_n);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

// Several views of the same Gaussians: the inputs are read and the world covariance
// formed once, then every view's record is written ([view][N][GM_REC]).  Each view's
// record is computed by the same code as the single-view kernel, so it is bitwise
// the same.
constexpr int PROJ_MAX_VIEWS = 16;
struct ViewSet {
    DevCamera cam[PROJ_MAX_VIEWS];
};

__global__ void __launch_bounds__(256)
k_project_gaussians_multi(ViewSet views, int nviews, int N, const float* __restrict__ means,
                          const float* __restrict__ quats, const float* __restrict__ scales,
                          const float* __restrict__ opacity, const float* __restrict__ sh, int sh_degree,
                          float* __restrict__ rec)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const WorldGauss g = world_gaussian(N, i, means, quats, scales);
    float shc[48];
    load_colour(N, i, sh, sh_degree, shc);
    const float o = opacity[i];
    for (int v = 0; v < nviews; ++v)
        project_view(views.cam[v], g, o, shc, sh_degree, rec + ((size_t)v * N + i) * GM_REC);
}

}  // namespace gm

using namespace gm;

extern "C" gm_status gm_project_gaussians(const gm_camera* cam, int32_t N, const float* means,
                                          const float* quats, const float* scales,
                                          const float* opacity, const float* sh, int32_t sh_degree,
                                          float* rec, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_project_args(cam, N, means, quats, scales, opacity, sh, sh_degree, rec)) return s;
    if (N == 0) return GM_OK;
    const DevCamera dc = dev_camera(*cam);
    k_project_gaussians<false><<<(unsigned)div_up(N, 256), 256, 0, stream>>>(dc, N, means, quats, scales, opacity,
                                                                             sh, sh_degree, rec);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

extern "C" gm_status gm_project_gaussians_multi(const gm_camera* cams, int32_t nviews, int32_t N, const float* means,
                                                const float* quats, const float* scales, const float* opacity,
                                                const float* sh, int32_t sh_degree, float* rec, hipStream_t stream)
{
    clear_error();
    GM_ARG_CHECK(cams != nullptr && nviews >= 0, "cams is NULL or nviews negative");
    for (int v = 0; v < nviews; ++v)
        if (gm_status s = check_camera(&cams[v])) return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(sh_degree >= -1 && sh_degree <= 3, "sh_degree %d outside -1..3", sh_degree);
    if (N == 0 || nviews == 0) return GM_OK;
    GM_ARG_CHECK(means && quats && scales && opacity && sh && rec, "an input or rec is NULL");
    GM_ARG_CHECK(((uintptr_t)rec & 15) == 0, "rec must be 16-byte aligned");
    for (int v0 = 0; v0 < nviews; v0 += PROJ_MAX_VIEWS) {
        const int nv = std::min(PROJ_MAX_VIEWS, nviews - v0);
        ViewSet vs{};
        for (int v = 0; v < nv; ++v) vs.cam[v] = dev_camera(cams[v0 + v]);
        k_project_gaussians_multi<<<(unsigned)div_up(N, 256), 256, 0, stream>>>(
            vs, nv, N, means, quats, scales, opacity, sh, sh_degree, rec + (size_t)v0 * N * GM_REC);
        GM_LAUNCH_CHECK();
    }
    return GM_OK;
}
