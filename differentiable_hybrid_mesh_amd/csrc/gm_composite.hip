// Hybrid compositing, forward and backward (gmesh README, "Design Details > Hybrid
// rendering"), with the mesh surface resolve of "Mesh rasterizer" step 2 and the
// v1.1 texture and lighting notes as its prologue.
//
// One 256-thread block per 16x16 tile, one thread per pixel, each wave an 8x8
// quadrant (the most compact 64-pixel footprint).  Records of the tile's
// list are staged in LDS in batches of 256 (64 bytes each, read by all lanes at the
// same address: an LDS broadcast).  The forward walks front to back with a
// tile-level early exit; the backward walks back to front from the last entry any
// pixel of the tile used, recovering the transmittance by division, reduces the 13
// per-Gaussian gradients over each wave with shuffles into LDS accumulators, and
// flushes one float atomic per (tile, Gaussian, field).
//
// The per-pair arithmetic is one inline function shared by both kernels and built
// without contraction, so the forward and the backward take the same skip and stop
// decisions bit for bit.
#pragma clang fp contract(off)

#include <mutex>
#include <type_traits>

#include "gm_internal.h"

namespace gm {

constexpr int CT = 256;     // threads per block = pixels per tile
constexpr int CBF = 256;    // records per LDS batch of the forward (<= CT, a multiple of 64)
constexpr int CBB = 192;    // records per LDS batch of the backward (<= CT, a multiple of 32): 24 KB of
                            // LDS per block, six blocks per CU (five at 256: 0.550 -> 0.509 ms at C3)
constexpr float SKIP_ALPHA = 1.0f / 255.0f;
constexpr float STOP_T = 1e-4f;
constexpr float ALPHA_MAX = 0.99f;
constexpr int NBASIS = 14;  // per-entry basis sums accumulated by the backward

struct CompParams {
    DevCamera cam;
    const float* rec;
    const int32_t* ranges;
    const int32_t* ids;
    const int32_t* face_id;
    const float* depth;
    // mesh surface
    int V, F, Vt, tex_size, nlev;
    const float* vscreen;
    const int32_t* faces;
    const float* vcolor;
    const float* vnormal;
    const float* uv;
    const int32_t* faces_uv;
    const float* mips;
    int lit;
    float lpos[3], lamb[3], ldif[3], lspec[3], lshin;
    float bg[3];
    float softness;
};

// ---------------------------------------------------------------------------
// mesh surface colour c_m at a covered pixel
// ---------------------------------------------------------------------------
__device__ inline void bilinear_tex(const float* __restrict__ lvl, int s, float u, float v, float* out)
{
    u = fminf(fmaxf(u, 0.0f), 1.0f);
    v = fminf(fmaxf(v, 0.0f), 1.0f);
    const float x = u * (float)s - 0.5f, y = v * (float)s - 0.5f;
    const float x0 = floorf(x), y0 = floorf(y);
    const float ax = x - x0, ay = y - y0;
    int ix0 = (int)x0, iy0 = (int)y0;
    int ix1 = min(max(ix0 + 1, 0), s - 1), iy1 = min(max(iy0 + 1, 0), s - 1);
    ix0 = min(max(ix0, 0), s - 1);
    iy0 = min(max(iy0, 0), s - 1);
    const float* p00 = lvl + ((size_t)iy0 * s + ix0) * 3;
    const float* p01 = lvl + ((size_t)iy0 * s + ix1) * 3;
    const float* p10 = lvl + ((size_t)iy1 * s + ix0) * 3;
    const float* p11 = lvl + ((size_t)iy1 * s + ix1) * 3;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const float top = p00[c] + (p01[c] - p00[c]) * ax;
        const float bot = p10[c] + (p11[c] - p10[c]) * ax;
        out[c] = top + (bot - top) * ay;
    }
}

__device__ void surface_color(const CompParams& P, int f, int px, int py, float* cm)
{
    const int V = P.V, F = P.F;
    const float* vs = P.vscreen;
    int vi[3];
    double u[3], v[3], z[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        vi[k] = P.faces[k * F + f];
        u[k] = (double)vs[vi[k]];
        v[k] = (double)vs[V + vi[k]];
        z[k] = (double)vs[2 * V + vi[k]];
    }
    const double pu = px + 0.5, pv = py + 0.5;
    const double A = (u[1] - u[0]) * (v[2] - v[0]) - (v[1] - v[0]) * (u[2] - u[0]);
    const double E[3] = {(u[2] - u[1]) * (pv - v[1]) - (v[2] - v[1]) * (pu - u[1]),
                         (u[0] - u[2]) * (pv - v[2]) - (v[0] - v[2]) * (pu - u[2]),
                         (u[1] - u[0]) * (pv - v[0]) - (v[1] - v[0]) * (pu - u[0])};
    double lam[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) lam[k] = E[k] / A;
    const double zz = 1.0 / ((lam[0] / z[0] + lam[1] / z[1]) + lam[2] / z[2]);
    float b[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) b[k] = (float)(lam[k] / z[k] * zz);

    float base[3] = {0.0f, 0.0f, 0.0f};
    if (P.mips && P.uv) {
        float uvk[3][2];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int ti = P.faces_uv[k * F + f];
            uvk[k][0] = P.uv[ti];
            uvk[k][1] = P.uv[P.Vt + ti];
        }
        const float uu = b[0] * uvk[0][0] + b[1] * uvk[1][0] + b[2] * uvk[2][0];
        const float vv = b[0] * uvk[0][1] + b[1] * uvk[1][1] + b[2] * uvk[2][1];
        // analytic screen derivatives of the perspective-correct uv (quotient rule)
        const int ea[3] = {1, 2, 0}, eb[3] = {2, 0, 1};
        double W = 0.0, dwx[3], dwy[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            W += lam[k] / z[k];
            dwx[k] = (-(v[eb[k]] - v[ea[k]]) / A) / z[k];
            dwy[k] = ((u[eb[k]] - u[ea[k]]) / A) / z[k];
        }
        float dux = 0.f, dvx = 0.f, duy = 0.f, dvy = 0.f;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const float ax = (float)(dwx[k] / W), ay = (float)(dwy[k] / W);
            dux += ax * (uvk[k][0] - uu);
            dvx += ax * (uvk[k][1] - vv);
            duy += ay * (uvk[k][0] - uu);
            dvy += ay * (uvk[k][1] - vv);
        }
        const float S0 = (float)P.tex_size;
        const float lx = sqrtf((S0 * dux) * (S0 * dux) + (S0 * dvx) * (S0 * dvx));
        const float ly = sqrtf((S0 * duy) * (S0 * duy) + (S0 * dvy) * (S0 * dvy));
        const float rho = fmaxf(lx, ly);
        const float lmax = (float)(P.nlev - 1);
        float lod = rho > 0.0f ? log2f(rho) : 0.0f;
        lod = fminf(fmaxf(lod, 0.0f), lmax);
        const int l0 = (int)floorf(lod);
        const int l1 = min(l0 + 1, P.nlev - 1);
        const float tl = lod - (float)l0;
        size_t o0 = 0, o1 = 0, o = 0;
        for (int l = 0; l < P.nlev; ++l) {
            if (l == l0) o0 = o;
            if (l == l1) o1 = o;
            const size_t s = (size_t)(P.tex_size >> l);
            o += s * s * 3;
        }
        float c0[3], c1[3];
        bilinear_tex(P.mips + o0, P.tex_size >> l0, uu, vv, c0);
        bilinear_tex(P.mips + o1, P.tex_size >> l1, uu, vv, c1);
#pragma unroll
        for (int c = 0; c < 3; ++c) base[c] = c0[c] + (c1[c] - c0[c]) * tl;
    } else if (P.vcolor) {
#pragma unroll
        for (int c = 0; c < 3; ++c)
            base[c] = b[0] * P.vcolor[c * V + vi[0]] + b[1] * P.vcolor[c * V + vi[1]] + b[2] * P.vcolor[c * V + vi[2]];
    }
    if (P.lit && P.vnormal) {
        const float* R = P.cam.R;
        float nw[3];
#pragma unroll
        for (int c = 0; c < 3; ++c)
            nw[c] = b[0] * P.vnormal[c * V + vi[0]] + b[1] * P.vnormal[c * V + vi[1]] + b[2] * P.vnormal[c * V + vi[2]];
        float n[3], L[3], x[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            n[r] = R[r * 3 + 0] * nw[0] + R[r * 3 + 1] * nw[1] + R[r * 3 + 2] * nw[2];
            L[r] = R[r * 3 + 0] * P.lpos[0] + R[r * 3 + 1] * P.lpos[1] + R[r * 3 + 2] * P.lpos[2] + P.cam.t[r];
        }
        const float zf = (float)zz;
        x[0] = ((float)pu - P.cam.cx) / P.cam.fx * zf;
        x[1] = ((float)pv - P.cam.cy) / P.cam.fy * zf;
        x[2] = zf;
        float l[3] = {L[0] - x[0], L[1] - x[1], L[2] - x[2]};
        float e[3] = {-x[0], -x[1], -x[2]};
        const float in = 1.0f / sqrtf(n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);
        const float il = 1.0f / sqrtf(l[0] * l[0] + l[1] * l[1] + l[2] * l[2]);
        const float ie = 1.0f / sqrtf(e[0] * e[0] + e[1] * e[1] + e[2] * e[2]);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            n[r] *= in;
            l[r] *= il;
            e[r] *= ie;
        }
        const float ndl = n[0] * l[0] + n[1] * l[1] + n[2] * l[2];
        const float rde = (2.0f * ndl * n[0] - l[0]) * e[0] + (2.0f * ndl * n[1] - l[1]) * e[1] +
                          (2.0f * ndl * n[2] - l[2]) * e[2];
        const float diff = fmaxf(ndl, 0.0f);
        const float spec = (ndl > 0.0f && rde > 0.0f) ? powf(rde, P.lshin) : 0.0f;
#pragma unroll
        for (int c = 0; c < 3; ++c) cm[c] = base[c] * (P.lamb[c] + P.ldif[c] * diff) + P.lspec[c] * spec;
    } else {
#pragma unroll
        for (int c = 0; c < 3; ++c) cm[c] = base[c];
    }
}

// ---------------------------------------------------------------------------
// surface colour prepass: state_cm = c_m on the mesh, bg elsewhere
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_shade(CompParams P, float* __restrict__ state_cm)
{
    const int pix = blockIdx.x * blockDim.x + threadIdx.x;
    if (pix >= P.cam.width * P.cam.height) return;
    const int fid = P.face_id[pix];
    float cm[3] = {P.bg[0], P.bg[1], P.bg[2]};
    if (fid >= 0) surface_color(P, fid, pix % P.cam.width, pix / P.cam.width, cm);
    state_cm[3 * pix + 0] = cm[0];
    state_cm[3 * pix + 1] = cm[1];
    state_cm[3 * pix + 2] = cm[2];
}

// ---------------------------------------------------------------------------
// the per-pair evaluation shared by both walks
// ---------------------------------------------------------------------------
struct Staged {
    float4 a;  // u, v, l0, l1 (Cholesky factor of Q / 2, see conic_cholesky)
    float4 b;  // l2, opacity, r, g
    float4 c;  // b, z_c, g0, g1
    float4 d;  // sigma, kappa = 1/(sigma softness), q_skip, 1/sigma
};

// q = (Q00 dx^2 + 2 Q01 dx dy + Q11 dy^2) / 2 from the half-conic (hq00, q01, hq11).
__device__ __forceinline__ float quad_form(float hq00, float q01, float hq11, float dx, float dy)
{
    return __builtin_fmaf(dx, __builtin_fmaf(hq00, dx, q01 * dy), (hq11 * dy) * dy);
}

// The same q from the Cholesky factor of Q / 2 = L L^T, L = [[l0, 0], [l1, l2]]:
// q = |L^T d|^2 = (l0 dx + l1 dy)^2 + (l2 dy)^2, a sum of two squares.  For a
// Gaussian that is long and thin on screen the three terms of the expanded form
// cancel, and in fp32 their rounding grows with the conic's condition number (up to
// 4e-4 in q, i.e. in log alpha, at 100-200 px offsets in the 1080p four-sphere
// scene); the squares' error grows only with its square root.  Five operations, as
// for the expanded form.
__device__ __forceinline__ float chol_form(float l0, float l1, float l2, float dx, float dy)
{
    const float t1 = __builtin_fmaf(l0, dx, l1 * dy);
    const float t2 = l2 * dy;
    return __builtin_fmaf(t1, t1, t2 * t2);
}

// Cholesky factor of Q / 2 from the conic (Q00 > 0 on a listed record): l0 =
// sqrt(Q00 / 2), l1 = (Q01 / 2) / l0, l2 = sqrt(det Q / (2 Q00)).  det Q = Q00 Q11 -
// Q01^2 is formed with the exact error of the product Q01^2 (Kahan's difference of
// products), so it keeps its relative accuracy when the two products nearly cancel.
__device__ __forceinline__ void conic_cholesky(float Q00, float Q01, float Q11, float& l0, float& l1, float& l2)
{
    const float p = Q01 * Q01;
    const float e = __builtin_fmaf(Q01, Q01, -p);
    const float det = fmaxf(__builtin_fmaf(Q00, Q11, -p) - e, 0.0f);
    l0 = sqrtf(0.5f * Q00);
    l1 = l0 > 0.0f ? (0.5f * Q01) / l0 : 0.0f;
    l2 = Q00 > 0.0f ? sqrtf((0.5f * det) / Q00) : 0.0f;
}

// Standard normal CDF Phi(s) and density phi(s) from one exponential.
// erfc(z) for z >= 0 follows Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error| <= 1.5e-7): erfc(z) = t P(t) exp(-z^2),
// t = 1 / (1 + p z).  With z = |s| / sqrt(2), exp(-z^2) = exp(-s^2 / 2), which is
// also what phi needs, so the backward gets both for the price of one exp.
__device__ __forceinline__ float normal_cdf_pdf(float s, float& pdf, float& comp)
{
    const float e = __expf(-0.5f * s * s);
    pdf = 0.39894228040143268f * e;
    const float z = fabsf(s) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
    float poly = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
    poly = __builtin_fmaf(t, poly, 1.421413741f);
    poly = __builtin_fmaf(t, poly, -0.284496736f);
    poly = __builtin_fmaf(t, poly, 0.254829592f);
    poly *= t;
    const float half_tail = 0.5f * poly * e;  // Phi(-|s|)
    comp = s <= 0.0f ? 1.0f - half_tail : half_tail;  // 1 - Phi(s), without cancellation
    return s <= 0.0f ? half_tail : 1.0f - half_tail;
}

// One (pixel, entry) pair, straight-line (an entry that passed its wave's mask is
// live for most lanes, so branching would only serialise both paths):
// alpha = min(0.99, o exp(-q)), split f = Phi((D - z*) / (sigma softness)) on the
// mesh (1 off it), alpha_F = alpha f.  The pair is included when q <= q_skip (a
// pair above it is below the 1/255 threshold with margin), alpha >= 1/255 and
// alpha_F >= 1/255.  Both walks call this one function, so the forward and the
// backward take the same decisions bit for bit.
struct Pair {
    float dx, dy, q, oG, al, f, fb, pdf, s, aF;  // fb = 1 - f (the back share)
    bool ok;  // passes the skip rules of the front layer
};

__device__ __forceinline__ Pair eval_pair(const Staged& g, float pxc, float pyc, bool on, bool wave_on, float D,
                                          float softness)
{
    Pair p;
    p.dx = pxc - g.a.x;
    p.dy = pyc - g.a.y;
    p.q = chol_form(g.a.z, g.a.w, g.b.x, p.dx, p.dy);
    p.oG = g.b.y * __expf(-p.q);
    p.al = fminf(p.oG, ALPHA_MAX);
    p.f = 1.0f;
    p.fb = 0.0f;
    p.pdf = 0.0f;
    p.s = 0.0f;
    if (wave_on) {  // uniform: some pixel of the wave is on the mesh
        const float num = (D - g.c.y) - __builtin_fmaf(g.c.z, p.dx, g.c.w * p.dy);
        if (softness > 0.0f) {
            p.s = on ? num * g.d.y : 0.0f;  // off the mesh D = +inf: keep s finite
            if ((__ballot(on) & __ballot(fabsf(p.s) <= 6.0f)) != 0ull) {  // scalar masks (see the backward's entry skip)
                float pd, fc;
                const float fo = normal_cdf_pdf(p.s, pd, fc);
                p.f = on ? fo : 1.0f;
                p.fb = on ? fc : 0.0f;
                p.pdf = on ? pd : 0.0f;
            } else {
                // every lane of the wave is off the mesh or has |s| > 6: there the
                // tail Phi(-|s|) <= exp(-18)/2 < 2^-25, so the evaluation above gives
                // exactly 1 for the larger share and, for the smaller one, a value
                // whose product with alpha is far below the 1/255 skip threshold; the
                // same decisions and, with the density computed as above, the same
                // gradients, without the erfc polynomial
                const bool behind = on && !(p.s > 0.0f);
                p.f = behind ? 0.0f : 1.0f;
                p.fb = behind ? 1.0f : 0.0f;
                p.pdf = on ? 0.39894228040143268f * __expf(-0.5f * p.s * p.s) : 0.0f;
            }
        } else {
            const bool behind = on && !(num > 0.0f);
            p.f = behind ? 0.0f : 1.0f;
            p.fb = behind ? 1.0f : 0.0f;
        }
    }
    p.aF = p.al * p.f;
    p.ok = !(p.q > g.d.z) & (p.al >= SKIP_ALPHA) & (p.aF >= SKIP_ALPHA);
    return p;
}

// Minimum of q over the rectangle [xa, xb] x [ya, yb] of offsets (dx, dy): zero
// when the rectangle holds the centre, else the least of the four edge minima (q
// is convex; on an edge it is a 1D quadratic minimised at a clamped stationary point).
__device__ __forceinline__ float quad_min_rect(float hq00, float q01, float hq11, float xa, float xb, float ya,
                                               float yb)
{
    if (xa <= 0.0f && xb >= 0.0f && ya <= 0.0f && yb >= 0.0f) return 0.0f;
    float m = INFINITY;
    const float ix = -q01 / (2.0f * hq11), iy = -q01 / (2.0f * hq00);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float X = e ? xb : xa;
        const float Y = fminf(fmaxf(ix * X, ya), yb);
        m = fminf(m, quad_form(hq00, q01, hq11, X, Y));
        const float Y2 = e ? yb : ya;
        const float X2 = fminf(fmaxf(iy * Y2, xa), xb);
        m = fminf(m, quad_form(hq00, q01, hq11, X2, Y2));
    }
    return m;
}

// Stage one record and decide for which of the tile's four 8x8-pixel waves it can
// matter.  A wave bit is cleared only when every pixel of the wave would skip the
// entry anyway (alpha_F < 1/255), so skipping it leaves every result bit-identical:
//  * q exceeds q_skip on the whole rectangle of the wave's pixel centres, with a
//    margin that covers fp32 rounding of q scaled by the conic's conditioning; or
//  * the wave lies entirely on the mesh (wdmax = max D over its pixels) and the
//    conditional depth, minimal at a corner of the wave's rectangle, keeps f small
//    enough that min(0.99, o) f < (1/255)(1 - 1e-3), with a 1e-5 |D| depth slack.
__device__ __forceinline__ uint32_t stage_record(const CompParams& P, float4 ra, float4 rb, float4 rc,
                                                 float4 rd, int tx, int ty, const float* wdmax, Staged& st)
{
    const float Q00 = ra.z, Q01 = ra.w, Q11 = rb.x;
    float l0, l1, l2;
    conic_cholesky(Q00, Q01, Q11, l0, l1, l2);
    st.a = make_float4(ra.x, ra.y, l0, l1);
    st.b = make_float4(l2, rb.y, rb.z, rb.w);
    st.c = rc;
    const float o = rb.y;
    const float lq = o > 0.0f ? logf(255.0f * o) : -1.0f;
    const float qs = o > 0.0f ? lq + 1e-4f + 1e-4f * fabsf(lq) : -1.0f;
    const float kap = P.softness > 0.0f ? 1.0f / (rd.x * P.softness) : 0.0f;
    st.d = make_float4(rd.x, kap, qs, 1.0f / rd.x);
    if (!(qs >= 0.0f)) return 0u;  // o exp(-q) < 1/255 everywhere
    const float detQ = Q00 * Q11 - Q01 * Q01;
    if (!(detQ > 0.0f) || !(Q00 > 0.0f) || !(Q11 > 0.0f)) return 0xFu;
    const float rho = fminf(fabsf(Q01) / sqrtf(Q00 * Q11), 0.999999f);
    const float qe = qs * (1.0f + 1e-5f * (1.0f + rho) / (1.0f - rho)) + 1e-4f;
    const float u = ra.x, v = ra.y;
    const float amax = fminf(o, ALPHA_MAX);
    const float thr = (1.0f / 255.0f) * (1.0f - 1e-3f);
    // f must reach thr/amax somewhere for the entry to matter
    const float scrit = P.softness > 0.0f && amax > thr ? -1.41421356237309515f * erfcinvf(2.0f * thr / amax) - 1e-3f
                                                         : 0.0f;
    const float g0 = rc.z, g1 = rc.w, zc = rc.y;
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // wave w covers the 8x8 pixel quadrant (w & 1, w >> 1) of the tile
        const float xa = (float)(tx * GM_TILE + 8 * (w & 1)) + 0.5f - u, xb = xa + 7.0f;
        const float ya = (float)(ty * GM_TILE + 8 * (w >> 1)) + 0.5f - v, yb = ya + 7.0f;
        const float gxm = fminf(g0 * xa, g0 * xb);
        const float dm = wdmax[w];
        if (dm < 0.0f) continue;  // no pixel of this wave is in the image
        if (quad_min_rect(0.5f * Q00, Q01, 0.5f * Q11, xa, xb, ya, yb) * (1.0f - 1e-5f) > qe) continue;
        if (dm < INFINITY) {
            const float zmin = zc + (gxm + fminf(g1 * ya, g1 * yb));
            const float lim = dm + 1e-5f * fabsf(dm);
            if (P.softness > 0.0f) {
                if (amax <= thr) continue;
                if ((lim - zmin) * kap < scrit) continue;
            } else if (zmin >= lim) {
                continue;
            }
        }
        m |= 1u << w;
    }
    return m;
}

__device__ __forceinline__ void load_record(const float* __restrict__ rec, int id, float4& ra, float4& rb,
                                            float4& rc, float4& rd)
{
    const float4* r = reinterpret_cast<const float4*>(rec + (size_t)id * GM_REC);
    ra = r[0];
    rb = r[1];
    rc = r[2];
    rd = r[3];
}

// Per-wave max mesh depth: +inf when a pixel of the wave is off the mesh, -1 when no
// pixel of the wave is in the image.
__device__ __forceinline__ void wave_dmax(bool inside, bool on, float D, float* s_wd)
{
    float m = inside ? (on ? D : INFINITY) : -1.0f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) s_wd[threadIdx.x >> 6] = m;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// AA = false: binary mesh coverage from the z-buffer; the back layer is inert
// (off the mesh f = 1, on it the weight 1 - a_m = 0), so only the front layer is
// composited: C = C_F + T_F c_m (c_m = bg off the mesh).
// AA = true: the antialiased mesh layer (premultiplied colour M and depth M_D,
// coverage a_m, split depth D) and the general two-layer form
// C = C_F + T_F (M + (1 - a_m)(C_B + T_B bg)); the back layer is composited where
// it is visible (a_m < 1, finite D), with the same per-layer rules, and stops when
// the front layer stops (the 3DGS stop is per pixel; the back layer is seen only
// through T_F).
struct AaLayer {
    float M0, M1, M2, MD, am, D;
};

__device__ __forceinline__ AaLayer load_layer(const float* __restrict__ layer, int pix)
{
    const float4 l0 = reinterpret_cast<const float4*>(layer)[2 * pix];
    const float4 l1 = reinterpret_cast<const float4*>(layer)[2 * pix + 1];
    return AaLayer{l0.x, l0.y, l0.z, l0.w, l1.x, l1.y};
}

// STATS = true (a measurement build of the same kernel): adds to stats[0] the
// included (pixel, entry) pairs, to stats[1] the entries the waves evaluate (each
// wave-wide evaluation of one entry counts once) and to stats[2] the list entries
// staged; the outputs are those of STATS = false.
template <bool AA, bool STATS = false>
__global__ void __launch_bounds__(CT)
k_composite_fwd(CompParams P, const float* __restrict__ state_cm, const float* __restrict__ layer,
                float* __restrict__ out_rgb, float* __restrict__ out_depth, float* __restrict__ out_alpha,
                float* __restrict__ state_T, int32_t* __restrict__ state_last, float* __restrict__ state_aa,
                unsigned long long* __restrict__ stats = nullptr)
{
    __shared__ Staged s_g[CBF];
    __shared__ uint8_t s_m[CBF];
    __shared__ float s_wd[CT / 64];
    const int tile = blockIdx.x;
    const int tx = tile % P.cam.tx, ty = tile / P.cam.tx;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int px = tx * GM_TILE + 8 * (wave & 1) + (lane & 7), py = ty * GM_TILE + 8 * (wave >> 1) + (lane >> 3);
    const bool inside = px < P.cam.width && py < P.cam.height;
    const int pix = py * P.cam.width + px;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const int start = P.ranges[2 * tile], end = P.ranges[2 * tile + 1];

    bool on;
    float D;
    AaLayer ml{};
    if constexpr (AA) {
        ml = inside ? load_layer(layer, pix) : AaLayer{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, INFINITY};
        D = ml.D;
        on = D < INFINITY;
        // the wave's depth bound only counts pixels the mesh covers completely
        wave_dmax(inside, on && ml.am >= 1.0f, D, s_wd);
    } else {
        const int fid = inside ? P.face_id[pix] : -1;
        on = fid >= 0;
        D = on ? P.depth[pix] : INFINITY;
        wave_dmax(inside, on, D, s_wd);
    }
    const bool wave_on = __ballot(on) != 0;

    // one layer: a pixel that has stopped (or lies outside the image) carries -T, so
    // the sign of T is its done flag and the walk needs no separate one (T >= 1e-4
    // while it runs; the stopping entry is not taken, so |T| is the final value)
    float T = AA || inside ? 1.0f : -1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f, Z = 0.0f;
    int last = 0;
    bool done = !inside;  // two layers only
    // back layer (AA only)
    float TB = 1.0f, B0 = 0.0f, B1 = 0.0f, B2 = 0.0f, ZB = 0.0f;
    int lastB = 0;
    bool doneB = true;
    if constexpr (AA) doneB = !(inside && on && ml.am < 1.0f);
    int ninc = 0, nev = 0, nst = 0;  // STATS only
    float4 ra, rb, rc, rd;
    if ((int)threadIdx.x < CBF && start + (int)threadIdx.x < end)
        load_record(P.rec, P.ids[start + threadIdx.x], ra, rb, rc, rd);
    for (int b0 = start; b0 < end; b0 += CBF) {
        if (__syncthreads_count(AA ? done & doneB : T < 0.0f) == CT) break;
        const int nb = min(CBF, end - b0);
        if constexpr (STATS) nst += nb;
        if ((int)threadIdx.x < CBF)
            s_m[threadIdx.x] = (int)threadIdx.x < nb ? (uint8_t)stage_record(P, ra, rb, rc, rd, tx, ty, s_wd, s_g[threadIdx.x]) : 0;
        if ((int)threadIdx.x < CBF && b0 + CBF + (int)threadIdx.x < end)
            load_record(P.rec, P.ids[b0 + CBF + threadIdx.x], ra, rb, rc, rd);
        __syncthreads();
        bool wdone = __ballot(AA ? !(done & doneB) : T > 0.0f) == 0;
        for (int i = 0; i < CBF / 64 && !wdone; ++i) {
            unsigned long long m = __ballot((s_m[i * 64 + lane] >> wave) & 1);
            // two entries per iteration: their evaluations are independent of the
            // pixel state, the compositing takes them in order
            auto composite_entry = [&](const Staged& g, const Pair& pr, int k) {
                const float aF = pr.aF;
                if constexpr (!AA) {
                    // T < 0 (stopped) makes Tn < 0: low, not included, -|T| kept
                    const float Tn = T * (1.0f - aF);
                    const bool low = Tn < STOP_T;
                    const bool inc = pr.ok & !low;
                    const float w = inc ? aF * T : 0.0f;
                    C0 = __builtin_fmaf(w, g.b.z, C0);
                    C1 = __builtin_fmaf(w, g.b.w, C1);
                    C2 = __builtin_fmaf(w, g.c.x, C2);
                    Z = __builtin_fmaf(w, g.c.y, Z);
                    T = inc ? Tn : (pr.ok & low) ? -fabsf(T) : T;
                    last = inc ? b0 + k - start + 1 : last;
                    if constexpr (STATS) ninc += inc ? 1 : 0;
                    return;
                }
                const bool live = !done & pr.ok;
                const float Tn = T * (1.0f - aF);
                const bool stop = live & (Tn < STOP_T);
                const bool inc = live & !stop;
                const float w = inc ? aF * T : 0.0f;
                C0 = __builtin_fmaf(w, g.b.z, C0);
                C1 = __builtin_fmaf(w, g.b.w, C1);
                C2 = __builtin_fmaf(w, g.c.x, C2);
                Z = __builtin_fmaf(w, g.c.y, Z);
                T = inc ? Tn : T;
                last = inc ? b0 + k - start + 1 : last;
                done = done | stop;
                if constexpr (STATS) ninc += inc ? 1 : 0;
                if constexpr (AA) {
                    const float aB = pr.al * pr.fb;
                    doneB = doneB | done;  // the pixel stops with its front layer
                    const bool liveB = !doneB & !(pr.q > g.d.z) & (pr.al >= SKIP_ALPHA) & (aB >= SKIP_ALPHA);
                    const float TnB = TB * (1.0f - aB);
                    const bool stopB = liveB & (TnB < STOP_T);
                    const bool incB = liveB & !stopB;
                    const float wB = incB ? aB * TB : 0.0f;
                    B0 = __builtin_fmaf(wB, g.b.z, B0);
                    B1 = __builtin_fmaf(wB, g.b.w, B1);
                    B2 = __builtin_fmaf(wB, g.c.x, B2);
                    ZB = __builtin_fmaf(wB, g.c.y, ZB);
                    TB = incB ? TnB : TB;
                    lastB = incB ? b0 + k - start + 1 : lastB;
                    doneB = doneB | stopB;
                }
            };
            while (m) {
                const int k = i * 64 + __builtin_ctzll(m);
                m &= m - 1;
                const bool two = m != 0;
                const int k2 = two ? i * 64 + __builtin_ctzll(m) : k;
                if (two) m &= m - 1;
                const Staged g = s_g[k];  // one 64-byte LDS broadcast read
                const Staged g2 = s_g[k2];
                const Pair pr = eval_pair(g, pxc, pyc, on, wave_on, D, P.softness);
                const Pair pr2 = eval_pair(g2, pxc, pyc, on, wave_on, D, P.softness);
                composite_entry(g, pr, k);
                if (two) composite_entry(g2, pr2, k2);
                if constexpr (STATS) nev += two ? 2 : 1;
                if (__ballot(AA ? !(done & doneB) : T > 0.0f) == 0) {
                    wdone = true;
                    break;
                }
            }
        }
    }
    if constexpr (STATS) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ninc += __shfl_xor(ninc, o, 64);
        if (lane == 0) {
            atomicAdd(&stats[0], (unsigned long long)ninc);
            atomicAdd(&stats[1], (unsigned long long)nev);
        }
        if (threadIdx.x == 0) atomicAdd(&stats[2], (unsigned long long)nst);
    }
    if (!inside) return;
    if constexpr (!AA) T = fabsf(T);
    if constexpr (AA) {
        const float ob = 1.0f - ml.am;
        const float Y0 = B0 + TB * P.bg[0], Y1 = B1 + TB * P.bg[1], Y2 = B2 + TB * P.bg[2];
        out_rgb[3 * pix + 0] = C0 + T * (ml.M0 + ob * Y0);
        out_rgb[3 * pix + 1] = C1 + T * (ml.M1 + ob * Y1);
        out_rgb[3 * pix + 2] = C2 + T * (ml.M2 + ob * Y2);
        out_alpha[pix] = 1.0f - T * ob * TB;
        out_depth[pix] = Z + T * (ml.MD + ob * ZB);
        float4* st = reinterpret_cast<float4*>(state_aa) + 2 * pix;
        st[0] = make_float4(T, __int_as_float(last), TB, __int_as_float(lastB));
        st[1] = make_float4(B0, B1, B2, ZB);
    } else {
        out_rgb[3 * pix + 0] = C0 + T * state_cm[3 * pix + 0];
        out_rgb[3 * pix + 1] = C1 + T * state_cm[3 * pix + 1];
        out_rgb[3 * pix + 2] = C2 + T * state_cm[3 * pix + 2];
        out_alpha[pix] = on ? 1.0f : 1.0f - T;
        out_depth[pix] = Z + (on ? T * D : 0.0f);
        state_T[pix] = T;
        state_last[pix] = last;
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// The same reduction of the first 10 values only (a wave off the mesh, where the
// four depth-density sums are zero): 5 + 3 + 2 + 1 exchanges before the quad steps.
// Every value meets the lanes in the same pairing order as in wave_sum16 (l ^ 32,
// l ^ 16, l ^ 8, the half-row mirror, the quad), so its total is bit-identical.
// On return lane l holds the total of value basis10(l) when (l & 3) == 0 and that
// index is not negative.
__device__ __forceinline__ float wave_sum10(const float* v, int lane)
{
    float a[5], b[3];
#pragma unroll
    for (int i = 0; i < 5; ++i) {  // lanes 0-31 keep v[i], lanes 32-63 keep v[5+i]
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[5 + i]), false,
                                                        false);
        a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {  // even rows keep a[i], odd rows a[3+i] (a[2] alone: odd rows unused)
        const float hi = i < 2 ? a[3 + i] : a[2];
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(hi), false, false);
        b[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool h3 = lane & 8, h2 = lane & 4;
    // partner lane ^ 8: pair (b0, b2) split by bit 3; b1 alone (lanes with bit 3 unused)
    const float c0 = (h3 ? b[2] : b[0]) + dpp<0x128>(h3 ? b[0] : b[2]);
    const float c1 = b[1] + dpp<0x128>(b[1]);
    const float send = h2 ? c0 : c1;
    float d = (h2 ? c1 : c0) + dpp<0x141>(send);
    d += dpp<0x4E>(d);
    d += dpp<0xB1>(d);
    return d;
}

// Value index whose total wave_sum10 leaves in lane l (l & 3 == 0), or -1.
__device__ __forceinline__ int basis10(int lane)
{
    const bool H = lane & 32, R = lane & 16, h3 = lane & 8, h2 = lane & 4;
    const int ai = h3 ? ((h2 || R) ? -1 : 2) : ((R ? 3 : 0) + (h2 ? 1 : 0));
    return ai < 0 ? -1 : ai + (H ? 5 : 0);
}

// The same reduction of 14 values (a wave on the mesh: the ten above and the four
// depth-density sums), without the two zero values wave_sum16 would carry: 7 + 4 +
// 2 + 1 exchanges.  Same pairing order, so bit-identical totals.  On return lane l
// holds the total of value basis14(l) when (l & 3) == 0 and that index is not
// negative.
__device__ __forceinline__ float wave_sum14(const float* v, int lane)
{
    float a[7], b[4];
#pragma unroll
    for (int i = 0; i < 7; ++i) {  // lanes 0-31 keep v[i], lanes 32-63 keep v[7+i]
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[7 + i]), false,
                                                        false);
        a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // even rows keep a[i], odd rows a[4+i] (a[3] alone: odd rows unused)
        const float hi = i < 3 ? a[4 + i] : a[3];
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(hi), false, false);
        b[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool h3 = lane & 8, h2 = lane & 4;
    const float c0 = (h3 ? b[2] : b[0]) + dpp<0x128>(h3 ? b[0] : b[2]);
    const float c1 = (h3 ? b[3] : b[1]) + dpp<0x128>(h3 ? b[1] : b[3]);
    const float send = h2 ? c0 : c1;
    float d = (h2 ? c1 : c0) + dpp<0x141>(send);
    d += dpp<0x4E>(d);
    d += dpp<0xB1>(d);
    return d;
}

// Value index whose total wave_sum14 leaves in lane l (l & 3 == 0), or -1.
__device__ __forceinline__ int basis14(int lane)
{
    const bool H = lane & 32, R = lane & 16;
    const int j = ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
    const int ai = j == 3 ? (R ? -1 : 3) : (R ? 4 + j : j);
    return ai < 0 ? -1 : ai + (H ? 7 : 0);
}

// AA = true: the reverse mode of the two-layer form.  The back layer sees the
// upstream gradients scaled by k = T_F (1 - a_m) and, behind it, bg (depth 0) and
// the alpha term; per entry dL/dalpha = f dL/dalpha_F + (1 - f) dL/dalpha_B and
// dL/ds = alpha phi(s) (dL/dalpha_F - dL/dalpha_B).  Both layers recover their
// transmittance by division while walking back from max(last_F, last_B).  The
// per-pixel outputs are dL/d(M, M_D, a_m, D) of the mesh layer.
// Order in which the backward takes the tiles: longest walk first.  A tile's walk is
// the longest pixel walk (entries up to the last included one, of either layer) of
// its four waves, which run side by side, one per SIMD (ordering by their sum was
// 1.7% slower); walks differ by an order of magnitude across an image, and blocks
// taken in raster order leave long tiles for the end of the grid.
//
// The same launch clears the n record gradients the composite kernel accumulates
// into (a grid-stride fill: the walk reads are latency-bound, the fill is
// store-bound, and one launch overlaps the two).
template <bool AA>
__global__ void __launch_bounds__(CT)
k_tile_walk(CompParams P, const int32_t* __restrict__ state_last, const float* __restrict__ state_aa,
            int32_t* __restrict__ walk, float* __restrict__ g_rec, int64_t n)
{
    __shared__ int s_w[CT / 64];
    const int tile = blockIdx.x;
    {
        const int64_t stride = (int64_t)gridDim.x * CT, me = (int64_t)tile * CT + threadIdx.x;
        // floats before the first 16-byte boundary, whole float4s, the rest
        const int64_t head = min(n, (int64_t)(((16u - ((uintptr_t)g_rec & 15u)) & 15u) >> 2));
        const int64_t n4 = (n - head) >> 2;
        if (me < head) g_rec[me] = 0.0f;
        float4* body = reinterpret_cast<float4*>(g_rec + head);
        for (int64_t i = me; i < n4; i += stride) body[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int64_t i = head + (n4 << 2) + me; i < n; i += stride) g_rec[i] = 0.0f;
    }
    const int tx = tile % P.cam.tx, ty = tile / P.cam.tx;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int px = tx * GM_TILE + 8 * (wave & 1) + (lane & 7), py = ty * GM_TILE + 8 * (wave >> 1) + (lane >> 3);
    int m = 0;
    if (px < P.cam.width && py < P.cam.height) {
        const int pix = py * P.cam.width + px;
        if constexpr (AA) {
            const float4 s0 = reinterpret_cast<const float4*>(state_aa)[2 * pix];
            m = max(__float_as_int(s0.y), __float_as_int(s0.w));
        } else {
            m = state_last[pix];
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if (lane == 0) s_w[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) walk[tile] = max(max(s_w[0], s_w[1]), max(s_w[2], s_w[3]));
}

// Order in which the backward takes the tiles: longest walk first (the shared
// counting sort of the tiles by a per-tile key, one block).
__global__ void __launch_bounds__(TO_THREADS) k_tile_order(int T, const int32_t* __restrict__ walk,
                                                           int32_t* __restrict__ order)
{
    order_tiles_desc(T, [=](int t) { return walk[t]; }, order);
}

// Six blocks of the backward fit a CU's LDS; the register budget is held to the
// same six waves per SIMD (80 VGPRs; the two-layer form needs more and runs five).
template <bool AA>
__global__ void __launch_bounds__(CT) __attribute__((amdgpu_waves_per_eu(AA ? 5 : 6, AA ? 5 : 6)))
k_composite_bwd(CompParams P, const float* __restrict__ state_T, const int32_t* __restrict__ state_last,
                const float* __restrict__ state_cm, const float* __restrict__ layer,
                const float* __restrict__ state_aa, const float* __restrict__ g_rgb,
                const float* __restrict__ g_depth, const float* __restrict__ g_alpha, float* __restrict__ g_rec,
                float* __restrict__ g_mesh_rgb, float* __restrict__ g_mesh_depth, float* __restrict__ g_layer,
                const int32_t* __restrict__ order)
{
    __shared__ Staged s_g[CBB];
    __shared__ int s_id[CBB];
    __shared__ uint8_t s_m[CBB];
    __shared__ float s_acc[CBB][NBASIS];
    __shared__ float s_wd[CT / 64];
    __shared__ int s_wl[CT / 64];
    const int tile = order[blockIdx.x];  // longest walks first
    const int tx = tile % P.cam.tx, ty = tile / P.cam.tx;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int px = tx * GM_TILE + 8 * (wave & 1) + (lane & 7), py = ty * GM_TILE + 8 * (wave >> 1) + (lane >> 3);
    const bool inside = px < P.cam.width && py < P.cam.height;
    const int pix = py * P.cam.width + px;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const int start = P.ranges[2 * tile];

    bool on;
    float D, TF;
    int last;
    AaLayer ml{};
    float TB = 1.0f, Y0 = 0.0f, Y1 = 0.0f, Y2 = 0.0f, ZB = 0.0f, kB = 0.0f;
    int lastB = 0;
    if constexpr (AA) {
        ml = inside ? load_layer(layer, pix) : AaLayer{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, INFINITY};
        D = ml.D;
        on = D < INFINITY;
        float4 s0 = make_float4(1.0f, 0.0f, 1.0f, 0.0f), s1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (inside) {
            s0 = reinterpret_cast<const float4*>(state_aa)[2 * pix];
            s1 = reinterpret_cast<const float4*>(state_aa)[2 * pix + 1];
        }
        TF = s0.x;
        last = __float_as_int(s0.y);
        TB = s0.z;
        lastB = __float_as_int(s0.w);
        Y0 = s1.x + TB * P.bg[0];
        Y1 = s1.y + TB * P.bg[1];
        Y2 = s1.z + TB * P.bg[2];
        ZB = s1.w;
        kB = TF * (1.0f - ml.am);
    } else {
        const int fid = inside ? P.face_id[pix] : -1;
        on = fid >= 0;
        D = on ? P.depth[pix] : INFINITY;
        TF = inside ? state_T[pix] : 1.0f;
        last = inside ? state_last[pix] : 0;
    }
    float GC0 = 0.0f, GC1 = 0.0f, GC2 = 0.0f, GZ = 0.0f, GA = 0.0f, Bt = 0.0f, BtB = 0.0f;
    if (inside) {
        GC0 = g_rgb[3 * pix + 0];
        GC1 = g_rgb[3 * pix + 1];
        GC2 = g_rgb[3 * pix + 2];
        if (g_depth) GZ = g_depth[pix];
        if (g_alpha) GA = g_alpha[pix];
        if constexpr (AA) {
            // dL/dT_F: everything behind the front layer; dL/dT_B (scaled by kB): bg and alpha
            const float ob = 1.0f - ml.am;
            Bt = GC0 * (ml.M0 + ob * Y0) + GC1 * (ml.M1 + ob * Y1) + GC2 * (ml.M2 + ob * Y2) +
                 GZ * (ml.MD + ob * ZB) - GA * ob * TB;
            BtB = kB * (GC0 * P.bg[0] + GC1 * P.bg[1] + GC2 * P.bg[2] - GA);
        } else {
            // B = dL/dT_F: the colour behind the Gaussians, the mesh depth and the alpha
            Bt = GC0 * state_cm[3 * pix + 0] + GC1 * state_cm[3 * pix + 1] + GC2 * state_cm[3 * pix + 2] +
                 (on ? GZ * D : -GA);
        }
    }
    float acc = TF * Bt;
    float T = TF;
    float accB = TB * BtB;
    float TBw = TB;
    float gD = 0.0f;

    if constexpr (AA)
        wave_dmax(inside, on && ml.am >= 1.0f, D, s_wd);
    else
        wave_dmax(inside, on, D, s_wd);
    const bool wave_on = __ballot(on) != 0;
    int m = AA ? max(last, lastB) : last;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if (lane == 0) s_wl[wave] = m;
    __syncthreads();
    const int mlast = max(max(s_wl[0], s_wl[1]), max(s_wl[2], s_wl[3]));

    float4 ra, rb, rc, rd;
    int id = 0;
    {
        const int bend = start + mlast;
        const int b0 = max(start, bend - CBB);
        if (b0 + (int)threadIdx.x < bend) {
            id = P.ids[b0 + threadIdx.x];
            load_record(P.rec, id, ra, rb, rc, rd);
        }
    }
    for (int bend = start + mlast; bend > start; bend -= CBB) {
        const int b0 = max(start, bend - CBB);
        const int nb = bend - b0;
        __syncthreads();
        uint32_t msk = 0;
        if ((int)threadIdx.x < nb) {
            msk = stage_record(P, ra, rb, rc, rd, tx, ty, s_wd, s_g[threadIdx.x]);
            const int rel = b0 + threadIdx.x - start;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if (rel >= s_wl[w]) msk &= ~(1u << w);
            s_id[threadIdx.x] = id;
#pragma unroll
            for (int c = 0; c < NBASIS; ++c) s_acc[threadIdx.x][c] = 0.0f;
        }
        if (threadIdx.x < CBB) s_m[threadIdx.x] = (uint8_t)msk;
        {
            const int nend = b0, nb0 = max(start, nend - CBB);
            if (nb0 + (int)threadIdx.x < nend) {
                id = P.ids[nb0 + threadIdx.x];
                load_record(P.rec, id, ra, rb, rc, rd);
            }
        }
        __syncthreads();
        // the entries of the batch, back to front; instantiated apart for waves with
        // and without a pixel on the mesh (a uniform choice made once per wave), so
        // each form is one straight-line loop body
        auto entries = [&](auto on_mesh) {
            constexpr bool ON = decltype(on_mesh)::value;
            for (int i = (CBB + 63) / 64 - 1; i >= 0; --i) {
                unsigned long long mm = __ballot(i * 64 + lane < CBB && ((s_m[i * 64 + lane] >> wave) & 1));
                while (mm) {
                    const int kk = 63 - __builtin_clzll(mm);
                    mm &= ~(1ull << kk);
                    const int k = i * 64 + kk;
                    const Staged g = s_g[k];  // one 64-byte LDS broadcast read
                    const int rel = b0 + k - start;
                    // inactive lanes carry zeros through the same arithmetic
                    const Pair pr = eval_pair(g, pxc, pyc, on, ON, D, P.softness);
                    const float dx = pr.dx, dy = pr.dy, oG = pr.oG, al = pr.al, f = pr.f, pdf = pr.pdf, sv = pr.s;
                    const float aF = pr.aF;
                    bool act = (rel < last) & pr.ok;
                    // whether a lane of the wave takes the entry: the ballot of each
                    // comparison of act (one layer), so the branch tests a scalar mask
                    // instead of turning act into a vector value and back
                    auto any_act = [&]() -> bool {
                        if constexpr (AA) return __ballot(act) != 0ull;
                        return (__ballot(rel < last) & __ballot(!(pr.q > g.d.z)) & __ballot(pr.al >= SKIP_ALPHA) &
                                __ballot(pr.aF >= SKIP_ALPHA)) != 0ull;
                    };
                    // per-pixel basis sums; the 13 record gradients are linear in them
                    // (formed once per entry at the flush):
                    //  0-2 w GC, 3 w GZ, 4 H, 5 H dx, 6 H dy, 7 H dx^2, 8 H dx dy, 9 H dy^2,
                    //  10 ds, 11 ds dx, 12 ds dy, 13 ds s   (H = o G dL/dalpha, ds = dL/ds)
                    const float aFe = act ? aF : 0.0f;
                    // 1 - alpha_F >= 0.01: a hardware reciprocal (1 ulp) keeps the
                    // recovered transmittance far inside the gradient tolerance
                    const float iom = __builtin_amdgcn_rcpf(1.0f - aFe);
                    const float Ti = T * iom;
                    const float w = aFe * Ti;
                    const float Vv = __builtin_fmaf(GC0, g.b.z,
                                                    __builtin_fmaf(GC1, g.b.w, __builtin_fmaf(GC2, g.c.x, GZ * g.c.y)));
                    const float daF = act ? __builtin_fmaf(Ti, Vv, -acc * iom) : 0.0f;
                    acc = __builtin_fmaf(w, Vv, acc);
                    T = Ti;
                    float wt = w, da = f * daF, dsF = daF;
                    if constexpr (AA) {
                        const float aB = al * pr.fb;
                        const bool actB = (rel < lastB) & !(pr.q > g.d.z) & (al >= SKIP_ALPHA) & (aB >= SKIP_ALPHA);
                        const float aBe = actB ? aB : 0.0f;
                        const float iomB = __builtin_amdgcn_rcpf(1.0f - aBe);
                        const float TiB = TBw * iomB;
                        const float wB = aBe * TiB;
                        const float VB = kB * Vv;
                        const float daB = actB ? __builtin_fmaf(TiB, VB, -accB * iomB) : 0.0f;
                        accB = __builtin_fmaf(wB, VB, accB);
                        TBw = TiB;
                        wt = __builtin_fmaf(kB, wB, w);
                        da = __builtin_fmaf(pr.fb, daB, da);
                        dsF = daF - daB;
                        act = act | actB;
                    }
                    float gr[14];
                    gr[0] = wt * GC0;
                    gr[1] = wt * GC1;
                    gr[2] = wt * GC2;
                    gr[3] = wt * GZ;
                    const float H = oG <= ALPHA_MAX ? oG * da : 0.0f;
                    const float Hx = H * dx, Hy = H * dy;
                    gr[4] = H;
                    gr[5] = Hx;
                    gr[6] = Hy;
                    gr[7] = Hx * dx;
                    gr[8] = Hx * dy;
                    gr[9] = Hy * dy;
                    if constexpr (ON) {
                        const float ds = (al * pdf) * dsF;
                        gr[10] = ds;
                        gr[11] = ds * dx;
                        gr[12] = ds * dy;
                        gr[13] = ds * sv;
                        gD = __builtin_fmaf(g.d.y, ds, gD);
                        if (any_act()) {
                            const float v = wave_sum14(gr, lane);
                            const int c = basis14(lane);
                            if ((lane & 3) == 0 && c >= 0 && v != 0.0f) atomicAdd(&s_acc[k][c], v);
                        }
                    } else if (any_act()) {  // off the mesh the density (and so ds) is zero
                        const float v = wave_sum10(gr, lane);
                        const int c = basis10(lane);
                        if ((lane & 3) == 0 && c >= 0 && v != 0.0f) atomicAdd(&s_acc[k][c], v);
                    }
                }
            }
        };
        if (wave_on) entries(std::true_type{});
        else entries(std::false_type{});
        __syncthreads();
        if ((int)threadIdx.x < nb) {
            const float* S = s_acc[threadIdx.x];
            const Staged& g = s_g[threadIdx.x];
            const float kap = g.d.y;
            // the conic from its staged Cholesky factor: Q = 2 L L^T
            const float q00 = 2.0f * (g.a.z * g.a.z), q01 = 2.0f * (g.a.z * g.a.w),
                        q11 = 2.0f * __builtin_fmaf(g.a.w, g.a.w, g.b.x * g.b.x);
            float gv[GM_GRAD];
            gv[0] = __builtin_fmaf(q00, S[5], __builtin_fmaf(q01, S[6], kap * g.c.z * S[10]));
            gv[1] = __builtin_fmaf(q01, S[5], __builtin_fmaf(q11, S[6], kap * g.c.w * S[10]));
            gv[2] = -0.5f * S[7];
            gv[3] = -S[8];
            gv[4] = -0.5f * S[9];
            gv[5] = S[4] != 0.0f ? S[4] / g.b.y : 0.0f;  // dL/do = sum G f dL/dalpha_F = (sum H) / o
            gv[6] = S[0];
            gv[7] = S[1];
            gv[8] = S[2];
            gv[9] = S[3] - kap * S[10];
            gv[10] = -kap * S[11];
            gv[11] = -kap * S[12];
            gv[12] = -S[13] * g.d.w;
            float* dst = s_acc[threadIdx.x];
#pragma unroll
            for (int c = 0; c < GM_GRAD; ++c) dst[c] = gv[c];
        }
        __syncthreads();
        // flush with 16 lanes per entry (one lane per field): each atomic instruction
        // then touches the 52-byte gradient records of only four Gaussians instead of
        // 64, so the memory-side atomics arrive grouped by cache line
        for (int e0 = 0; e0 < nb; e0 += CT / 16) {
            const int e = e0 + (int)(threadIdx.x >> 4), c = threadIdx.x & 15;
            if (e < nb && c < GM_GRAD) {
                const float v = s_acc[e][c];
                if (v != 0.0f) unsafeAtomicAdd(g_rec + (size_t)s_id[e] * GM_GRAD + c, v);
            }
        }
    }
    if (!inside) return;
    if constexpr (AA) {
        float4* gl = reinterpret_cast<float4*>(g_layer) + 2 * pix;
        gl[0] = make_float4(TF * GC0, TF * GC1, TF * GC2, TF * GZ);
        gl[1] = make_float4(TF * (GA * TB - (GC0 * Y0 + GC1 * Y1 + GC2 * Y2) - GZ * ZB), gD, 0.0f, 0.0f);
        return;
    }
    const float am = on ? 1.0f : 0.0f;
    if (g_mesh_rgb) {
        g_mesh_rgb[3 * pix + 0] = TF * am * GC0;
        g_mesh_rgb[3 * pix + 1] = TF * am * GC1;
        g_mesh_rgb[3 * pix + 2] = TF * am * GC2;
    }
    if (g_mesh_depth) g_mesh_depth[pix] = TF * am * GZ + gD;
}

// Mesh surface and light fields of the parameters (for the colour prepass).
static gm_status fill_surface(CompParams& P, const gm_mesh* mesh, const float* vscreen, const gm_light* light)
{
    if (mesh && mesh->F > 0) {
        GM_ARG_CHECK(mesh->faces && vscreen, "mesh faces / vscreen is NULL");
        P.V = mesh->V;
        P.F = mesh->F;
        P.Vt = mesh->Vt;
        P.vscreen = vscreen;
        P.faces = mesh->faces;
        P.vcolor = mesh->vcolor;
        P.vnormal = mesh->vnormal;
        if (mesh->mips) {
            GM_ARG_CHECK(mesh->uv && mesh->faces_uv, "textured mesh needs uv and faces_uv");
            GM_ARG_CHECK(mesh->tex_size > 0 && (mesh->tex_size & (mesh->tex_size - 1)) == 0,
                         "tex_size %d is not a power of two", mesh->tex_size);
            P.uv = mesh->uv;
            P.faces_uv = mesh->faces_uv;
            P.mips = mesh->mips;
            P.tex_size = mesh->tex_size;
            int n = 0;
            for (int s = mesh->tex_size; s >= 1; s >>= 1) ++n;
            P.nlev = n;
        }
    }
    if (light) {
        P.lit = 1;
        for (int i = 0; i < 3; ++i) {
            P.lpos[i] = light->pos[i];
            P.lamb[i] = light->ambient[i];
            P.ldif[i] = light->diffuse[i];
            P.lspec[i] = light->specular[i];
        }
        P.lshin = light->shininess;
    }
    return GM_OK;
}

static gm_status fill_params(CompParams& P, const gm_camera* cam, const float* rec, const int32_t* ranges,
                             const int32_t* ids, const int32_t* face_id, const float* depth,
                             const gm_mesh* mesh, const float* vscreen, const gm_light* light,
                             const float* bg, float softness)
{
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(ranges && face_id && depth && bg, "tile_ranges / face_id / depth / bg is NULL");
    GM_ARG_CHECK(softness >= 0.0f, "softness must be >= 0");
    GM_ARG_CHECK(((uintptr_t)rec & 15) == 0, "rec must be 16-byte aligned");
    P = CompParams{};
    P.cam = dev_camera(*cam);
    P.rec = rec;
    P.ranges = ranges;
    P.ids = ids;
    P.face_id = face_id;
    P.depth = depth;
    if (gm_status s = fill_surface(P, mesh, vscreen, light)) return s;
    for (int i = 0; i < 3; ++i) P.bg[i] = bg[i];
    P.softness = softness;
    return GM_OK;
}

// Parameters of the two-layer kernels: the mesh enters through its layer only.
static gm_status fill_params_aa(CompParams& P, const gm_camera* cam, const float* rec, const int32_t* ranges,
                                const int32_t* ids, const float* layer, const float* bg, float softness)
{
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(ranges && layer && bg, "tile_ranges / layer / bg is NULL");
    GM_ARG_CHECK(softness >= 0.0f, "softness must be >= 0");
    GM_ARG_CHECK(((uintptr_t)rec & 15) == 0 && ((uintptr_t)layer & 15) == 0, "rec and layer must be 16-byte aligned");
    P = CompParams{};
    P.cam = dev_camera(*cam);
    P.rec = rec;
    P.ranges = ranges;
    P.ids = ids;
    for (int i = 0; i < 3; ++i) P.bg[i] = bg[i];
    P.softness = softness;
    return GM_OK;
}

gm_status launch_surface_colour(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                                const gm_light* light, const int32_t* face_id, const float* bg, float* colour,
                                hipStream_t stream)
{
    CompParams P{};
    P.cam = dev_camera(*cam);
    P.face_id = face_id;
    if (gm_status s = fill_surface(P, mesh, vscreen, light)) return s;
    for (int i = 0; i < 3; ++i) P.bg[i] = bg ? bg[i] : 0.0f;
    const int64_t HW = (int64_t)P.cam.width * P.cam.height;
    k_shade<<<(unsigned)div_up(HW, 256), 256, 0, stream>>>(P, colour);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

}  // namespace gm

using namespace gm;

// The backward's workspace: per-tile walk lengths, then the tile order.
static gm_status tile_order_ws(const gm_camera* cam, void* ws, size_t ws_bytes, int32_t** walk, int32_t** order)
{
    const size_t need = gm_composite_hybrid_bwd_ws(cam->width, cam->height);
    GM_ARG_CHECK(ws != nullptr && ws_bytes >= need, "workspace %zu bytes, %zu needed", ws_bytes, need);
    const int64_t T = div_up(cam->width, GM_TILE) * div_up(cam->height, GM_TILE);
    *walk = static_cast<int32_t*>(ws);
    *order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(sizeof(int32_t) * (size_t)T, 256));
    return GM_OK;
}

// Host checks of the one-layer reverse mode; fills its kernel parameters.
static gm_status bwd_params(CompParams& P, const gm_camera* cam, int32_t N, const float* rec,
                            const int32_t* tile_ranges, const int32_t* sorted_ids, const int32_t* face_id,
                            const float* depth, float softness, const float* state_T, const int32_t* state_last,
                            const float* state_cm, const float* g_rgb, const float* g_rec)
{
    const float zero3[3] = {0.0f, 0.0f, 0.0f};
    if (gm_status s = fill_params(P, cam, rec, tile_ranges, sorted_ids, face_id, depth, nullptr, nullptr, nullptr,
                                  zero3, softness))
        return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(state_T && state_last && state_cm && g_rgb, "state or g_rgb is NULL");
    GM_ARG_CHECK(N == 0 || g_rec, "g_rec is NULL");
    return GM_OK;
}

// Reverse mode of the one-layer composite with the tile walk lengths and order in
// walk [T] and order [T] (device scratch; every entry is written before it is read).
static gm_status bwd_launch(const CompParams& P, int32_t N, const float* state_T, const int32_t* state_last,
                            const float* state_cm, const float* g_rgb, const float* g_depth, const float* g_alpha,
                            float* g_rec, float* g_mesh_rgb, float* g_mesh_depth, int32_t* walk, int32_t* order,
                            hipStream_t stream)
{
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    const int64_t n = N > 0 ? (int64_t)N * GM_GRAD : 0;
    k_tile_walk<false><<<(unsigned)T, CT, 0, stream>>>(P, state_last, nullptr, walk, g_rec, n);
    GM_LAUNCH_CHECK();
    k_tile_order<<<1, TO_THREADS, 0, stream>>>((int)T, walk, order);
    GM_LAUNCH_CHECK();
    k_composite_bwd<false><<<(unsigned)T, CT, 0, stream>>>(P, state_T, state_last, state_cm, nullptr, nullptr,
                                                          g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth,
                                                          nullptr, order);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

// Fixed scratch of gm_composite_hybrid_bwd_noalloc, for callers that cannot
// allocate: the walk lengths (first GM_NOALLOC_MAX_TILES ints) and the tile order
// (next GM_NOALLOC_MAX_TILES) of one image.  Every GPU the library runs on holds its
// own copy, at its own address, until the process ends.  In host code the array's
// name is not a device address: the kernels receive the address that
// hipGetSymbolAddress gives on that device, looked up once per device.
static __device__ __align__(256) int32_t scratch[2 * GM_NOALLOC_MAX_TILES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static int32_t* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// Device address of `scratch` on the device that owns `stream`, which must be the
// current device (the symbol address is looked up with that device current).
static gm_status noalloc_scratch(hipStream_t stream, int32_t** out)
{
    int cur = -1, dev = -1;
    GM_HIP_CHECK(hipGetDevice(&cur));
    GM_HIP_CHECK(hipStreamGetDevice(stream, &dev));
    GM_ARG_CHECK(dev == cur, "stream belongs to device %d, current device is %d", dev, cur);
    GM_ARG_CHECK(cur >= 0 && cur < NOALLOC_MAX_DEVICES, "device %d above %d", cur, NOALLOC_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[cur]) {
        void* p = nullptr;
        GM_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        GM_ARG_CHECK(p != nullptr, "no device address for the fixed scratch on device %d", cur);
        g_scratch_ptr[cur] = static_cast<int32_t*>(p);
    }
    *out = g_scratch_ptr[cur];
    return GM_OK;
}

extern "C" {

gm_status gm_composite_hybrid_fwd(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                  const int32_t* sorted_ids, const int32_t* face_id, const float* depth,
                                  const gm_mesh* mesh, const float* vscreen, const gm_light* light,
                                  const float* bg, float softness, float* out_rgb, float* out_depth,
                                  float* out_alpha, float* state_T, int32_t* state_last, float* state_cm,
                                  hipStream_t stream)
{
    clear_error();
    CompParams P;
    if (gm_status s = fill_params(P, cam, rec, tile_ranges, sorted_ids, face_id, depth, mesh, vscreen, light,
                                  bg, softness))
        return s;
    GM_ARG_CHECK(out_rgb && out_depth && out_alpha && state_T && state_last && state_cm, "an output is NULL");
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    const int64_t HW = (int64_t)P.cam.width * P.cam.height;
    k_shade<<<(unsigned)div_up(HW, 256), 256, 0, stream>>>(P, state_cm);
    GM_LAUNCH_CHECK();
    k_composite_fwd<false><<<(unsigned)T, CT, 0, stream>>>(P, state_cm, nullptr, out_rgb, out_depth, out_alpha,
                                                          state_T, state_last, nullptr);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

gm_status gm_shade_surface(const gm_camera* cam, const int32_t* face_id, const gm_mesh* mesh, const float* vscreen,
                           const gm_light* light, const float* bg, float* state_cm, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(face_id && bg && state_cm, "face_id / bg / state_cm is NULL");
    return launch_surface_colour(cam, mesh, vscreen, light, face_id, bg, state_cm, stream);
}

gm_status gm_composite_hybrid_fwd_shaded(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                         const int32_t* sorted_ids, const int32_t* face_id, const float* depth,
                                         float softness, const float* state_cm, float* out_rgb, float* out_depth,
                                         float* out_alpha, float* state_T, int32_t* state_last, hipStream_t stream)
{
    clear_error();
    CompParams P;
    const float zero3[3] = {0.0f, 0.0f, 0.0f};  // bg enters through state_cm
    if (gm_status s = fill_params(P, cam, rec, tile_ranges, sorted_ids, face_id, depth, nullptr, nullptr, nullptr,
                                  zero3, softness))
        return s;
    GM_ARG_CHECK(state_cm, "state_cm is NULL");
    GM_ARG_CHECK(out_rgb && out_depth && out_alpha && state_T && state_last, "an output is NULL");
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    k_composite_fwd<false><<<(unsigned)T, CT, 0, stream>>>(P, state_cm, nullptr, out_rgb, out_depth, out_alpha,
                                                          state_T, state_last, nullptr);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

gm_status gm_composite_hybrid_fwd_stats(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                        const int32_t* sorted_ids, const int32_t* face_id, const float* depth,
                                        float softness, const float* state_cm, float* out_rgb, float* out_depth,
                                        float* out_alpha, float* state_T, int32_t* state_last, int64_t* stats,
                                        hipStream_t stream)
{
    clear_error();
    CompParams P;
    const float zero3[3] = {0.0f, 0.0f, 0.0f};
    if (gm_status s = fill_params(P, cam, rec, tile_ranges, sorted_ids, face_id, depth, nullptr, nullptr, nullptr,
                                  zero3, softness))
        return s;
    GM_ARG_CHECK(state_cm && stats, "state_cm / stats is NULL");
    GM_ARG_CHECK(out_rgb && out_depth && out_alpha && state_T && state_last, "an output is NULL");
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    k_composite_fwd<false, true><<<(unsigned)T, CT, 0, stream>>>(P, state_cm, nullptr, out_rgb, out_depth, out_alpha,
                                                                state_T, state_last, nullptr,
                                                                reinterpret_cast<unsigned long long*>(stats));
    GM_LAUNCH_CHECK();
    return GM_OK;
}

gm_status gm_composite_hybrid_fwd_aa(const gm_camera* cam, const float* rec, const int32_t* tile_ranges,
                                     const int32_t* sorted_ids, const float* layer, const float* bg, float softness,
                                     float* out_rgb, float* out_depth, float* out_alpha, float* state,
                                     hipStream_t stream)
{
    clear_error();
    CompParams P;
    if (gm_status s = fill_params_aa(P, cam, rec, tile_ranges, sorted_ids, layer, bg, softness)) return s;
    GM_ARG_CHECK(out_rgb && out_depth && out_alpha && state, "an output is NULL");
    GM_ARG_CHECK(((uintptr_t)state & 15) == 0, "state must be 16-byte aligned");
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    k_composite_fwd<true><<<(unsigned)T, CT, 0, stream>>>(P, nullptr, layer, out_rgb, out_depth, out_alpha, nullptr,
                                                         nullptr, state);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

size_t gm_composite_hybrid_bwd_ws(int32_t width, int32_t height)
{
    const int64_t T = div_up(width > 0 ? width : 1, GM_TILE) * div_up(height > 0 ? height : 1, GM_TILE);
    return 2 * align_up(sizeof(int32_t) * (size_t)T, 256);
}

gm_status gm_composite_hybrid_bwd(const gm_camera* cam, int32_t N, const float* rec, const int32_t* tile_ranges,
                                  const int32_t* sorted_ids, const int32_t* face_id, const float* depth,
                                  float softness, const float* state_T, const int32_t* state_last,
                                  const float* state_cm, const float* g_rgb, const float* g_depth,
                                  const float* g_alpha, float* g_rec, float* g_mesh_rgb, float* g_mesh_depth,
                                  void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    CompParams P;
    if (gm_status s = bwd_params(P, cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T,
                                 state_last, state_cm, g_rgb, g_rec))
        return s;
    int32_t *walk, *order;
    if (gm_status s = tile_order_ws(cam, ws, ws_bytes, &walk, &order)) return s;
    return bwd_launch(P, N, state_T, state_last, state_cm, g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth,
                      walk, order, stream);
}

gm_status gm_composite_hybrid_bwd_noalloc(const gm_camera* cam, int32_t N, const float* rec,
                                          const int32_t* tile_ranges, const int32_t* sorted_ids,
                                          const int32_t* face_id, const float* depth, float softness,
                                          const float* state_T, const int32_t* state_last, const float* state_cm,
                                          const float* g_rgb, const float* g_depth, const float* g_alpha,
                                          float* g_rec, float* g_mesh_rgb, float* g_mesh_depth, hipStream_t stream)
{
    clear_error();
    CompParams P;
    if (gm_status s = bwd_params(P, cam, N, rec, tile_ranges, sorted_ids, face_id, depth, softness, state_T,
                                 state_last, state_cm, g_rgb, g_rec))
        return s;
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    GM_ARG_CHECK(T <= GM_NOALLOC_MAX_TILES, "%dx%d image has %lld tiles, above the fixed scratch's %d", cam->width,
                 cam->height, (long long)T, GM_NOALLOC_MAX_TILES);
    int32_t* base = nullptr;
    if (gm_status s = noalloc_scratch(stream, &base)) return s;
    return bwd_launch(P, N, state_T, state_last, state_cm, g_rgb, g_depth, g_alpha, g_rec, g_mesh_rgb, g_mesh_depth,
                      base, base + GM_NOALLOC_MAX_TILES, stream);
}

gm_status gm_composite_hybrid_bwd_aa(const gm_camera* cam, int32_t N, const float* rec, const int32_t* tile_ranges,
                                     const int32_t* sorted_ids, const float* layer, const float* bg, float softness,
                                     const float* state, const float* g_rgb, const float* g_depth,
                                     const float* g_alpha, float* g_rec, float* g_layer, void* ws, size_t ws_bytes,
                                     hipStream_t stream)
{
    clear_error();
    CompParams P;
    if (gm_status s = fill_params_aa(P, cam, rec, tile_ranges, sorted_ids, layer, bg, softness)) return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(state && g_rgb && g_layer, "state, g_rgb or g_layer is NULL");
    GM_ARG_CHECK(((uintptr_t)state & 15) == 0 && ((uintptr_t)g_layer & 15) == 0,
                 "state and g_layer must be 16-byte aligned");
    GM_ARG_CHECK(N == 0 || g_rec, "g_rec is NULL");
    const int64_t T = (int64_t)P.cam.tx * P.cam.ty;
    int32_t *walk, *order;
    if (gm_status s = tile_order_ws(cam, ws, ws_bytes, &walk, &order)) return s;
    const int64_t n = N > 0 ? (int64_t)N * GM_GRAD : 0;
    k_tile_walk<true><<<(unsigned)T, CT, 0, stream>>>(P, nullptr, state, walk, g_rec, n);
    GM_LAUNCH_CHECK();
    k_tile_order<<<1, TO_THREADS, 0, stream>>>((int)T, walk, order);
    GM_LAUNCH_CHECK();
    k_composite_bwd<true><<<(unsigned)T, CT, 0, stream>>>(P, nullptr, nullptr, nullptr, layer, state, g_rgb, g_depth,
                                                         g_alpha, g_rec, nullptr, nullptr, g_layer, order);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

}  // extern "C"
