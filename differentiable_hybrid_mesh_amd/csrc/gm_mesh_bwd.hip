// Mesh side of the backward: from dL/dc_m and dL/dD per pixel to the gradients of
// the vertex positions, vertex colours, vertex normals, texture coordinates, texels
// and the point light (gmesh README, "Design Details": the surface colour comes from
// perspective-correct barycentrics of the nearest triangle, vertex colours or a
// trilinear mip-mapped texture, per-pixel Phong shading of interpolated normals;
// the mesh depth D enters the hybrid composite through the split; the renderer is
// differentiable with respect to the mesh as well).
//
// One block per 16 x 16 pixel tile, one thread per pixel; a covered pixel
// re-evaluates its surface in fp64 (the barycentric chain divides by the triangle's
// area and by depths, and the level of detail must select the same pyramid levels as
// the forward's definition) and runs the reverse mode.  Corner gradients are summed
// over each run of one face within a wave, then per vertex (and texture vertex) in an
// LDS table of the block, which adds its totals to global memory with float atomics;
// texel gradients go straight to global atomics; the light's 13 gradients are summed
// per block first.  Texel gradients
// land on the two pyramid levels each lookup used, and a level-by-level pass then
// hands every coarse texel's gradient down to its 2x2 children (the adjoint of the
// box-filter pyramid), so level 0 ends up holding dL/dtexture.  Visibility and the
// level of detail are taken as given (no gradient), as in the reverse mode's
// definition.  Value arithmetic only, so contraction is on.
#include "gm_internal.h"

namespace gm {

constexpr int MB_THREADS = 256;
constexpr int MB_TILE = 16;  // a block covers a 16 x 16 pixel tile, a wave 16 x 4 of it
// LDS table slots per block: a 16 x 16 tile of a dense mesh shows a few dozen
// vertices (hundreds at a limb of tiny, foreshortened triangles); a key that finds
// the table full goes straight to a global atomic.
constexpr int MB_SLOTS_LOG2 = 9;
constexpr int MB_SLOTS = 1 << MB_SLOTS_LOG2;
static_assert(MB_TILE * MB_TILE == MB_THREADS, "one thread per pixel of the tile");

struct MeshBwdParams {
    DevCamera cam;
    int V, F, Vt, S, nlev;
    const float* verts;
    const int32_t* faces;
    const float* vcolor;
    const float* vnormal;
    const float* uv;
    const int32_t* faces_uv;
    const float* mips;
    int lit;
    double lpos[3], lamb[3], ldif[3], lspec[3], lshin;
    // the camera widened to fp64 on the host: uniform operands stay in scalar
    // registers instead of taking vector registers from the per-pixel chain
    double R[9], t[3], fx, fy, cx, cy, ifx, ify;
};

__host__ __device__ inline size_t level_offset(int S, int l)
{
    size_t o = 0;
    for (int k = 0; k < l; ++k) o += (size_t)(S >> k) * (S >> k) * 3;
    return o;
}

// Bilinear lookup (clamp to edge) with its texel indices, weights and d/d(u, v).
struct Bilin {
    int idx[4];
    double wgt[4];
    double col[3], du[3], dv[3];
};

__device__ inline void bilin(const float* __restrict__ lvl, int s, double u, double v, Bilin& b)
{
    const double cu = fmin(fmax(u, 0.0), 1.0), cv = fmin(fmax(v, 0.0), 1.0);
    const double su = (u > 0.0 && u < 1.0) ? 1.0 : 0.0, sv = (v > 0.0 && v < 1.0) ? 1.0 : 0.0;
    const double x = cu * s - 0.5, y = cv * s - 0.5;
    const double x0 = floor(x), y0 = floor(y);
    const double ax = x - x0, ay = y - y0;
    int ix0 = (int)x0, iy0 = (int)y0;
    const int ix1 = min(max(ix0 + 1, 0), s - 1), iy1 = min(max(iy0 + 1, 0), s - 1);
    ix0 = min(max(ix0, 0), s - 1);
    iy0 = min(max(iy0, 0), s - 1);
    b.idx[0] = (iy0 * s + ix0) * 3;
    b.idx[1] = (iy0 * s + ix1) * 3;
    b.idx[2] = (iy1 * s + ix0) * 3;
    b.idx[3] = (iy1 * s + ix1) * 3;
    b.wgt[0] = (1.0 - ax) * (1.0 - ay);
    b.wgt[1] = ax * (1.0 - ay);
    b.wgt[2] = (1.0 - ax) * ay;
    b.wgt[3] = ax * ay;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const double t00 = lvl[b.idx[0] + c], t01 = lvl[b.idx[1] + c];
        const double t10 = lvl[b.idx[2] + c], t11 = lvl[b.idx[3] + c];
        const double top = t00 + (t01 - t00) * ax, bot = t10 + (t11 - t10) * ax;
        b.col[c] = top + (bot - top) * ay;
        b.du[c] = ((t01 - t00) * (1.0 - ay) + (t11 - t10) * ay) * s * su;
        b.dv[c] = (bot - top) * s * sv;
    }
}

// 1/x in fp64: the hardware's reciprocal estimate refined by two Newton-Raphson
// steps (r <- r + r (1 - x r)), each of which squares the relative error, so the
// result is correct to within an ulp or two (the quotients here are values, not
// decisions); x is a depth, a triangle's doubled area or a sum of perspective
// weights, never zero, infinite or subnormal at a covered pixel.
__device__ __forceinline__ double rcp64(double x)
{
    double r = __builtin_amdgcn_rcp(x);
    double e = __builtin_fma(-x, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-x, r, 1.0);
    return __builtin_fma(r, e, r);
}

__device__ __forceinline__ void addf(float* p, double v)
{
    if (v != 0.0) unsafeAtomicAdd(p, (float)v);
}

// Which per-corner gradient planes a variant produces: position (0-2) always,
// vertex colour (3-5) when untextured, normal (6-8) when lit, uv (9-10) when textured.
template <bool TEX, bool LIT>
__device__ __forceinline__ constexpr bool plane_live(int j)
{
    return j < 3 || (j < 6 ? !TEX : (j < 9 ? LIT : TEX));
}

// Per-vertex planes a variant sums in its LDS table: position, then colour when
// untextured, then normal when lit.
template <bool TEX, bool LIT>
__device__ __forceinline__ constexpr int vertex_planes()
{
    return 3 + (TEX ? 0 : 3) + (LIT ? 3 : 0);
}

// Table plane of corner-gradient plane j (0-8; not uv).
template <bool TEX, bool LIT>
__device__ __forceinline__ constexpr int vertex_plane(int j)
{
    return j < 3 ? j : (j < 6 ? j : (TEX ? j - 3 : j));
}

// Slot of `key` in an open-addressed LDS table of MB_SLOTS entries (empty = -1),
// claiming a free one on first sight; -1 when a whole probe sequence finds neither
// the key nor a free slot (the caller then adds to global memory).
__device__ __forceinline__ int table_slot(int* keys, int key)
{
    unsigned h = ((unsigned)key * 2654435761u) >> (32 - MB_SLOTS_LOG2);
    for (int probe = 0; probe < MB_SLOTS; ++probe) {
        const int seen = keys[h];
        if (seen == key) return (int)h;
        if (seen == -1) {
            const int old = atomicCAS(&keys[h], -1, key);
            if (old == -1 || old == key) return (int)h;
        }
        h = (h + 1) & (MB_SLOTS - 1);
    }
    return -1;
}

// DPP move of v (CTRL) into the rows of ROWMASK; lanes without a source read 0.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp0(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, false));
}

// One variant per (textured, lit) pair, so that each holds only its own state.
template <bool TEX, bool LIT>
__global__ void __launch_bounds__(MB_THREADS, TEX ? 2 : 3)
k_mesh_bwd(MeshBwdParams P, const int32_t* __restrict__ face_id, const float* __restrict__ g_rgb,
           const float* __restrict__ g_depth, float* __restrict__ g_verts, float* __restrict__ g_vcolor,
           float* __restrict__ g_vnormal, float* __restrict__ g_uv, float* __restrict__ g_mips,
           float* __restrict__ g_light)
{
    constexpr int NVP = vertex_planes<TEX, LIT>();
    __shared__ float s_light[13][MB_THREADS / 64];
    __shared__ int s_vkey[MB_SLOTS];
    __shared__ float s_vval[NVP][MB_SLOTS];
    __shared__ int s_tkey[TEX ? MB_SLOTS : 1];
    __shared__ float s_tval[2][TEX ? MB_SLOTS : 1];
    const int W = P.cam.width, H = P.cam.height;
    const int tiles_x = (W + MB_TILE - 1) / MB_TILE;
    const int px = (int)(blockIdx.x % tiles_x) * MB_TILE + (int)(threadIdx.x % MB_TILE);
    const int py = (int)(blockIdx.x / tiles_x) * MB_TILE + (int)(threadIdx.x / MB_TILE);
    const int pix = py * W + px;
    const bool inside = px < W && py < H;
    const int f = inside ? face_id[pix] : -1;
    // the upstream gradients depend on the pixel only: loaded beside its face id
    float gzf = 0.0f, gcf[3] = {0.0f, 0.0f, 0.0f};
    if (inside) {
        if (g_depth) gzf = g_depth[pix];
        if (g_rgb)
#pragma unroll
            for (int c = 0; c < 3; ++c) gcf[c] = g_rgb[3 * pix + c];
    }
    // a tile the mesh does not reach has nothing to add (uniform exit, before any
    // table work)
    if (!__syncthreads_or(f >= 0)) return;
    for (int s = threadIdx.x; s < MB_SLOTS; s += MB_THREADS) {
        s_vkey[s] = -1;
#pragma unroll
        for (int p = 0; p < NVP; ++p) s_vval[p][s] = 0.0f;
        if (TEX) {
            s_tkey[s] = -1;
            s_tval[0][s] = 0.0f;
            s_tval[1][s] = 0.0f;
        }
    }
    float gl[13];
#pragma unroll
    for (int i = 0; i < 13; ++i) gl[i] = 0.0f;
    // per-corner gradients of this pixel: position (3), colour (3), normal (3), uv (2)
    float acc[3][11];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int j = 0; j < 11; ++j) acc[k][j] = 0.0f;
    int vi[3] = {0, 0, 0}, ti[3] = {0, 0, 0};
    if (f >= 0) {
        const double pu = px + 0.5, pv = py + 0.5;
        const double* R = P.R;
        const double* t = P.t;
        const double fx = P.fx, fy = P.fy, cx = P.cx, cy = P.cy;
        const double rx = (pu - cx) * P.ifx, ry = (pv - cy) * P.ify;  // the pixel's ray, z = 1
        // ---- forward ---------------------------------------------------------------
        // reciprocals taken once (the chain below multiplies by them: these are
        // values, not decisions, so the rounding order is free)
        double xc[3][3], u[3], v[3], z[3], iz[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) vi[k] = P.faces[k * P.F + f];
        // everything the corners index goes out in one batch (positions, colours,
        // normals): one round trip, which the scheduler must not split
        float vpos[3][3], vcol[3][3] = {}, vnor[3][3] = {};
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int c = 0; c < 3; ++c) vpos[k][c] = P.verts[c * P.V + vi[k]];
        if constexpr (LIT)
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int c = 0; c < 3; ++c) vnor[k][c] = P.vnormal[c * P.V + vi[k]];
        if (!TEX && P.vcolor)  // the same for every thread
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int c = 0; c < 3; ++c) vcol[k][c] = P.vcolor[c * P.V + vi[k]];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const double X0 = vpos[k][0], X1 = vpos[k][1], X2 = vpos[k][2];
#pragma unroll
            for (int r = 0; r < 3; ++r) xc[k][r] = R[3 * r] * X0 + R[3 * r + 1] * X1 + R[3 * r + 2] * X2 + t[r];
            z[k] = xc[k][2];
            iz[k] = rcp64(z[k]);
            u[k] = fx * xc[k][0] * iz[k] + cx;
            v[k] = fy * xc[k][1] * iz[k] + cy;
        }
        const int ea[3] = {1, 2, 0}, eb[3] = {2, 0, 1};  // edge opposite corner k
        double lam[3], w[3], Wsum = 0.0;
        const double A = (u[1] - u[0]) * (v[2] - v[0]) - (v[1] - v[0]) * (u[2] - u[0]);
        const double iA = rcp64(A);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int a = ea[k], b = eb[k];
            const double E = (u[b] - u[a]) * (pv - v[a]) - (v[b] - v[a]) * (pu - u[a]);
            lam[k] = E * iA;
            w[k] = lam[k] * iz[k];
            Wsum += w[k];
        }
        const double zz = rcp64(Wsum);
        double bb[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) bb[k] = w[k] * zz;

        double gc[3], gz = gzf;
#pragma unroll
        for (int c = 0; c < 3; ++c) gc[c] = gcf[c];
        double gb[3] = {0.0, 0.0, 0.0}, gbase[3];

        // base colour (forward values needed by the lighting's backward)
        double base[3] = {0.0, 0.0, 0.0};
        constexpr bool textured = TEX;
        Bilin B0, B1;
        int l0 = 0, l1 = 0;
        double tl = 0.0, uvk[3][2], uu = 0.0, vv = 0.0;
        if constexpr (textured) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                ti[k] = P.faces_uv[k * P.F + f];
                uvk[k][0] = P.uv[ti[k]];
                uvk[k][1] = P.uv[P.Vt + ti[k]];
                uu += bb[k] * uvk[k][0];
                vv += bb[k] * uvk[k][1];
            }
            double dux = 0.0, dvx = 0.0, duy = 0.0, dvy = 0.0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const double dwx = (-(v[eb[k]] - v[ea[k]]) * iA) * iz[k];
                const double dwy = ((u[eb[k]] - u[ea[k]]) * iA) * iz[k];
                dux += dwx * (uvk[k][0] - uu) * zz;
                dvx += dwx * (uvk[k][1] - vv) * zz;
                duy += dwy * (uvk[k][0] - uu) * zz;
                dvy += dwy * (uvk[k][1] - vv) * zz;
            }
            const double S0 = P.S;
            const double lx = sqrt(S0 * dux * S0 * dux + S0 * dvx * S0 * dvx);
            const double ly = sqrt(S0 * duy * S0 * duy + S0 * dvy * S0 * dvy);
            const double rho = fmax(lx, ly);
            const double lmax = P.nlev - 1;
            double lod = rho > 0.0 ? log2(rho) : 0.0;
            lod = fmin(fmax(lod, 0.0), lmax);
            l0 = (int)floor(lod);
            l1 = min(l0 + 1, P.nlev - 1);
            tl = lod - l0;
            bilin(P.mips + level_offset(P.S, l0), P.S >> l0, uu, vv, B0);
            bilin(P.mips + level_offset(P.S, l1), P.S >> l1, uu, vv, B1);
#pragma unroll
            for (int c = 0; c < 3; ++c) base[c] = B0.col[c] + (B1.col[c] - B0.col[c]) * tl;
        } else if (P.vcolor) {
#pragma unroll
            for (int c = 0; c < 3; ++c)
#pragma unroll
                for (int k = 0; k < 3; ++k) base[c] += bb[k] * vcol[k][c];
        }

        // ---- lighting (fp32: well conditioned): forward values, then reverse ---------------
        if constexpr (LIT) {
            const float* Rf = P.cam.R;
            float nw[3], nt[3], L[3], x[3], lt[3], et[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                nw[c] = 0.0f;
#pragma unroll
                for (int k = 0; k < 3; ++k) nw[c] += (float)bb[k] * vnor[k][c];
            }
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                nt[r] = Rf[3 * r] * nw[0] + Rf[3 * r + 1] * nw[1] + Rf[3 * r + 2] * nw[2];
                L[r] = Rf[3 * r] * (float)P.lpos[0] + Rf[3 * r + 1] * (float)P.lpos[1] + Rf[3 * r + 2] * (float)P.lpos[2] +
                       P.cam.t[r];
            }
            const float zf = (float)zz;
            x[0] = (float)rx * zf;
            x[1] = (float)ry * zf;
            x[2] = zf;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                lt[r] = L[r] - x[r];
                et[r] = -x[r];
            }
            const float nn = sqrtf(nt[0] * nt[0] + nt[1] * nt[1] + nt[2] * nt[2]);
            const float ln = sqrtf(lt[0] * lt[0] + lt[1] * lt[1] + lt[2] * lt[2]);
            const float en = sqrtf(et[0] * et[0] + et[1] * et[1] + et[2] * et[2]);
            const float inn = 1.0f / nn, iln = 1.0f / ln, ien = 1.0f / en;
            float n[3], l[3], e[3], rv[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                n[r] = nt[r] * inn;
                l[r] = lt[r] * iln;
                e[r] = et[r] * ien;
            }
            const float ndl = n[0] * l[0] + n[1] * l[1] + n[2] * l[2];
#pragma unroll
            for (int r = 0; r < 3; ++r) rv[r] = 2.0f * ndl * n[r] - l[r];
            const float rde = rv[0] * e[0] + rv[1] * e[1] + rv[2] * e[2];
            const float diff = ndl > 0.0f ? ndl : 0.0f;
            const bool spec_on = ndl > 0.0f && rde > 0.0f;
            const float shin = (float)P.lshin;
            const float spec = spec_on ? __powf(rde, shin) : 0.0f;
            float gdiff = 0.0f, gspec = 0.0f;
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const float g = (float)gc[c], bs = (float)base[c];
                gbase[c] = gc[c] * (P.lamb[c] + P.ldif[c] * diff);
                gl[3 + c] = g * bs;
                gl[6 + c] = g * bs * diff;
                gl[9 + c] = g * spec;
                gdiff += g * bs * (float)P.ldif[c];
                gspec += g * (float)P.lspec[c];
            }
            float gndl = ndl > 0.0f ? gdiff : 0.0f, grde = 0.0f;
            if (spec_on) {
                grde = gspec * shin * (spec / rde);  // d rde^s / d rde = s rde^(s-1)
                gl[12] = gspec * spec * __logf(rde);
            }
            float gn[3], glv[3], ge[3], rn = 0.0f;
#pragma unroll
            for (int r = 0; r < 3; ++r) {  // rde = r . e, r = 2 ndl n - l
                const float grr = grde * e[r];
                ge[r] = grde * rv[r];
                rn += grr * n[r];
                gn[r] = 2.0f * ndl * grr;
                glv[r] = -grr;
            }
            gndl += 2.0f * rn;
            float dn = 0.0f, dl = 0.0f, de = 0.0f;
#pragma unroll
            for (int r = 0; r < 3; ++r) {  // ndl = n . l
                gn[r] += gndl * l[r];
                glv[r] += gndl * n[r];
                dn += n[r] * gn[r];
                dl += l[r] * glv[r];
                de += e[r] * ge[r];
            }
            float gnt[3], glt[3], get[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {  // normalisations
                gnt[r] = (gn[r] - n[r] * dn) * inn;
                glt[r] = (glv[r] - l[r] * dl) * iln;
                get[r] = (ge[r] - e[r] * de) * ien;
            }
            float gnw[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {  // nt = R nw, L = R pos + t
                gnw[j] = Rf[j] * gnt[0] + Rf[3 + j] * gnt[1] + Rf[6 + j] * gnt[2];
                gl[j] = Rf[j] * glt[0] + Rf[3 + j] * glt[1] + Rf[6 + j] * glt[2];
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {  // nw = sum b_k normal_k
                float sum = 0.0f;
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    sum += vnor[k][c] * gnw[c];
                    acc[k][6 + c] = (float)bb[k] * gnw[c];
                }
                gb[k] += sum;
            }
            // x = ((pu - cx)/fx z, (pv - cy)/fy z, z); lt = L - x, et = -x
            const float gx0 = -glt[0] - get[0], gx1 = -glt[1] - get[1], gx2 = -glt[2] - get[2];
            gz += gx0 * rx + gx1 * ry + gx2;
        } else {
#pragma unroll
            for (int c = 0; c < 3; ++c) gbase[c] = gc[c];
        }

        // ---- base colour ---------------------------------------------------------------
        if constexpr (textured) {
            double guu = 0.0, gvv = 0.0;
            float* m0 = g_mips ? g_mips + level_offset(P.S, l0) : nullptr;
            float* m1 = g_mips ? g_mips + level_offset(P.S, l1) : nullptr;
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const double a0 = gbase[c] * (1.0 - tl), a1 = gbase[c] * tl;
                guu += a0 * B0.du[c] + a1 * B1.du[c];
                gvv += a0 * B0.dv[c] + a1 * B1.dv[c];
                if (g_mips)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        addf(&m0[B0.idx[q] + c], a0 * B0.wgt[q]);
                        addf(&m1[B1.idx[q] + c], a1 * B1.wgt[q]);
                    }
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                gb[k] += uvk[k][0] * guu + uvk[k][1] * gvv;
                acc[k][9] = (float)(bb[k] * guu);
                acc[k][10] = (float)(bb[k] * gvv);
            }
        } else if (P.vcolor) {
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    gb[k] += vcol[k][c] * gbase[c];
                    acc[k][3 + c] = (float)(bb[k] * gbase[c]);
                }
        }

        // ---- vertex positions: b_k = w_k z, z = 1/W, w_k = lam_k / z_k, lam_k = E_k / A
        if (g_verts) {
            double gw[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                gw[k] = gb[k] * zz;
                gz += gb[k] * w[k];
            }
            const double gW = -gz * zz * zz;
            double glam[3], gzk[3], gu[3] = {0.0, 0.0, 0.0}, gv[3] = {0.0, 0.0, 0.0}, gA = 0.0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                gw[k] += gW;
                glam[k] = gw[k] * iz[k];
                gzk[k] = -gw[k] * lam[k] * (iz[k] * iz[k]);
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const double gE = glam[k] * iA;
                gA -= glam[k] * lam[k] * iA;
                const int a = ea[k], b = eb[k];
                gu[a] += gE * (v[b] - pv);
                gu[b] += gE * (pv - v[a]);
                gv[a] += gE * (pu - u[b]);
                gv[b] += gE * (u[a] - pu);
            }
            gu[0] += gA * (v[1] - v[2]);
            gu[1] += gA * (v[2] - v[0]);
            gu[2] += gA * (v[0] - v[1]);
            gv[0] += gA * (u[2] - u[1]);
            gv[1] += gA * (u[0] - u[2]);
            gv[2] += gA * (u[1] - u[0]);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const double i2 = iz[k] * iz[k];
                const double gxc = gu[k] * fx * iz[k], gyc = gv[k] * fy * iz[k];
                const double gzc = gzk[k] - gu[k] * fx * xc[k][0] * i2 - gv[k] * fy * xc[k][1] * i2;
#pragma unroll
                for (int j = 0; j < 3; ++j) acc[k][j] = (float)(R[j] * gxc + R[3 + j] * gyc + R[6 + j] * gzc);
            }
        }
    }
    // Pixels of one face are runs of neighbouring lanes (a triangle meets a row in an
    // interval): a segmented sum over each run leaves the run's total in its last lane,
    // which alone adds it to the face's corners (one set of atomics per run).
    __syncthreads();  // the tables are cleared
    if (__ballot(f >= 0)) {  // a wave with no covered pixel has nothing to add
        const int lane = threadIdx.x & 63;
        const int prev = __shfl_up(f, 1, 64);
        const unsigned long long heads = __ballot(lane == 0 || prev != f);
        const unsigned long long upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
        const int start = 63 - __builtin_clzll(heads & upto);
        const bool tail = lane == 63 || ((heads >> (lane + 1)) & 1ull);
        // Segmented sums over [start, lane] with DPP moves only: shifts by 1, 2, 4
        // and 8 inside each 16-lane row (Hillis-Steele, each step adding only within
        // the run), then lane 15 of each even row into the next row and lane 31 into
        // rows 2 and 3, each added where the run reaches back to that lane.  Each step
        // is taken for all planes at once and skipped (uniformly) when no run of the
        // wave reaches back that far: runs are mostly shorter than 8 lanes and rarely
        // cross a 16-lane row.
        auto each = [&](auto step) {
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int j = 0; j < 11; ++j)
                    if (plane_live<TEX, LIT>(j)) acc[k][j] = step(acc[k][j]);
        };
        const int r = lane & 15;
        const bool s1 = r >= 1 && lane - 1 >= start, s2 = r >= 2 && lane - 2 >= start,
                   s4 = r >= 4 && lane - 4 >= start, s8 = r >= 8 && lane - 8 >= start,
                   b15 = (lane & 16) && start <= (lane & ~15) - 1, b31 = lane >= 32 && start <= 31;
        if (__ballot(s1)) each([&](float x) { const float y = dpp0<0x111>(x); return s1 ? x + y : x; });
        if (__ballot(s2)) each([&](float x) { const float y = dpp0<0x112>(x); return s2 ? x + y : x; });
        if (__ballot(s4)) each([&](float x) { const float y = dpp0<0x114>(x); return s4 ? x + y : x; });
        if (__ballot(s8)) each([&](float x) { const float y = dpp0<0x118>(x); return s8 ? x + y : x; });
        if (__ballot(b15)) each([&](float x) { const float y = dpp0<0x142, 0xa>(x); return b15 ? x + y : x; });
        if (__ballot(b31)) each([&](float x) { const float y = dpp0<0x143, 0xc>(x); return b31 ? x + y : x; });
        // Run totals go into the block's LDS tables keyed by vertex (and texture
        // vertex): a vertex's faces meet inside one tile, so its many runs become one
        // set of global atomics when the block flushes.
        if (tail && f >= 0) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int s = table_slot(s_vkey, vi[k]);
#pragma unroll
                for (int j = 0; j < 9; ++j) {
                    if (!plane_live<TEX, LIT>(j) || acc[k][j] == 0.0f) continue;
                    if (s >= 0) {
                        atomicAdd(&s_vval[vertex_plane<TEX, LIT>(j)][s], acc[k][j]);
                    } else {
                        float* g = j < 3 ? g_verts : (j < 6 ? g_vcolor : g_vnormal);
                        if (g) unsafeAtomicAdd(&g[(j % 3) * P.V + vi[k]], acc[k][j]);
                    }
                }
                if (TEX) {
                    const int st = table_slot(s_tkey, ti[k]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (acc[k][9 + j] == 0.0f) continue;
                        if (st >= 0) atomicAdd(&s_tval[j][st], acc[k][9 + j]);
                        else if (g_uv) unsafeAtomicAdd(&g_uv[j * P.Vt + ti[k]], acc[k][9 + j]);
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int s = threadIdx.x; s < MB_SLOTS; s += MB_THREADS) {
        const int v = s_vkey[s];
        if (v >= 0) {
#pragma unroll
            for (int j = 0; j < 9; ++j) {
                if (!plane_live<TEX, LIT>(j)) continue;
                float* g = j < 3 ? g_verts : (j < 6 ? g_vcolor : g_vnormal);
                const float x = s_vval[vertex_plane<TEX, LIT>(j)][s];
                if (g && x != 0.0f) unsafeAtomicAdd(&g[(j % 3) * P.V + v], x);
            }
        }
        if (TEX) {
            const int t = s_tkey[s];
            if (t >= 0 && g_uv) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (s_tval[j][s] != 0.0f) unsafeAtomicAdd(&g_uv[j * P.Vt + t], s_tval[j][s]);
            }
        }
    }
    // light: per-wave sums (one halving reduction of the 13 values), then per-block atomics
    if (g_light) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        float g16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) g16[i] = i < 13 ? gl[i] : 0.0f;
        const float s = wave_sum16(g16, lane);
        if ((lane & 3) == 0 && (lane >> 2) < 13) s_light[lane >> 2][wave] = s;
        __syncthreads();
        if (threadIdx.x < 13) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < MB_THREADS / 64; ++w) s += s_light[threadIdx.x][w];
            if (s != 0.0f) unsafeAtomicAdd(&g_light[threadIdx.x], s);
        }
    }
}

// Adjoint of one pyramid step: fine[2y + a][2x + b] += coarse[y][x] / 4.
__global__ void k_pyramid_adjoint(float* __restrict__ fine, const float* __restrict__ coarse, int s)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int sf = 2 * s;
    if (i >= sf * sf * 3) return;
    const int c = i % 3, x = (i / 3) % sf, y = i / (3 * sf);
    fine[i] += 0.25f * coarse[((y >> 1) * s + (x >> 1)) * 3 + c];
}

// Clears of the gradient outputs, all in one launch: buffer j is zeroed over its n[j]
// floats (absent buffers have n[j] = 0).
constexpr int MB_NZERO = 6;
struct ZeroList {
    float* p[MB_NZERO];
    int64_t n[MB_NZERO];
};

__global__ void k_zero(ZeroList z)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int j = 0; j < MB_NZERO; ++j)
        if (i < z.n[j]) z.p[j][i] = 0.0f;
}

static gm_status zero(const ZeroList& z, hipStream_t stream)
{
    int64_t n = 0;
    for (int j = 0; j < MB_NZERO; ++j) n = std::max(n, z.n[j]);
    if (n <= 0) return GM_OK;
    k_zero<<<(unsigned)div_up(n, 256), 256, 0, stream>>>(z);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

}  // namespace gm

using namespace gm;

extern "C" gm_status gm_mesh_bwd(const gm_camera* cam, const gm_mesh* mesh, const gm_light* light,
                                 const int32_t* face_id, const float* g_mesh_rgb, const float* g_mesh_depth,
                                 float* g_verts, float* g_vcolor, float* g_vnormal, float* g_uv, float* g_mips,
                                 float* g_light, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(mesh != nullptr && face_id != nullptr, "mesh / face_id is NULL");
    GM_ARG_CHECK(mesh->V >= 0 && mesh->F >= 0, "negative mesh size");
    GM_ARG_CHECK(mesh->F == 0 || (mesh->verts && mesh->faces), "verts / faces is NULL");
    GM_ARG_CHECK(!g_vcolor || mesh->vcolor, "g_vcolor needs vertex colours");
    GM_ARG_CHECK(!g_vnormal || (mesh->vnormal && light), "g_vnormal needs normals and a light");
    GM_ARG_CHECK(!g_light || light, "g_light needs a light");
    GM_ARG_CHECK(!(g_uv || g_mips) || mesh->mips, "g_uv / g_mips need a textured mesh");
    MeshBwdParams P{};
    P.cam = dev_camera(*cam);
    for (int i = 0; i < 9; ++i) P.R[i] = P.cam.R[i];
    for (int i = 0; i < 3; ++i) P.t[i] = P.cam.t[i];
    P.fx = P.cam.fx;
    P.fy = P.cam.fy;
    P.cx = P.cam.cx;
    P.cy = P.cam.cy;
    P.ifx = 1.0 / P.fx;
    P.ify = 1.0 / P.fy;
    P.V = mesh->V;
    P.F = mesh->F;
    P.verts = mesh->verts;
    P.faces = mesh->faces;
    P.vcolor = mesh->vcolor;
    P.vnormal = mesh->vnormal;
    if (mesh->mips) {
        GM_ARG_CHECK(mesh->uv && mesh->faces_uv, "textured mesh needs uv and faces_uv");
        GM_ARG_CHECK(mesh->tex_size > 0 && (mesh->tex_size & (mesh->tex_size - 1)) == 0,
                     "tex_size %d is not a power of two", mesh->tex_size);
        P.Vt = mesh->Vt;
        P.S = mesh->tex_size;
        P.uv = mesh->uv;
        P.faces_uv = mesh->faces_uv;
        P.mips = mesh->mips;
        for (int s = P.S; s >= 1; s >>= 1) ++P.nlev;
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
    const size_t nmips = P.mips ? gm_mipmaps_floats(P.S) : 0;
    ZeroList z{{g_verts, g_vcolor, g_vnormal, g_uv, g_mips, g_light},
               {3 * (int64_t)P.V, 3 * (int64_t)P.V, 3 * (int64_t)P.V, 2 * (int64_t)P.Vt, (int64_t)nmips, 13}};
    for (int j = 0; j < MB_NZERO; ++j)
        if (!z.p[j]) z.n[j] = 0;
    if (gm_status s = zero(z, stream)) return s;
    if (P.F > 0) {
        const bool tex = P.mips != nullptr, lit = P.lit && P.vnormal;
        auto kern = tex ? (lit ? k_mesh_bwd<true, true> : k_mesh_bwd<true, false>)
                        : (lit ? k_mesh_bwd<false, true> : k_mesh_bwd<false, false>);
        const int64_t tiles = div_up(cam->width, MB_TILE) * div_up(cam->height, MB_TILE);
        kern<<<(unsigned)tiles, MB_THREADS, 0, stream>>>(
            P, face_id, g_mesh_rgb, g_mesh_depth, g_verts, g_vcolor, lit ? g_vnormal : nullptr, g_uv, g_mips,
            lit ? g_light : nullptr);
        GM_LAUNCH_CHECK();
    }
    if (g_mips && P.nlev > 1) {  // coarse to fine: level l - 1 += adjoint(level l)
        for (int l = P.nlev - 1; l >= 1; --l) {
            const int s = P.S >> l;
            const int64_t nf = (int64_t)(2 * s) * (2 * s) * 3;
            k_pyramid_adjoint<<<(unsigned)div_up(nf, 256), 256, 0, stream>>>(g_mips + level_offset(P.S, l - 1),
                                                                            g_mips + level_offset(P.S, l), s);
            GM_LAUNCH_CHECK();
        }
    }
    return GM_OK;
}
