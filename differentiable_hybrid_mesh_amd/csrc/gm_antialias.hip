// Analytic edge antialiasing of the mesh and its reverse mode (gmesh README,
// "Design Details > Mesh rasterizer", step 3: for every pair of neighbouring pixels
// that sees a silhouette, the crossing of the front surface's edge between the two
// pixel centres gives a fractional coverage and blends over the farther surface;
// internal edges of a connected surface are left alone; "Limitations and Todos":
// per-axis 1D approximation; "Hybrid rendering": a_m is fractional at silhouettes).
//
// The per-pair rules (front pixel, following the segment over internal edges to the
// first silhouette edge, the axis split, the 1D box filter, the clamp and the split
// depth of pixels that receive coverage) are those of include/gm.h.  Decisions and
// crossings are fp64 from the fp32 screen vertices, in the written order with no
// contraction; every pixel gathers the effects of its four pairs, so no atomics are
// needed in the forward.
//
// Edge adjacency is built once per mesh with an open-addressing hash table keyed by
// the edge's two vertex indices.
#pragma clang fp contract(off)

#include "gm_internal.h"

namespace gm {

// ---------------------------------------------------------------------------
// edge adjacency
// ---------------------------------------------------------------------------
constexpr unsigned long long EMPTY_KEY = ~0ull;

struct AdjTable {
    unsigned long long* keys;
    int* count;
    int* faces;  // [2 * cap]
    uint32_t mask;
};

static size_t adj_capacity(int32_t F)
{
    size_t need = 2 * 3 * (size_t)(F > 0 ? F : 1), cap = 1024;
    while (cap < need) cap <<= 1;
    return cap;
}

static AdjTable adj_table(void* ws, size_t cap)
{
    char* p = (char*)ws;
    AdjTable t;
    t.keys = (unsigned long long*)p;
    p += align_up(cap * 8, 256);
    t.count = (int*)p;
    p += align_up(cap * 4, 256);
    t.faces = (int*)p;
    t.mask = (uint32_t)(cap - 1);
    return t;
}

// SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): a well-mixed slot from the 64-bit edge key.
__device__ __forceinline__ uint32_t slot_of(unsigned long long k)
{
    k ^= k >> 30;
    k *= 0xbf58476d1ce4e5b9ull;
    k ^= k >> 27;
    k *= 0x94d049bb133111ebull;
    k ^= k >> 31;
    return (uint32_t)k;
}

__device__ __forceinline__ unsigned long long edge_key(const int32_t* faces, int F, int f, int k)
{
    const int c1 = k == 2 ? 0 : k + 1, c2 = k == 0 ? 2 : k - 1;  // corners k+1, k+2 (mod 3)
    const unsigned a = (unsigned)faces[c1 * F + f], b = (unsigned)faces[c2 * F + f];
    return a < b ? ((unsigned long long)a << 32) | b : ((unsigned long long)b << 32) | a;
}

__global__ void k_adj_init(AdjTable t, int64_t cap)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < cap) {
        t.keys[i] = EMPTY_KEY;
        t.count[i] = 0;
    }
}

__global__ void k_adj_insert(AdjTable t, const int32_t* __restrict__ faces, int F)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= 3 * F) return;
    const int f = e / 3, k = e - 3 * f;
    const unsigned long long key = edge_key(faces, F, f, k);
    uint32_t h = slot_of(key) & t.mask;
    for (uint32_t probe = 0; probe <= t.mask; ++probe) {  // the table is at most half full
        const unsigned long long prev = atomicCAS(&t.keys[h], EMPTY_KEY, key);
        if (prev == EMPTY_KEY || prev == key) {
            const int n = atomicAdd(&t.count[h], 1);
            if (n < 2) t.faces[2 * h + n] = f;
            return;
        }
        h = (h + 1) & t.mask;
    }
}

__global__ void k_adj_lookup(AdjTable t, const int32_t* __restrict__ faces, int F, int32_t* __restrict__ adj)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= 3 * F) return;
    const int f = e / 3, k = e - 3 * f;
    const unsigned long long key = edge_key(faces, F, f, k);
    uint32_t h = slot_of(key) & t.mask;
    int other = -1;
    for (uint32_t probe = 0; probe <= t.mask; ++probe) {
        const unsigned long long cur = t.keys[h];
        if (cur == key) {
            const int n = t.count[h];
            other = n == 1 ? -1 : (n == 2 ? (t.faces[2 * h] == f ? t.faces[2 * h + 1] : t.faces[2 * h]) : -2);
            break;
        }
        if (cur == EMPTY_KEY) break;  // not reachable: every key was inserted
        h = (h + 1) & t.mask;
    }
    adj[k * F + f] = other;
}

// ---------------------------------------------------------------------------
// pair analysis (fp64)
// ---------------------------------------------------------------------------
constexpr int AA_MAX_WALK = 16;  // triangles followed from the front pixel's

struct AaParams {
    DevCamera cam;
    int V, F;
    const float* vs;  // [3][V]
    const int32_t* faces;
    const uint8_t* mask;
    const int32_t* adj;
    const int32_t* face_id;
    const float* depth;
    const float* colour;  // [H][W][3]
};

struct AaTri {
    double u[3], v[3];
    double sgn;
    bool valid;
};

__device__ __forceinline__ AaTri tri_of(const AaParams& P, int f)
{
    AaTri t;
    t.valid = false;
    t.sgn = 0.0;
    if (P.mask && !P.mask[f]) return t;
    bool near_ok = true;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int vi = P.faces[k * P.F + f];
        t.u[k] = (double)P.vs[vi];
        t.v[k] = (double)P.vs[P.V + vi];
        near_ok = near_ok && (P.vs[2 * P.V + vi] >= P.cam.near_z);
    }
    if (!near_ok) return t;
    const double A = (t.u[1] - t.u[0]) * (t.v[2] - t.v[0]) - (t.v[1] - t.v[0]) * (t.u[2] - t.u[0]);
    if (A == 0.0) return t;
    t.sgn = A > 0.0 ? 1.0 : -1.0;
    t.valid = true;
    return t;
}

// inside-positive edge function of edge k (corner k+1 -> corner k+2) at (pu, pv)
template <int K>
__device__ __forceinline__ double edge_fn(const AaTri& t, double pu, double pv)
{
    constexpr int i = (K + 1) % 3, j = (K + 2) % 3;
    return t.sgn * ((t.u[j] - t.u[i]) * (pv - t.v[i]) - (t.v[j] - t.v[i]) * (pu - t.u[i]));
}

struct AaPair {
    int a, b;       // front pixel, other pixel
    int face, k;    // face whose silhouette edge k is crossed
    double ea, eb;  // its edge function at the two centres
    double t;       // crossing from a's centre (0) to b's (1)
    double sgn;     // sign of that face's screen-space area
};

template <int K>
__device__ __forceinline__ void exit_candidate(const AaTri& t, double au, double av, double bu, double bv, int& ke,
                                               double& te, double& ea_e, double& eb_e)
{
    const double ea = edge_fn<K>(t, au, av), eb = edge_fn<K>(t, bu, bv);
    if (eb < ea) {
        const double tk = ea / (ea - eb);
        if (tk < te) {
            te = tk;
            ke = K;
            ea_e = ea;
            eb_e = eb;
        }
    }
}

// Pixel q is the right (axis 0) or lower (axis 1) neighbour of p.  True when the
// pair changes a coverage (t != 1/2).
__device__ bool analyse(const AaParams& P, int p, int q, int axis, AaPair& r)
{
    const int W = P.cam.width;
    const int fp = P.face_id[p], fq = P.face_id[q];
    if (fp == fq) return false;
    int a;
    if (fq < 0) a = p;
    else if (fp < 0) a = q;
    else {
        const float dp = P.depth[p], dq = P.depth[q];
        a = dp < dq ? p : (dq < dp ? q : (fp < fq ? p : q));
    }
    const int b = a == p ? q : p;
    int G = P.face_id[a];
    AaTri t = tri_of(P, G);
    if (!t.valid) return false;
    const double au = (double)(a % W) + 0.5, av = (double)(a / W) + 0.5;
    const double bu = (double)(b % W) + 0.5, bv = (double)(b / W) + 0.5;
    for (int step = 0; step < AA_MAX_WALK; ++step) {
        int ke = -1;
        double te = INFINITY, ea_e = 0.0, eb_e = 0.0;
        exit_candidate<0>(t, au, av, bu, bv, ke, te, ea_e, eb_e);
        exit_candidate<1>(t, au, av, bu, bv, ke, te, ea_e, eb_e);
        exit_candidate<2>(t, au, av, bu, bv, ke, te, ea_e, eb_e);
        if (ke < 0 || !(te < 1.0)) return false;  // G holds the rest of the segment
        const int g = P.adj[ke * P.F + G];
        AaTri tg;
        tg.valid = false;
        bool internal = false;
        if (g >= 0) {
            tg = tri_of(P, g);
            internal = tg.valid && tg.sgn == t.sgn;
        }
        if (!internal) {
            // axis: horizontal pairs take edges at least as steep as 45 degrees
            // (edge ke runs from corner ke+1 to corner ke+2)
            const double ui = ke == 0 ? t.u[1] : (ke == 1 ? t.u[2] : t.u[0]);
            const double uj = ke == 0 ? t.u[2] : (ke == 1 ? t.u[0] : t.u[1]);
            const double vi = ke == 0 ? t.v[1] : (ke == 1 ? t.v[2] : t.v[0]);
            const double vj = ke == 0 ? t.v[2] : (ke == 1 ? t.v[0] : t.v[1]);
            const double du = fabs(uj - ui), dv = fabs(vj - vi);
            if (axis == 0 ? !(dv >= du) : !(du > dv)) return false;
            if (te == 0.5) return false;
            r.a = a;
            r.b = b;
            r.face = G;
            r.k = ke;
            r.ea = ea_e;
            r.eb = eb_e;
            r.t = te;
            r.sgn = t.sgn;
            return true;
        }
        G = g;
        t = tg;
    }
    return false;
}

// The pair of pixel x in direction d (0 left, 1 right, 2 up, 3 down), with x's
// neighbour n.  Returns false when the neighbour is outside the image or the pair
// changes nothing.
__device__ __forceinline__ bool pair_of(const AaParams& P, int x, int px, int py, int d, int& n, AaPair& r)
{
    const int W = P.cam.width, H = P.cam.height;
    int p, q, axis;
    if (d == 0) {
        if (px == 0) return false;
        n = x - 1;
        p = n, q = x, axis = 0;
    } else if (d == 1) {
        if (px == W - 1) return false;
        n = x + 1;
        p = x, q = n, axis = 0;
    } else if (d == 2) {
        if (py == 0) return false;
        n = x - W;
        p = n, q = x, axis = 1;
    } else {
        if (py == H - 1) return false;
        n = x + W;
        p = x, q = n, axis = 1;
    }
    return analyse(P, p, q, axis, r);
}

// Weights of pixel x: w_self and the weights of its four neighbours' surfaces.
// mod[d]: the pair in direction d changes x (and pr[d] is that pair).
struct AaPixel {
    double wself;
    double wn[4];
    int nb[4];
    bool mod[4];
    AaPair pr[4];
};

__device__ void pixel_weights(const AaParams& P, int x, int px, int py, bool cov, AaPixel& w)
{
    w.wself = cov ? 1.0 : 0.0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        w.wn[d] = 0.0;
        w.mod[d] = false;
        w.nb[d] = -1;
        int n = -1;
        AaPair& r = w.pr[d];
        if (!pair_of(P, x, px, py, d, n, r)) continue;
        w.nb[d] = n;
        if (r.t < 0.5) {
            if (r.a != x) continue;  // the pair changes the neighbour
            const double lost = 0.5 - r.t;
            w.wself -= lost;
            if (P.face_id[r.b] >= 0) w.wn[d] += lost;
        } else {
            if (r.b != x) continue;
            const double gained = r.t - 0.5;
            w.wn[d] += gained;
            if (cov) w.wself -= gained;
        }
        w.mod[d] = true;
    }
}

__device__ __forceinline__ int neighbour_index(int x, int d, int W)
{
    return d == 0 ? x - 1 : (d == 1 ? x + 1 : (d == 2 ? x - W : x + W));
}

// ---------------------------------------------------------------------------
// forward: layer [H][W][8] = (M_r, M_g, M_b, M_D, a_m, D_split, 0, 0)
// ---------------------------------------------------------------------------
// Per-pixel record of the pairs for the reverse mode, [H][W][12]:
//   (w_self, w_left, w_right, w_up), (w_down, clamp branch as int32, raw coverage, 0),
//   four int32 codes, one per direction: -1 when that pair does not change the pixel,
//   else ((3 face + edge) << 2) | (area sign > 0) << 1 | (the pixel is the front one).
// clamp branch: 0 coverage used as is, 1 scaled down from above 1, 2 below 0 (zero).
__device__ __forceinline__ int pair_code(const AaPair& r, int x)
{
    return ((3 * r.face + r.k) << 2) | ((r.sgn > 0.0 ? 1 : 0) << 1) | (r.a == x ? 1 : 0);
}

__global__ void __launch_bounds__(256) k_antialias(AaParams P, float* __restrict__ layer,
                                                   float* __restrict__ tile_dmax, float* __restrict__ pairs)
{
    const int W = P.cam.width, H = P.cam.height;
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= W * H) return;
    const int px = x % W, py = x / W;
    const bool cov = P.face_id[x] >= 0;
    AaPixel w;
    pixel_weights(P, x, px, py, cov, w);
    double a = w.wself, M0 = 0.0, M1 = 0.0, M2 = 0.0, MD = 0.0;
    double Ds = cov ? (double)P.depth[x] : INFINITY;
    if (cov) {
        M0 = w.wself * (double)P.colour[3 * x];
        M1 = w.wself * (double)P.colour[3 * x + 1];
        M2 = w.wself * (double)P.colour[3 * x + 2];
        MD = w.wself * (double)P.depth[x];
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const double wd = w.wn[d];
        if (wd == 0.0) continue;
        const int n = w.nb[d];
        a += wd;
        M0 += wd * (double)P.colour[3 * n];
        M1 += wd * (double)P.colour[3 * n + 1];
        M2 += wd * (double)P.colour[3 * n + 2];
        const double Dn = (double)P.depth[n];
        MD += wd * Dn;
        if (!cov && wd > 0.0 && Dn < Ds) Ds = Dn;
    }
    const double s = a > 1.0 ? 1.0 / a : (a < 0.0 ? 0.0 : 1.0);
    const double ac = a > 1.0 ? 1.0 : (a < 0.0 ? 0.0 : a);
    float4* o = reinterpret_cast<float4*>(layer) + 2 * (size_t)x;
    o[0] = make_float4((float)(s * M0), (float)(s * M1), (float)(s * M2), (float)(s * MD));
    o[1] = make_float4((float)ac, (float)Ds, 0.0f, 0.0f);
    if (pairs) {
        const int branch = a > 1.0 ? 1 : (a < 0.0 ? 2 : 0);
        int code[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) code[d] = w.mod[d] ? pair_code(w.pr[d], x) : -1;
        float4* q = reinterpret_cast<float4*>(pairs) + 3 * (size_t)x;
        q[0] = make_float4((float)w.wself, (float)w.wn[0], (float)w.wn[1], (float)w.wn[2]);
        q[1] = make_float4((float)w.wn[3], __int_as_float(branch), (float)a, 0.0f);
        q[2] = make_float4(__int_as_float(code[0]), __int_as_float(code[1]), __int_as_float(code[2]),
                           __int_as_float(code[3]));
    }
    // the back layer is visible here: no occlusion cull on this tile
    if (tile_dmax && cov && ac < 1.0) tile_dmax[(py / GM_TILE) * P.cam.tx + px / GM_TILE] = INFINITY;
}

// ---------------------------------------------------------------------------
// reverse mode
// ---------------------------------------------------------------------------
// Pass 1, per pixel x, from the forward's pair record: dL/d(M, M_D) and dL/da
// before the clamp (kept in scratch [H][W][8] = (gM_r, gM_g, gM_b, gM_D, g_split
// of an uncovered pixel, direction of the neighbour giving its split depth, -, -)),
// and the crossing gradients of the pairs that change x, carried to the crossed
// edge's two screen vertices (the crossing is recomputed from the edge alone).
__global__ void __launch_bounds__(256) k_antialias_bwd1(AaParams P, const float* __restrict__ pairs,
                                                        const float* __restrict__ g_layer,
                                                        float* __restrict__ scratch, float* __restrict__ g_vs)
{
    const int W = P.cam.width, H = P.cam.height;
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= W * H) return;
    const int px = x % W, py = x / W;
    const bool cov = P.face_id[x] >= 0;
    const float4 q0 = reinterpret_cast<const float4*>(pairs)[3 * (size_t)x];
    const float4 q1 = reinterpret_cast<const float4*>(pairs)[3 * (size_t)x + 1];
    const float4 q2 = reinterpret_cast<const float4*>(pairs)[3 * (size_t)x + 2];
    const double wself = q0.x;
    const double wn[4] = {q0.y, q0.z, q0.w, q1.x};
    const int branch = __float_as_int(q1.y);
    const int code[4] = {__float_as_int(q2.x), __float_as_int(q2.y), __float_as_int(q2.z), __float_as_int(q2.w)};
    const float4 g0 = reinterpret_cast<const float4*>(g_layer)[2 * (size_t)x];
    const float4 g1 = reinterpret_cast<const float4*>(g_layer)[2 * (size_t)x + 1];
    double c[3] = {0.0, 0.0, 0.0}, Dx = 0.0;
    if (cov) {
        c[0] = P.colour[3 * x];
        c[1] = P.colour[3 * x + 1];
        c[2] = P.colour[3 * x + 2];
        Dx = P.depth[x];
    }
    double M0 = wself * c[0], M1 = wself * c[1], M2 = wself * c[2], MD = wself * Dx;
    double cn[4][4];  // neighbour colour and depth
    int nb[4];
    int dsel = -1;
    double Ds = cov ? Dx : INFINITY;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const bool has = d == 0 ? px > 0 : (d == 1 ? px < W - 1 : (d == 2 ? py > 0 : py < H - 1));
        const int n = has ? neighbour_index(x, d, W) : -1;
        nb[d] = n;
        const bool ncov = n >= 0 && P.face_id[n] >= 0;
        cn[d][0] = ncov ? (double)P.colour[3 * n] : 0.0;
        cn[d][1] = ncov ? (double)P.colour[3 * n + 1] : 0.0;
        cn[d][2] = ncov ? (double)P.colour[3 * n + 2] : 0.0;
        cn[d][3] = ncov ? (double)P.depth[n] : 0.0;
        const double wd = wn[d];
        if (wd == 0.0) continue;
        M0 += wd * cn[d][0];
        M1 += wd * cn[d][1];
        M2 += wd * cn[d][2];
        MD += wd * cn[d][3];
        if (!cov && wd > 0.0 && cn[d][3] < Ds) {
            Ds = cn[d][3];
            dsel = d;
        }
    }
    double gM[4] = {0.0, 0.0, 0.0, 0.0}, ga = 0.0;
    if (branch == 1) {
        const double s = 1.0 / (double)q1.z;
        gM[0] = s * g0.x;
        gM[1] = s * g0.y;
        gM[2] = s * g0.z;
        gM[3] = s * g0.w;
        ga = -s * s * ((double)g0.x * M0 + (double)g0.y * M1 + (double)g0.z * M2 + (double)g0.w * MD);
    } else if (branch == 0) {
        gM[0] = g0.x;
        gM[1] = g0.y;
        gM[2] = g0.z;
        gM[3] = g0.w;
        ga = g1.x;
    }
    float4* sc = reinterpret_cast<float4*>(scratch) + 2 * (size_t)x;
    sc[0] = make_float4((float)gM[0], (float)gM[1], (float)gM[2], (float)gM[3]);
    sc[1] = make_float4(dsel >= 0 ? g1.y : 0.0f, __int_as_float(dsel), 0.0f, 0.0f);

    const double gws = cov ? gM[0] * c[0] + gM[1] * c[1] + gM[2] * c[2] + gM[3] * Dx + ga : 0.0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (code[d] < 0) continue;
        const int n = nb[d];
        const bool ncov = P.face_id[n] >= 0;
        const bool front = code[d] & 1;
        const double sg = (code[d] & 2) ? 1.0 : -1.0;
        const int fk = code[d] >> 2, face = fk / 3, k = fk - 3 * face;
        const double gwn = ncov ? gM[0] * cn[d][0] + gM[1] * cn[d][1] + gM[2] * cn[d][2] + gM[3] * cn[d][3] + ga : 0.0;
        const double gt = front ? gws - (ncov ? gwn : 0.0) : gwn - (cov ? gws : 0.0);
        if (gt == 0.0) continue;
        const int ci = k == 2 ? 0 : k + 1, cj = k == 0 ? 2 : k - 1;
        const int vi = P.faces[ci * P.F + face], vj = P.faces[cj * P.F + face];
        const double ui = (double)P.vs[vi], uj = (double)P.vs[vj];
        const double vvi = (double)P.vs[P.V + vi], vvj = (double)P.vs[P.V + vj];
        const int pa = front ? x : n, pb = front ? n : x;
        const double au = (double)(pa % W) + 0.5, av = (double)(pa / W) + 0.5;
        const double bu = (double)(pb % W) + 0.5, bv = (double)(pb / W) + 0.5;
        // the crossing, as in the forward: e(p) = sgn((u_j - u_i)(p_v - v_i) - (v_j - v_i)(p_u - u_i))
        const double ea = sg * ((uj - ui) * (av - vvi) - (vvj - vvi) * (au - ui));
        const double eb = sg * ((uj - ui) * (bv - vvi) - (vvj - vvi) * (bu - ui));
        const double den = ea - eb;
        const double dt_dea = -eb / (den * den), dt_deb = ea / (den * den);
        const double dui = dt_dea * sg * (vvj - av) + dt_deb * sg * (vvj - bv);
        const double dvi = dt_dea * sg * (au - uj) + dt_deb * sg * (bu - uj);
        const double duj = dt_dea * sg * (av - vvi) + dt_deb * sg * (bv - vvi);
        const double dvj = dt_dea * sg * (ui - au) + dt_deb * sg * (ui - bu);
        unsafeAtomicAdd(&g_vs[vi], (float)(gt * dui));
        unsafeAtomicAdd(&g_vs[P.V + vi], (float)(gt * dvi));
        unsafeAtomicAdd(&g_vs[vj], (float)(gt * duj));
        unsafeAtomicAdd(&g_vs[P.V + vj], (float)(gt * dvj));
    }
}

// Pass 2, per pixel x: the gradients of its own surface colour and depth, from its
// own layer and from every neighbour whose layer weighs x's surface (the weight a
// neighbour gives x is in the neighbour's record, in the direction of x).
__global__ void __launch_bounds__(256) k_antialias_bwd2(AaParams P, const float* __restrict__ pairs,
                                                        const float* __restrict__ g_layer,
                                                        const float* __restrict__ scratch,
                                                        float* __restrict__ g_mesh_rgb,
                                                        float* __restrict__ g_mesh_depth)
{
    const int W = P.cam.width, H = P.cam.height;
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= W * H) return;
    const int px = x % W, py = x / W;
    const bool cov = P.face_id[x] >= 0;
    float gc0 = 0.0f, gc1 = 0.0f, gc2 = 0.0f, gd = 0.0f;
    if (cov) {
        const float ws = pairs[12 * (size_t)x];
        const float4 s0 = reinterpret_cast<const float4*>(scratch)[2 * (size_t)x];
        gc0 = ws * s0.x;
        gc1 = ws * s0.y;
        gc2 = ws * s0.z;
        gd = ws * s0.w + g_layer[8 * (size_t)x + 5];  // own depth also splits the Gaussians
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const bool has = d == 0 ? px > 0 : (d == 1 ? px < W - 1 : (d == 2 ? py > 0 : py < H - 1));
            if (!has) continue;
            const int n = neighbour_index(x, d, W);
            // the neighbour's weight of x's surface: its entry in the direction of x
            const float wf = pairs[12 * (size_t)n + 1 + (d ^ 1)];
            const float4 n1 = reinterpret_cast<const float4*>(scratch)[2 * (size_t)n + 1];
            if (wf != 0.0f) {
                const float4 n0 = reinterpret_cast<const float4*>(scratch)[2 * (size_t)n];
                gc0 += wf * n0.x;
                gc1 += wf * n0.y;
                gc2 += wf * n0.z;
                gd += wf * n0.w;
            }
            // the split depth of an uncovered neighbour taken from x
            if (__float_as_int(n1.y) == (d ^ 1)) gd += n1.x;
        }
    }
    g_mesh_rgb[3 * (size_t)x] = gc0;
    g_mesh_rgb[3 * (size_t)x + 1] = gc1;
    g_mesh_rgb[3 * (size_t)x + 2] = gc2;
    g_mesh_depth[x] = gd;
}

// dL/d(world vertex) += chain of dL/d(u, v) through u = fx x_c / z_c + cx,
// v = fy y_c / z_c + cy, x_c = R X + t.
__global__ void k_vscreen_bwd(DevCamera cam, int V, const float* __restrict__ verts, const float* __restrict__ g_vs,
                              float* __restrict__ g_verts)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= V) return;
    const float gu = g_vs[i], gv = g_vs[V + i];
    if (gu == 0.0f && gv == 0.0f) return;
    const float X = verts[i], Y = verts[V + i], Z = verts[2 * V + i];
    const float* R = cam.R;
    const float xc = ((R[0] * X + R[1] * Y) + R[2] * Z) + cam.t[0];
    const float yc = ((R[3] * X + R[4] * Y) + R[5] * Z) + cam.t[1];
    const float zc = ((R[6] * X + R[7] * Y) + R[8] * Z) + cam.t[2];
    const float gx = gu * cam.fx / zc, gy = gv * cam.fy / zc;
    const float gz = -(gu * cam.fx * xc + gv * cam.fy * yc) / (zc * zc);
#pragma unroll
    for (int j = 0; j < 3; ++j) g_verts[j * V + i] += (R[j] * gx + R[3 + j] * gy) + R[6 + j] * gz;
}

__global__ void k_zero_vs(float* __restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

static gm_status aa_params(AaParams& P, const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                           const int32_t* adj, const int32_t* face_id, const float* depth, const float* colour,
                           bool need_adj)
{
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(mesh != nullptr, "mesh is NULL");
    GM_ARG_CHECK(mesh->F == 0 || (mesh->faces && vscreen && (adj || !need_adj)),
                 "mesh faces / vscreen / adjacency is NULL");
    GM_ARG_CHECK(face_id && depth && colour, "face_id / depth / colour is NULL");
    P = AaParams{};
    P.cam = dev_camera(*cam);
    P.V = mesh->V;
    P.F = mesh->F;
    P.vs = vscreen;
    P.faces = mesh->faces;
    P.mask = mesh->face_mask;
    P.adj = adj;
    P.face_id = face_id;
    P.depth = depth;
    P.colour = colour;
    return GM_OK;
}

}  // namespace gm

using namespace gm;

extern "C" {

size_t gm_edge_adjacency_ws(int32_t F)
{
    const size_t cap = adj_capacity(F);
    return align_up(cap * 8, 256) + align_up(cap * 4, 256) + align_up(cap * 8, 256);
}

gm_status gm_edge_adjacency(const gm_mesh* mesh, int32_t* adj, void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    GM_ARG_CHECK(mesh != nullptr && mesh->F >= 0, "mesh is NULL or F is negative");
    if (mesh->F == 0) return GM_OK;
    GM_ARG_CHECK(mesh->faces && adj && ws, "faces / adj / workspace is NULL");
    GM_ARG_CHECK(ws_bytes >= gm_edge_adjacency_ws(mesh->F), "workspace of %zu bytes is smaller than %zu", ws_bytes,
                 gm_edge_adjacency_ws(mesh->F));
    const size_t cap = adj_capacity(mesh->F);
    AdjTable t = adj_table(ws, cap);
    k_adj_init<<<(unsigned)div_up((int64_t)cap, 256), 256, 0, stream>>>(t, (int64_t)cap);
    GM_LAUNCH_CHECK();
    const int n = 3 * mesh->F;
    k_adj_insert<<<(unsigned)div_up(n, 256), 256, 0, stream>>>(t, mesh->faces, mesh->F);
    GM_LAUNCH_CHECK();
    k_adj_lookup<<<(unsigned)div_up(n, 256), 256, 0, stream>>>(t, mesh->faces, mesh->F, adj);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

gm_status gm_antialias(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen, const int32_t* adj,
                       const gm_light* light, const int32_t* face_id, const float* depth, float* colour, float* layer,
                       float* pairs, float* tile_dmax, hipStream_t stream)
{
    clear_error();
    AaParams P;
    if (gm_status s = aa_params(P, cam, mesh, vscreen, adj, face_id, depth, colour, true)) return s;
    GM_ARG_CHECK(layer != nullptr && ((uintptr_t)layer & 15) == 0, "layer is NULL or not 16-byte aligned");
    GM_ARG_CHECK(((uintptr_t)pairs & 15) == 0, "pairs must be 16-byte aligned");
    const int64_t HW = (int64_t)P.cam.width * P.cam.height;
    if (gm_status s = launch_surface_colour(cam, mesh, vscreen, light, face_id, nullptr, colour, stream)) return s;
    k_antialias<<<(unsigned)div_up(HW, 256), 256, 0, stream>>>(P, layer, tile_dmax, pairs);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

size_t gm_antialias_bwd_ws(int32_t width, int32_t height)
{
    return (size_t)(width > 0 ? width : 0) * (size_t)(height > 0 ? height : 0) * 8 * sizeof(float);
}

gm_status gm_antialias_bwd(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen, const float* pairs,
                           const int32_t* face_id, const float* depth, const float* colour, const float* g_layer,
                           float* g_mesh_rgb, float* g_mesh_depth, float* g_vscreen, void* ws, size_t ws_bytes,
                           hipStream_t stream)
{
    clear_error();
    AaParams P;
    GM_ARG_CHECK(pairs != nullptr, "pairs (the forward's record) is NULL");
    // the walk over internal edges is not repeated: no adjacency
    if (gm_status s = aa_params(P, cam, mesh, vscreen, nullptr, face_id, depth, colour, false)) return s;
    GM_ARG_CHECK(g_layer && g_mesh_rgb && g_mesh_depth && ws, "g_layer / outputs / workspace is NULL");
    GM_ARG_CHECK(((uintptr_t)g_layer & 15) == 0 && ((uintptr_t)ws & 15) == 0 && ((uintptr_t)pairs & 15) == 0,
                 "g_layer, pairs and the workspace must be 16-byte aligned");
    GM_ARG_CHECK(ws_bytes >= gm_antialias_bwd_ws(cam->width, cam->height), "workspace of %zu bytes is too small",
                 ws_bytes);
    GM_ARG_CHECK(mesh->V == 0 || g_vscreen, "g_vscreen is NULL");
    const int64_t HW = (int64_t)P.cam.width * P.cam.height;
    if (mesh->V > 0) {
        k_zero_vs<<<(unsigned)div_up(2 * (int64_t)mesh->V, 256), 256, 0, stream>>>(g_vscreen, 2 * (int64_t)mesh->V);
        GM_LAUNCH_CHECK();
    }
    k_antialias_bwd1<<<(unsigned)div_up(HW, 256), 256, 0, stream>>>(P, pairs, g_layer, (float*)ws, g_vscreen);
    GM_LAUNCH_CHECK();
    k_antialias_bwd2<<<(unsigned)div_up(HW, 256), 256, 0, stream>>>(P, pairs, g_layer, (const float*)ws, g_mesh_rgb,
                                                                    g_mesh_depth);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

gm_status gm_vscreen_bwd(const gm_camera* cam, const gm_mesh* mesh, const float* g_vscreen, float* g_verts,
                         hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(mesh != nullptr && mesh->V >= 0, "mesh is NULL or V is negative");
    if (mesh->V == 0) return GM_OK;
    GM_ARG_CHECK(mesh->verts && g_vscreen && g_verts, "verts / g_vscreen / g_verts is NULL");
    k_vscreen_bwd<<<(unsigned)div_up(mesh->V, 256), 256, 0, stream>>>(dev_camera(*cam), mesh->V, mesh->verts,
                                                                     g_vscreen, g_verts);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

}  // extern "C"
