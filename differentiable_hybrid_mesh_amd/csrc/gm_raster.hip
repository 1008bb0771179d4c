// Mesh visibility: vertex projection, 16x16 tile binning and the per-pixel
// nearest-triangle z-buffer (gmesh README, "Design Details > Mesh rasterizer",
// step 1, and the near-plane rule).
//
// Decisions here must be reproducible bit for bit: vertex projection runs in fp32
// in the written order with no contraction, edge functions and depth in fp64.
#pragma clang fp contract(off)

#include <algorithm>

#include "gm_internal.h"

namespace gm {

constexpr int ZB_THREADS = 256;  // one thread per pixel of a 16x16 tile
constexpr int ZB_BATCH = 128;    // triangles staged in LDS per round
constexpr double ZB_MARGIN = 1.0 / 64.0;  // candidate box margin d around the bounding box, pixels

// vscreen = (u, v, z_c) planes: x_c = ((R0 x + R1 y) + R2 z) + t0, u = (fx x_c)/z_c + cx.
// Also clears nz ints at zero (the per-tile counters of the binning that follows:
// one launch fewer).
__global__ void k_project_vertices(DevCamera cam, int V, const float* __restrict__ verts,
                                   float* __restrict__ vscreen, int32_t* __restrict__ zero, int64_t nz)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nz) zero[i] = 0;
    if (i >= V) return;
    const float x = verts[i], y = verts[V + i], z = verts[2 * V + i];
    const float xc = ((cam.R[0] * x + cam.R[1] * y) + cam.R[2] * z) + cam.t[0];
    const float yc = ((cam.R[3] * x + cam.R[4] * y) + cam.R[5] * z) + cam.t[1];
    const float zc = ((cam.R[6] * x + cam.R[7] * y) + cam.R[8] * z) + cam.t[2];
    vscreen[i] = (cam.fx * xc) / zc + cam.cx;
    vscreen[V + i] = (cam.fy * yc) / zc + cam.cy;
    vscreen[2 * V + i] = zc;
}

// Tile rectangle (inclusive) of a face's pixel-centre bounding box, or false.
__device__ inline bool face_tile_rect(const DevCamera& cam, int V, int F, int f,
                                      const int32_t* __restrict__ faces,
                                      const uint8_t* __restrict__ mask,
                                      const float* __restrict__ vs, int* r)
{
    if (mask && !mask[f]) return false;
    double u[3], v[3];
    for (int k = 0; k < 3; ++k) {
        const int vi = faces[k * F + f];
        u[k] = (double)vs[vi];
        v[k] = (double)vs[V + vi];
        if (!(vs[2 * V + vi] >= cam.near_z)) return false;  // near plane: skip
    }
    const double A = (u[1] - u[0]) * (v[2] - v[0]) - (v[1] - v[0]) * (u[2] - u[0]);
    if (!(A != 0.0)) return false;
    const double umin = fmin(fmin(u[0], u[1]), u[2]), umax = fmax(fmax(u[0], u[1]), u[2]);
    const double vmin = fmin(fmin(v[0], v[1]), v[2]), vmax = fmax(fmax(v[0], v[1]), v[2]);
    const double a = fmax(ceil(umin - 0.5), 0.0), b = fmin(floor(umax - 0.5), (double)(cam.width - 1));
    const double c = fmax(ceil(vmin - 0.5), 0.0), d = fmin(floor(vmax - 0.5), (double)(cam.height - 1));
    if (!(a <= b) || !(c <= d)) return false;
    r[0] = (int)a / GM_TILE;
    r[1] = (int)c / GM_TILE;
    r[2] = (int)b / GM_TILE;
    r[3] = (int)d / GM_TILE;
    return true;
}

// Faces of one wave are neighbours in the mesh and share tiles, so the wave walks
// the tiles of its faces' rects in lockstep (the k-th tile of every face at step k)
// and at each step groups lanes by tile with ballots: one atomic per distinct tile.
__device__ __forceinline__ void next_tile(int& cx, int& cy, int x0, int x1)
{
    if (++cx > x1) {
        cx = x0;
        ++cy;
    }
}

__global__ void k_bin_count(DevCamera cam, int V, int F, const int32_t* __restrict__ faces,
                            const uint8_t* __restrict__ mask, const float* __restrict__ vs,
                            int2* __restrict__ face_rect, int32_t* __restrict__ tile_cnt)
{
    const int f = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    int r[4] = {0, 0, 0, 0};
    const bool ok = f < F && face_tile_rect(cam, V, F, f, faces, mask, vs, r);
    if (f < F) face_rect[f] = ok ? make_int2(r[0] | (r[1] << 16), r[2] | (r[3] << 16)) : make_int2(1, 0);
    const int nt = ok ? (r[2] - r[0] + 1) * (r[3] - r[1] + 1) : 0;
    int cx = r[0], cy = r[1];
    for (int k = 0; __ballot(k < nt); ++k) {
        const int tk = k < nt ? cy * cam.tx + cx : -1;
        unsigned long long pend = __ballot(tk >= 0);
        while (pend) {
            const int leader = __builtin_ctzll(pend);
            const int tl = __builtin_amdgcn_readlane(tk, leader);
            const unsigned long long grp = __ballot(tk == tl);
            if (lane == leader) atomicAdd(&tile_cnt[tl], __popcll(grp));
            pend &= ~grp;
        }
        next_tile(cx, cy, r[0], r[2]);
    }
}

// Threads [0, F) scatter face ids, grouped as in the count.  When the pair total
// exceeds cap nothing is scattered and threads [0, T] instead clear tile_offsets,
// so the bins read as empty downstream (the caller enlarges tile_tris and bins
// again).
__global__ void k_bin_scatter(DevCamera cam, int F, int T, const int2* __restrict__ face_rect,
                              int32_t* __restrict__ tile_off, const long long* __restrict__ total,
                              int64_t cap, int32_t* __restrict__ cursor, int32_t* __restrict__ tile_tris)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (*total > cap) {  // uniform
        if (i <= T) tile_off[i] = 0;
        return;
    }
    const int lane = threadIdx.x & 63;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int2 pr = i < F ? face_rect[i] : make_int2(1, 0);
    const bool ok = !(pr.x == 1 && pr.y == 0);
    const int x0 = pr.x & 0xffff, y0 = pr.x >> 16, x1 = pr.y & 0xffff, y1 = pr.y >> 16;
    const int nt = ok ? (x1 - x0 + 1) * (y1 - y0 + 1) : 0;
    int cx = x0, cy = y0;
    for (int k = 0; __ballot(k < nt); ++k) {
        const int tk = k < nt ? cy * cam.tx + cx : -1;
        // group membership first, then every group's leader reserves its slots with
        // one atomic, all groups in the same instruction
        int leader = lane, rank = 0, cnt = 0;
        unsigned long long pend = __ballot(tk >= 0);
        while (pend) {
            const int l = __builtin_ctzll(pend);
            const int tl = __builtin_amdgcn_readlane(tk, l);
            const unsigned long long grp = __ballot(tk == tl);
            if (tk == tl) {
                leader = l;
                rank = __popcll(grp & lt);
            }
            if (lane == l) cnt = __popcll(grp);
            pend &= ~grp;
        }
        int base = 0;
        if (cnt > 0) base = atomicAdd(&cursor[tk], cnt);
        base = __shfl(base, leader, 64);
        if (tk >= 0) tile_tris[tile_off[tk] + base + rank] = i;
        next_tile(cx, cy, x0, x1);
    }
}

// Triangle setup as staged in LDS, one plane per field (structure of arrays), so
// that lanes reading the setups of different triangles hit consecutive banks:
// screen vertices u, v; camera depths z; twice the signed area A.  The edge
// deltas b - a of edges (v1,v2), (v2,v0), (v0,v1) are formed where they are used.
enum TriField { TU = 0, TV = 3, TZ = 6, TA = 9, TFIELDS = 10 };

// E_k = (b.u - a.u)(p.v - a.v) - (b.v - a.v)(p.u - a.u) for the edges above.
__device__ __forceinline__ void edge_functions(const double (*s_t)[ZB_BATCH], int j, double pu, double pv,
                                               double& E0, double& E1, double& E2)
{
    const double u0 = s_t[TU][j], u1 = s_t[TU + 1][j], u2 = s_t[TU + 2][j];
    const double v0 = s_t[TV][j], v1 = s_t[TV + 1][j], v2 = s_t[TV + 2][j];
    E0 = (u2 - u1) * (pv - v1) - (v2 - v1) * (pu - u1);
    E1 = (u0 - u2) * (pv - v2) - (v0 - v2) * (pu - u2);
    E2 = (u1 - u0) * (pv - v0) - (v1 - v0) * (pu - u0);
}

constexpr int ZB_CHUNK = 1024;  // candidates per round (bounds the covered list)
constexpr int ZB_PER_THREAD = ZB_CHUNK / ZB_THREADS;
constexpr unsigned long long ZB_INF = 0x7FF0000000000000ull;  // +inf as fp64 bits

// One block per tile.  Each staged triangle contributes as candidates the tile's
// pixel centres within ZB_MARGIN of its bounding box (the whole tile for a triangle
// too thin for that margin to be exact; see the staging code); the
// candidates of a batch form one flat sequence, walked in rounds of ZB_CHUNK with
// four consecutive candidates per thread, so lanes stay busy whatever the triangle
// size.  A round runs in three phases: the fp64 edge test appends covered
// candidates to a compact list; the perspective-correct depth of every listed
// candidate lowers its pixel's nearest depth with an LDS min on the fp64 bit
// pattern (positive doubles order like their bits); then every pixel takes the
// smallest face id among the candidates at exactly its nearest depth.  Decision
// rule and arithmetic are those of the per-pixel definition, bit for bit.
// Order in which the z-buffer takes the tiles: largest bin first.  A tile's work
// grows with its triangles (candidates, covered ones, depth rounds), which differ by
// an order of magnitude between the sphere's limb and its interior, and a grid taken
// in raster order left the longest tiles for its end (0.215 -> 0.155 ms at C3).
__global__ void __launch_bounds__(TO_THREADS) k_zbuffer_order(int T, const int32_t* __restrict__ tile_off,
                                                              int32_t* __restrict__ order)
{
    order_tiles_desc(T, [=](int t) { return tile_off[t + 1] - tile_off[t]; }, order);
}

__global__ void __launch_bounds__(ZB_THREADS)
k_zbuffer(DevCamera cam, int V, int F, const int32_t* __restrict__ faces,
          const float* __restrict__ vs, const int32_t* __restrict__ tile_off,
          const int32_t* __restrict__ tile_tris, int32_t* __restrict__ face_id,
          float* __restrict__ depth, float* __restrict__ tile_dmax, const int32_t* __restrict__ order)
{
    __shared__ double s_t[TFIELDS][ZB_BATCH];
    __shared__ int s_f[ZB_BATCH];
    __shared__ int4 s_box[ZB_BATCH];       // clipped box in tile-local pixels: x0, w, y0, bits of 1/w
    __shared__ int s_coff[ZB_BATCH + 1];   // candidate prefix sums
    __shared__ unsigned long long s_minz[ZB_THREADS];
    __shared__ int s_id[ZB_THREADS];
    __shared__ unsigned long long s_cz[ZB_CHUNK];
    __shared__ int s_cov[ZB_CHUNK];        // covered candidates: local pixel | staged index << 8
    __shared__ int s_ncov[2];              // list lengths, alternating between rounds
    __shared__ int s_wsum[ZB_THREADS / 64];
    __shared__ float s_red[ZB_THREADS / 64];

    const int tile = order[blockIdx.x];  // largest bins first
    const int tx = tile % cam.tx, ty = tile / cam.tx;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int px = tx * GM_TILE + (threadIdx.x & 15), py = ty * GM_TILE + (threadIdx.x >> 4);
    const bool inside = px < cam.width && py < cam.height;
    const int xlim = min(GM_TILE, cam.width - tx * GM_TILE), ylim = min(GM_TILE, cam.height - ty * GM_TILE);
    const int start = tile_off[tile], end = tile_off[tile + 1];
    const double ox = tx * GM_TILE, oy = ty * GM_TILE;

    s_minz[threadIdx.x] = ZB_INF;
    s_id[threadIdx.x] = 0x7fffffff;
    if (threadIdx.x == 0) s_ncov[0] = 0;
    int round = 0;
    for (int b0 = start; b0 < end; b0 += ZB_BATCH) {
        const int nb = min(ZB_BATCH, end - b0);
        __syncthreads();
        int cnt = 0;
        if (threadIdx.x < nb) {
            const int j = threadIdx.x;
            const int f = tile_tris[b0 + j];
            struct {
                double u[3], v[3], z[3];
            } t;
            for (int k = 0; k < 3; ++k) {
                const int vi = faces[k * F + f];
                t.u[k] = (double)vs[vi];
                t.v[k] = (double)vs[V + vi];
                t.z[k] = (double)vs[2 * V + vi];
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                s_t[TU + k][j] = t.u[k];
                s_t[TV + k][j] = t.v[k];
                s_t[TZ + k][j] = t.z[k];
            }
            const double A = (t.u[1] - t.u[0]) * (t.v[2] - t.v[0]) - (t.v[1] - t.v[0]) * (t.u[2] - t.u[0]);
            s_t[TA][j] = A;
            s_f[j] = f;
            // Candidates: the tile's pixel centres within ZB_MARGIN of the triangle's
            // bounding box, which hold every centre the fp64 edge test accepts when the
            // triangle is not too thin.  A centre p at distance >= d from the triangle
            // has an edge k with E_k(p) beyond |e_k| d sin(theta_min / 2) on the outer
            // side (the nearest point of the triangle is on edge k, or at a vertex whose
            // normal cone holds p), while the rounding of E_k (two differences, two
            // products, one subtraction) is below 8 eps |e_k| R, R bounding |p - vertex|
            // in the L1 norm over the tile.  With sin(theta_min / 2) >= |A| / (2 L^2)
            // (A twice the signed area, L the longest edge) the sign is exact once
            // |A| > 16 eps R L^2 / d = 2^-43 R L^2 at d = 1/64 px; the test uses 2^-40.
            // Thinner triangles test every pixel of the tile, as the definition does.
            const double umin = fmin(fmin(t.u[0], t.u[1]), t.u[2]), umax = fmax(fmax(t.u[0], t.u[1]), t.u[2]);
            const double vmin = fmin(fmin(t.v[0], t.v[1]), t.v[2]), vmax = fmax(fmax(t.v[0], t.v[1]), t.v[2]);
            double L2 = 0.0, R = 0.0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int k1 = k == 2 ? 0 : k + 1;
                const double du = t.u[k1] - t.u[k], dv = t.v[k1] - t.v[k];
                L2 = fmax(L2, du * du + dv * dv);
                R = fmax(R, fabs(t.u[k] - (ox + 8.0)) + fabs(t.v[k] - (oy + 8.0)));
            }
            R += 16.0;
            int x0 = 0, x1 = xlim - 1, y0 = 0, y1 = ylim - 1;
            if (fabs(A) > 0x1p-40 * R * L2) {
                // pixel-centre range [ceil(min - 1/2 - d), floor(max - 1/2 + d)]
                x0 = (int)fmax(ceil(umin - 0.5 - ZB_MARGIN) - ox, 0.0);
                x1 = (int)fmin(floor(umax - 0.5 + ZB_MARGIN) - ox, xlim - 1.0);
                y0 = (int)fmax(ceil(vmin - 0.5 - ZB_MARGIN) - oy, 0.0);
                y1 = (int)fmin(floor(vmax - 0.5 + ZB_MARGIN) - oy, ylim - 1.0);
            }
            const int w = max(x1 - x0 + 1, 1);
            if (x0 <= x1 && y0 <= y1) cnt = w * (y1 - y0 + 1);
            s_box[j] = make_int4(x0, w, y0, __float_as_int(1.0f / (float)w));
        }
        // exclusive scan of the candidate counts (threads >= nb contribute 0)
        int x = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) s_wsum[wave] = x;
        __syncthreads();
        int wo = 0;
        for (int w = 0; w < wave; ++w) wo += s_wsum[w];
        if (threadIdx.x < ZB_BATCH) s_coff[threadIdx.x] = wo + x - cnt;
        const int total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
        if (threadIdx.x == 0) s_coff[ZB_BATCH] = total;
        __syncthreads();
        for (int c0 = 0; c0 < total; c0 += ZB_CHUNK, ++round) {
            const int par = round & 1;
            const unsigned long long prev = s_minz[threadIdx.x];
            const int cend = min(c0 + ZB_CHUNK, total);
            // phase 1: edge test of four consecutive candidates per thread
            const int cf = c0 + ZB_PER_THREAD * threadIdx.x;
            int j = 0;
            if (cf < cend) {  // last staged triangle whose candidates start at or before cf
                int lo = 0, hi = nb - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_coff[mid] <= cf) lo = mid;
                    else hi = mid - 1;
                }
                j = lo;
            }
#pragma unroll
            for (int k = 0; k < ZB_PER_THREAD; ++k) {
                const int c = cf + k;
                bool cov = false;
                int p = 0;
                if (c < cend) {
                    while (s_coff[j + 1] <= c) ++j;
                    const int4 bx = s_box[j];
                    const int loc = c - s_coff[j];
                    const int qy = (int)(((float)loc + 0.5f) * __int_as_float(bx.w));
                    const int ly = bx.z + qy, lx = bx.x + (loc - qy * bx.y);
                    const double pu = ox + lx + 0.5, pv = oy + ly + 0.5;
                    double E0, E1, E2;
                    edge_functions(s_t, j, pu, pv, E0, E1, E2);
                    cov = s_t[TA][j] > 0 ? (E0 >= 0 && E1 >= 0 && E2 >= 0) : (E0 <= 0 && E1 <= 0 && E2 <= 0);
                    p = ly * GM_TILE + lx;
                }
                const unsigned long long m = __ballot(cov);
                if (m) {
                    const int leader = __ffsll((long long)m) - 1;
                    int slot = 0;
                    if (lane == leader) slot = atomicAdd(&s_ncov[par], __popcll(m));
                    slot = __builtin_amdgcn_readlane(slot, leader);
                    if (cov) s_cov[slot + __popcll(m & lt)] = p | (j << 8);
                }
            }
            __syncthreads();
            // phase 2: depth of the covered candidates, nearest depth per pixel
            const int ncov = s_ncov[par];
            if (threadIdx.x == 0) s_ncov[par ^ 1] = 0;
            for (int q = threadIdx.x; q < ncov; q += ZB_THREADS) {
                const int e = s_cov[q];
                const int p = e & 0xff, jj = e >> 8;
                const double pu = ox + (p & 15) + 0.5, pv = oy + (p >> 4) + 0.5;
                double E0, E1, E2;
                edge_functions(s_t, jj, pu, pv, E0, E1, E2);
                const double A = s_t[TA][jj];
                const double l0 = E0 / A, l1 = E1 / A, l2 = E2 / A;
                const double inv = (l0 / s_t[TZ + 0][jj] + l1 / s_t[TZ + 1][jj]) + l2 / s_t[TZ + 2][jj];
                const double z = 1.0 / inv;
                const unsigned long long zb = (unsigned long long)__double_as_longlong(z);
                atomicMin(&s_minz[p], zb);
                s_cz[q] = zb;
            }
            __syncthreads();
            if (s_minz[threadIdx.x] < prev) s_id[threadIdx.x] = 0x7fffffff;  // a nearer surface: forget older ties
            __syncthreads();
            // phase 3: smallest face id at exactly the nearest depth
            for (int q = threadIdx.x; q < ncov; q += ZB_THREADS) {
                const int e = s_cov[q];
                const int p = e & 0xff;
                if (s_cz[q] == s_minz[p]) atomicMin(&s_id[p], s_f[e >> 8]);
            }
            __syncthreads();
        }
    }
    __syncthreads();
    const unsigned long long mz = s_minz[threadIdx.x];
    const int bid = mz == ZB_INF ? -1 : s_id[threadIdx.x];
    const float d = bid >= 0 ? (float)__longlong_as_double((long long)mz) : INFINITY;
    if (inside) {
        face_id[py * cam.width + px] = bid;
        depth[py * cam.width + px] = d;
    }
    // tile_dmax: max depth over in-image pixels, +inf when any of them is empty
    float mx = inside ? d : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = s_red[0];
        for (int w = 1; w < ZB_THREADS / 64; ++w) r = fmaxf(r, s_red[w]);
        tile_dmax[tile] = r;  // an empty pixel has depth +inf, so the max is +inf
    }
}

}  // namespace gm

using namespace gm;

extern "C" {

size_t gm_bin_triangles_ws(int32_t V, int32_t F, int32_t width, int32_t height)
{
    (void)V;
    const int64_t T = div_up(width, GM_TILE) * div_up(height, GM_TILE);
    size_t b = 0;
    b += align_up(sizeof(int2) * (size_t)(F > 0 ? F : 1), 256);   // face rects
    b += align_up(sizeof(int32_t) * (size_t)T, 256);               // tile counts
    b += align_up(sizeof(int32_t) * (size_t)T, 256);               // cursors
    b += scan_ws_bytes(T);
    return b;
}

gm_status gm_bin_triangles(const gm_camera* cam, const gm_mesh* mesh, float* vscreen,
                           int32_t* tile_offsets, int32_t* tile_tris, int64_t cap, int64_t* n_pairs,
                           void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(mesh != nullptr, "mesh is NULL");
    GM_ARG_CHECK(mesh->V >= 0 && mesh->F >= 0, "negative mesh size");
    GM_ARG_CHECK(mesh->V == 0 || (mesh->verts && vscreen), "verts / vscreen is NULL");
    GM_ARG_CHECK(mesh->F == 0 || mesh->faces, "faces is NULL");
    GM_ARG_CHECK(tile_offsets && n_pairs && ws, "tile_offsets / n_pairs / ws is NULL");
    GM_ARG_CHECK(cap >= 0 && (cap == 0 || tile_tris), "tile_tris is NULL or cap negative");
    const size_t need = gm_bin_triangles_ws(mesh->V, mesh->F, cam->width, cam->height);
    GM_ARG_CHECK(ws_bytes >= need, "workspace %zu bytes, %zu needed", ws_bytes, need);

    const DevCamera dc = dev_camera(*cam);
    const int64_t T = (int64_t)dc.tx * dc.ty;
    const int V = mesh->V, F = mesh->F;
    char* w = (char*)ws;
    int2* face_rect = (int2*)w;
    w += align_up(sizeof(int2) * (size_t)(F > 0 ? F : 1), 256);
    int32_t* tile_cnt = (int32_t*)w;
    w += align_up(sizeof(int32_t) * (size_t)T, 256);
    int32_t* cursor = (int32_t*)w;
    w += align_up(sizeof(int32_t) * (size_t)T, 256);
    void* scan_ws = w;
    long long* total = reinterpret_cast<long long*>(n_pairs);

    const int64_t nz = (cursor - tile_cnt) + T;  // tile_cnt and cursor
    k_project_vertices<<<(unsigned)div_up(std::max<int64_t>(V, nz), 256), 256, 0, stream>>>(dc, V, mesh->verts,
                                                                                         vscreen, tile_cnt, nz);
    GM_LAUNCH_CHECK();
    if (F > 0) {
        k_bin_count<<<(unsigned)div_up(F, 256), 256, 0, stream>>>(dc, V, F, mesh->faces, mesh->face_mask,
                                                                 vscreen, face_rect, tile_cnt);
        GM_LAUNCH_CHECK();
    }
    if (gm_status s = exclusive_scan(tile_cnt, tile_offsets, T, total, scan_ws, stream)) return s;
    // the scatter compares the total with cap on the device
    const int64_t nthr = std::max<int64_t>(F, T + 1);
    k_bin_scatter<<<(unsigned)div_up(nthr, 256), 256, 0, stream>>>(dc, F, (int)T, face_rect, tile_offsets, total,
                                                                  std::min<int64_t>(cap, INT32_MAX), cursor,
                                                                  tile_tris);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

size_t gm_raster_zbuffer_ws(int32_t width, int32_t height)
{
    const int64_t T = div_up(width > 0 ? width : 1, GM_TILE) * div_up(height > 0 ? height : 1, GM_TILE);
    return align_up(sizeof(int32_t) * (size_t)T, 256);
}

gm_status gm_raster_zbuffer(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                            const int32_t* tile_offsets, const int32_t* tile_tris, int32_t* face_id,
                            float* depth, float* tile_dmax, void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(mesh != nullptr, "mesh is NULL");
    GM_ARG_CHECK(face_id && depth && tile_dmax && tile_offsets, "an output or tile_offsets is NULL");
    GM_ARG_CHECK(mesh->F == 0 || (mesh->faces && vscreen && tile_tris), "faces / vscreen / tile_tris is NULL");
    const size_t need = gm_raster_zbuffer_ws(cam->width, cam->height);
    GM_ARG_CHECK(ws != nullptr && ws_bytes >= need, "workspace %zu bytes, %zu needed", ws_bytes, need);
    const DevCamera dc = dev_camera(*cam);
    const int64_t T = (int64_t)dc.tx * dc.ty;
    int32_t* order = static_cast<int32_t*>(ws);
    k_zbuffer_order<<<1, TO_THREADS, 0, stream>>>((int)T, tile_offsets, order);
    GM_LAUNCH_CHECK();
    k_zbuffer<<<(unsigned)T, ZB_THREADS, 0, stream>>>(dc, mesh->V, mesh->F, mesh->faces, vscreen,
                                                     tile_offsets, tile_tris, face_id, depth, tile_dmax, order);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

}  // extern "C"
