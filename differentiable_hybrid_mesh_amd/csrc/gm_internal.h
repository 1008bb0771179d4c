// Internal helpers of libgm (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "gm.h"

namespace gm {

// ---------------------------------------------------------------------------
// host-side error state
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define GM_ARG_CHECK(cond, ...)                \
    do {                                       \
        if (!(cond)) {                         \
            ::gm::set_error(__VA_ARGS__);      \
            return GM_ERR_ARG;                 \
        }                                      \
    } while (0)

#define GM_HIP_CHECK(expr)                                                               \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess) {                                                          \
            ::gm::set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),       \
                            __FILE__, __LINE__);                                         \
            return GM_ERR_HIP;                                                           \
        }                                                                                \
    } while (0)

#define GM_LAUNCH_CHECK() GM_HIP_CHECK(hipGetLastError())

inline int tiles_x(const gm_camera& c) { return (c.width + GM_TILE - 1) / GM_TILE; }
inline int tiles_y(const gm_camera& c) { return (c.height + GM_TILE - 1) / GM_TILE; }
inline int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Camera as a kernel argument (by value).
struct DevCamera {
    int width, height, tx, ty;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    float near_z;
};

inline DevCamera dev_camera(const gm_camera& c)
{
    DevCamera d;
    d.width = c.width;
    d.height = c.height;
    d.tx = tiles_x(c);
    d.ty = tiles_y(c);
    d.fx = c.fx;
    d.fy = c.fy;
    d.cx = c.cx;
    d.cy = c.cy;
    for (int i = 0; i < 9; ++i) d.R[i] = c.R[i];
    for (int i = 0; i < 3; ++i) d.t[i] = c.t[i];
    d.near_z = c.near_z;
    return d;
}

gm_status check_camera(const gm_camera* cam);

// ---------------------------------------------------------------------------
// device-wide exclusive scan of int32 counts (gm_api.hip)
// ---------------------------------------------------------------------------
// out[i] = sum_{j<i} in[i] for i in [0, n]; out has n + 1 entries; *total (device,
// int64) receives the full sum.  Workspace: scan_ws_bytes(n).
size_t scan_ws_bytes(int64_t n);
gm_status exclusive_scan(const int32_t* in, int32_t* out, int64_t n, long long* total, void* ws,
                         hipStream_t stream);

// The same scan in one launch for callers whose previous kernel on the stream
// cleared the first scan_lb_clear_words(n) 64-bit words of ws (the blocks find their
// offsets by a decoupled look-back over those words; a single block does it all for
// short inputs).  Workspace: scan_ws_bytes(n).  skip (device, may be NULL): when it
// points to a non-zero word the multi-block launch does nothing (the single-block
// path ignores it).
int64_t scan_lb_clear_words(int64_t n);
gm_status exclusive_scan_lb(const int32_t* in, int32_t* out, int64_t n, long long* total, void* ws,
                            hipStream_t stream, const int32_t* skip = nullptr);

// Projection (gm_project.hip): the argument checks of gm_project_gaussians, and its
// kernel with the depth sort's input written beside the records (keys[i] = the bits
// of z_c when Gaussian i is listed, all ones otherwise; ids[i] = i; *d_n = N).
gm_status check_project_args(const gm_camera* cam, int32_t N, const float* means, const float* quats,
                             const float* scales, const float* opacity, const float* sh, int32_t sh_degree,
                             const float* rec);
gm_status launch_project_keys(const DevCamera& dc, int32_t N, const float* means, const float* quats,
                              const float* scales, const float* opacity, const float* sh, int32_t sh_degree,
                              float* rec, uint32_t* keys, int32_t* ids, long long* d_n, hipStream_t stream);

// Surface colour prepass of the composite (gm_composite.hip): colour [H][W][3] =
// the shaded mesh colour at covered pixels, bg (or 0 when bg is NULL) elsewhere.
gm_status launch_surface_colour(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                                const gm_light* light, const int32_t* face_id, const float* bg, float* colour,
                                hipStream_t stream);

// ---------------------------------------------------------------------------
// tile order: largest per-tile key first (one block of TO_THREADS)
// ---------------------------------------------------------------------------
// Blocks of a grid start in launch order, and per-tile work differs by an order of
// magnitude across an image, so a grid taken in raster order leaves its longest
// tiles for the end.  A counting sort of the T tiles into TO_BUCKETS buckets of
// key(t) >= 0, largest first, gives a launch order (the order inside a bucket is
// unspecified).  Counts and slots are taken per wave: thousands of empty tiles share
// one bucket, and one counter for the block serialised their LDS atomics.  Up to
// TO_PER keys per thread stay in registers (one evaluation of key); larger images
// evaluate it again in each loop.
constexpr int TO_BUCKETS = 64;
constexpr int TO_THREADS = 1024;
constexpr int TO_PER = 16;  // keys held in registers per thread (16384 tiles)

template <class Key>
__device__ inline void order_tiles_desc(int T, Key key, int32_t* __restrict__ order)
{
    constexpr int NW = TO_THREADS / 64;
    __shared__ int s_cnt[NW][TO_BUCKETS];  // per-wave counts, then per-wave next slots
    __shared__ int s_max;
    const int wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < NW * TO_BUCKETS; i += TO_THREADS) (&s_cnt[0][0])[i] = 0;
    if (threadIdx.x == 0) s_max = 0;
    __syncthreads();
    const bool held = T <= TO_THREADS * TO_PER;
    int kv[TO_PER];
    int m = 0;
#pragma unroll
    for (int k = 0; k < TO_PER; ++k) {
        const int t = threadIdx.x + k * TO_THREADS;
        kv[k] = held && t < T ? key(t) : 0;
        m = max(m, kv[k]);
    }
    if (!held)
        for (int t = threadIdx.x; t < T; t += TO_THREADS) m = max(m, key(t));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(&s_max, m);
    __syncthreads();
    const float scale = (float)TO_BUCKETS / ((float)s_max + 1.0f);
    auto bucket_of = [&](int v) { return TO_BUCKETS - 1 - min(TO_BUCKETS - 1, (int)((float)v * scale)); };
    if (held) {
#pragma unroll
        for (int k = 0; k < TO_PER; ++k)
            if (threadIdx.x + k * TO_THREADS < T) atomicAdd(&s_cnt[wave][bucket_of(kv[k])], 1);
    } else {
        for (int t = threadIdx.x; t < T; t += TO_THREADS) atomicAdd(&s_cnt[wave][bucket_of(key(t))], 1);
    }
    __syncthreads();
    if (threadIdx.x < TO_BUCKETS) {  // bucket-major exclusive offsets, waves in order
        const int b = threadIdx.x;
        int c[NW], tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            c[w] = s_cnt[w][b];
            tot += c[w];
        }
        int x = tot;  // inclusive scan of the bucket totals over the 64 lanes of wave 0
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if ((int)threadIdx.x >= d) x += y;
        }
        int run = x - tot;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            s_cnt[w][b] = run;
            run += c[w];
        }
    }
    __syncthreads();
    if (held) {
#pragma unroll
        for (int k = 0; k < TO_PER; ++k) {
            const int t = threadIdx.x + k * TO_THREADS;
            if (t < T) order[atomicAdd(&s_cnt[wave][bucket_of(kv[k])], 1)] = t;
        }
    } else {
        for (int t = threadIdx.x; t < T; t += TO_THREADS) order[atomicAdd(&s_cnt[wave][bucket_of(key(t))], 1)] = t;
    }
}

// ---------------------------------------------------------------------------
// wave reductions
// ---------------------------------------------------------------------------
// Sum 16 per-lane values over the 64 lanes of a wave with a halving ("transpose")
// reduction: at each butterfly step a lane keeps half of its values and receives its
// partner's copy of them, so 16 values need 8+4+2+1 exchanges plus two full steps
// instead of 16*6.  The exchanges use gfx950's cross-half lane swaps (lanes 32-63
// with 0-31, odd 16-lane rows with even ones) and DPP row/quad moves, all VALU.
// On return lane l holds the wave total of value (l >> 2) when (l & 3) == 0.
//
// dpp<CTRL>: a lane-permuting move for the controls used here (row rotate, half-row
// mirror, quad permutations), which read a valid lane everywhere, so bound_ctrl (zero
// for an invalid source lane) changes no value; with it set and all rows enabled the
// compiler folds the move into the add that consumes it (one v_add_f32_dpp instead
// of a move, a hazard wait and an add).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_sum16(const float* v, int lane)
{
    float a[8], b[4], c[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // lanes 0-31 keep v[i], lanes 32-63 keep v[8+i]
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[8 + i]), false,
                                                        false);
        a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // even 16-lane rows keep a[i], odd rows a[4+i]
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[4 + i]), false,
                                                        false);
        b[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool h3 = lane & 8, h2 = lane & 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // partner: lane ^ 8 (rotate a 16-lane row by 8)
        const float send = h3 ? b[i] : b[2 + i];
        const float keep = h3 ? b[2 + i] : b[i];
        c[i] = keep + dpp<0x128>(send);
    }
    // partner: the mirrored lane in the 8-lane half row (bit 2 flipped); the two
    // quad steps below sum the four lanes of each half, so the pairing is exact
    const float send = h2 ? c[0] : c[1];
    float d = (h2 ? c[1] : c[0]) + dpp<0x141>(send);
    d += dpp<0x4E>(d);  // quad_perm [2,3,0,1]
    d += dpp<0xB1>(d);  // quad_perm [1,0,3,2]
    return d;
}

}  // namespace gm
