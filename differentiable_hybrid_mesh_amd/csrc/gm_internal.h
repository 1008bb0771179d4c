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
// device-wide exclusive scan of int32 counts (gm_scan.hip)
// ---------------------------------------------------------------------------
// out[i] = sum_{j<i} in[i] for i in [0, n]; out has n + 1 entries; *total (device,
// int64) receives the full sum.  Workspace: scan_ws_bytes(n).
size_t scan_ws_bytes(int64_t n);
gm_status exclusive_scan(const int32_t* in, int32_t* out, int64_t n, long long* total, void* ws,
                         hipStream_t stream);

// Surface colour prepass of the composite (gm_composite.hip): colour [H][W][3] =
// the shaded mesh colour at covered pixels, bg (or 0 when bg is NULL) elsewhere.
gm_status launch_surface_colour(const gm_camera* cam, const gm_mesh* mesh, const float* vscreen,
                                const gm_light* light, const int32_t* face_id, const float* bg, float* colour,
                                hipStream_t stream);

// Read a device int64 into host memory (synchronises the stream).
gm_status read_back_i64(const long long* dev, int64_t* host, hipStream_t stream);

}  // namespace gm
