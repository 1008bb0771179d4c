// libgm: error state, device-wide scan, mip pyramid.
#include <cstdarg>
#include <cstring>

#include "gm_internal.h"

namespace gm {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

gm_status check_camera(const gm_camera* cam)
{
    GM_ARG_CHECK(cam != nullptr, "camera is NULL");
    GM_ARG_CHECK(cam->width > 0 && cam->height > 0, "image size %dx%d must be positive", cam->width,
                 cam->height);
    GM_ARG_CHECK(cam->width <= 16384 && cam->height <= 16384, "image size %dx%d above 16384",
                 cam->width, cam->height);
    GM_ARG_CHECK(cam->near_z > 0.0f, "near_z must be positive");
    GM_ARG_CHECK(cam->fx != 0.0f && cam->fy != 0.0f, "focal lengths must be non-zero");
    return GM_OK;
}

// ---------------------------------------------------------------------------
// exclusive scan: 256 threads x 16 items per block
// ---------------------------------------------------------------------------
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 16;
constexpr int SCAN_CHUNK = SCAN_THREADS * SCAN_ITEMS;

// Inclusive block scan of one int64 per thread (wave64 shuffles + LDS across waves).
__device__ inline long long block_incl_scan(long long x, long long* lds_waves, long long* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        long long y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) lds_waves[wave] = x;
    __syncthreads();
    long long off = 0, all = 0;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) {
        long long s = lds_waves[w];
        if (w < wave) off += s;
        all += s;
    }
    __syncthreads();
    if (total) *total = all;
    return x + off;
}

__global__ void __launch_bounds__(SCAN_THREADS) k_scan_block_sums(const int32_t* __restrict__ in,
                                                                  int64_t n,
                                                                  long long* __restrict__ sums)
{
    __shared__ long long lds[SCAN_THREADS / 64];
    const int64_t base = (int64_t)blockIdx.x * SCAN_CHUNK;
    long long s = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        int64_t i = base + (int64_t)k * SCAN_THREADS + threadIdx.x;
        if (i < n) s += in[i];
    }
    long long tot;
    block_incl_scan(s, lds, &tot);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// Single block: exclusive scan of the block sums in place, grand total to *total.
__global__ void __launch_bounds__(1024) k_scan_sums(long long* __restrict__ sums, int64_t nb,
                                                    long long* __restrict__ total)
{
    __shared__ long long lds[1024 / 64];
    long long carry = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += 1024) {
        int64_t i = b0 + threadIdx.x;
        long long v = i < nb ? sums[i] : 0;
        long long tot;
        long long inc = block_incl_scan(v, lds, &tot);
        if (i < nb) sums[i] = carry + inc - v;
        carry += tot;
    }
    if (threadIdx.x == 0) *total = carry;
}

__global__ void __launch_bounds__(SCAN_THREADS) k_scan_apply(const int32_t* __restrict__ in,
                                                             int64_t n,
                                                             const long long* __restrict__ sums,
                                                             const long long* __restrict__ total,
                                                             int32_t* __restrict__ out)
{
    __shared__ long long lds[SCAN_THREADS / 64];
    const int64_t base = (int64_t)blockIdx.x * SCAN_CHUNK + (int64_t)threadIdx.x * SCAN_ITEMS;
    int32_t v[SCAN_ITEMS];
    long long s = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        int64_t i = base + k;
        v[k] = i < n ? in[i] : 0;
        s += v[k];
    }
    long long inc = block_incl_scan(s, lds, nullptr);
    long long run = sums[blockIdx.x] + inc - s;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        int64_t i = base + k;
        if (i < n) out[i] = (int32_t)run;
        run += v[k];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = (int32_t)*total;
}

// Apply pass that forms its own block offset: the sum of the block sums before it
// (read by the whole block; used when there are few blocks, so the extra reads are
// small and the single-block pass over the sums is not needed).  The last block
// writes the grand total.
constexpr int64_t SCAN2_MAX_BLOCKS = 1024;

__global__ void __launch_bounds__(SCAN_THREADS) k_scan_apply_self(const int32_t* __restrict__ in, int64_t n,
                                                                  const long long* __restrict__ sums,
                                                                  long long* __restrict__ total,
                                                                  int32_t* __restrict__ out)
{
    __shared__ long long lds[SCAN_THREADS / 64];
    long long p = 0;
    for (int64_t i = threadIdx.x; i < (int64_t)blockIdx.x; i += SCAN_THREADS) p += sums[i];
    long long pre;
    block_incl_scan(p, lds, &pre);
    const int64_t base = (int64_t)blockIdx.x * SCAN_CHUNK + (int64_t)threadIdx.x * SCAN_ITEMS;
    int32_t v[SCAN_ITEMS];
    long long s = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        int64_t i = base + k;
        v[k] = i < n ? in[i] : 0;
        s += v[k];
    }
    long long btot;
    long long inc = block_incl_scan(s, lds, &btot);
    long long run = pre + inc - s;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        int64_t i = base + k;
        if (i < n) out[i] = (int32_t)run;
        run += v[k];
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        out[n] = (int32_t)(pre + btot);
        *total = pre + btot;
    }
}

// Single block of 1024 threads: the whole scan for short inputs (one launch).
// Thread t owns items [16 t, 16 t + 16), read as four 16-byte loads when both
// arrays are 16-byte aligned.
constexpr int SCAN1_THREADS = 1024;
constexpr int SCAN1_ITEMS = 16;
constexpr int64_t SCAN1_MAX = (int64_t)SCAN1_THREADS * SCAN1_ITEMS;

__global__ void __launch_bounds__(SCAN1_THREADS) k_scan_single(const int32_t* __restrict__ in, int64_t n,
                                                               int32_t* __restrict__ out,
                                                               long long* __restrict__ total)
{
    __shared__ long long lds[SCAN1_THREADS / 64];
    const int64_t base = (int64_t)threadIdx.x * SCAN1_ITEMS;
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 &&
                     base + SCAN1_ITEMS <= n;
    int32_t v[SCAN1_ITEMS];
    if (vec) {
#pragma unroll
        for (int k = 0; k < SCAN1_ITEMS / 4; ++k) {
            const int4 q = reinterpret_cast<const int4*>(in + base)[k];
            v[4 * k] = q.x;
            v[4 * k + 1] = q.y;
            v[4 * k + 2] = q.z;
            v[4 * k + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < SCAN1_ITEMS; ++k) v[k] = base + k < n ? in[base + k] : 0;
    }
    long long s = 0;
#pragma unroll
    for (int k = 0; k < SCAN1_ITEMS; ++k) s += v[k];
    long long tot;
    const long long inc = block_incl_scan(s, lds, &tot);
    long long run = inc - s;
    int32_t o[SCAN1_ITEMS];
#pragma unroll
    for (int k = 0; k < SCAN1_ITEMS; ++k) {
        o[k] = (int32_t)run;
        run += v[k];
    }
    if (vec) {
#pragma unroll
        for (int k = 0; k < SCAN1_ITEMS / 4; ++k)
            reinterpret_cast<int4*>(out + base)[k] = make_int4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < SCAN1_ITEMS; ++k)
            if (base + k < n) out[base + k] = o[k];
    }
    if (threadIdx.x == 0) {
        out[n] = (int32_t)tot;
        *total = tot;
    }
}

// ---------------------------------------------------------------------------
// single-launch scan with a decoupled look-back
// ---------------------------------------------------------------------------
// Blocks take tickets in start order; block b sums its SCAN_CHUNK items, publishes
// the sum (flag AGG), and one wave walks back over the blocks before it, 64 status
// words per round trip, adding aggregates up to the first inclusive prefix (flag
// PREFIX); it then publishes its own prefix and writes its items.  A block waits
// only for blocks with smaller tickets, which run already and publish before they
// wait, so every wait ends; it is still bounded (SCAN_SPIN_LIMIT polls).
constexpr unsigned long long SC_AGG = 1ull << 62, SC_PREFIX = 2ull << 62, SC_VALUE = SC_AGG - 1ull;
constexpr int SCAN_SPIN_LIMIT = 1 << 18;

__device__ __forceinline__ unsigned long long sc_load(const unsigned long long* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void sc_store(unsigned long long* p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// status: one word per block, then the ticket counter (low 32 bits of one more word);
// all zero on entry.
__global__ void __launch_bounds__(SCAN_THREADS) k_scan_lb(const int32_t* __restrict__ in, int64_t n,
                                                          int32_t* __restrict__ out, long long* __restrict__ total,
                                                          unsigned long long* __restrict__ status,
                                                          const int32_t* __restrict__ skip)
{
    if (skip && *skip) return;  // uniform
    __shared__ long long lds[SCAN_THREADS / 64];
    __shared__ int s_blk;
    __shared__ long long s_pre;
    if (threadIdx.x == 0) s_blk = (int)atomicAdd(reinterpret_cast<unsigned int*>(status + gridDim.x), 1u);
    __syncthreads();
    const int blk = s_blk;
    const int64_t base = (int64_t)blk * SCAN_CHUNK + (int64_t)threadIdx.x * SCAN_ITEMS;
    int32_t v[SCAN_ITEMS];
    long long s = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        const int64_t i = base + k;
        v[k] = i < n ? in[i] : 0;
        s += v[k];
    }
    long long btot;
    const long long inc = block_incl_scan(s, lds, &btot);
    if (threadIdx.x == 0) sc_store(status + blk, (blk == 0 ? SC_PREFIX : SC_AGG) | (unsigned long long)btot);
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        long long excl = 0;
        int spins = 0;
        for (int j = blk - 1; j >= 0;) {  // uniform over the wave
            const unsigned long long st = j - lane >= 0 ? sc_load(status + (j - lane)) : SC_PREFIX;
            const unsigned long long pm = __ballot((st & SC_PREFIX) != 0);
            const unsigned long long zm = __ballot((st & (SC_PREFIX | SC_AGG)) == 0);
            const int p = pm ? __builtin_ctzll(pm) : 64, z = zm ? __builtin_ctzll(zm) : 64;
            const int take = min(p + 1, z);  // published words, up to and including the first prefix
            long long x = lane < take ? (long long)(st & SC_VALUE) : 0;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
            excl += x;
            if (p < z) break;
            j -= take;
            if (z < 64) {  // an unpublished word: wait for it
                if (++spins > SCAN_SPIN_LIMIT) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            if (blk > 0) sc_store(status + blk, SC_PREFIX | (unsigned long long)(excl + btot));
            s_pre = excl;
        }
    }
    __syncthreads();
    long long run = s_pre + inc - s;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        const int64_t i = base + k;
        if (i < n) out[i] = (int32_t)run;
        run += v[k];
    }
    if (blk == (int)gridDim.x - 1 && threadIdx.x == 0) {
        out[n] = (int32_t)(s_pre + btot);
        *total = s_pre + btot;
    }
}

int64_t scan_lb_clear_words(int64_t n) { return n <= SCAN1_MAX ? 0 : div_up(n, SCAN_CHUNK) + 1; }

gm_status exclusive_scan_lb(const int32_t* in, int32_t* out, int64_t n, long long* total, void* ws,
                            hipStream_t stream, const int32_t* skip)
{
    if (n <= SCAN1_MAX) {
        k_scan_single<<<1, SCAN1_THREADS, 0, stream>>>(in, n, out, total);
        GM_LAUNCH_CHECK();
        return GM_OK;
    }
    k_scan_lb<<<(unsigned)div_up(n, SCAN_CHUNK), SCAN_THREADS, 0, stream>>>(in, n, out, total,
                                                                         (unsigned long long*)ws, skip);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

size_t scan_ws_bytes(int64_t n)
{
    int64_t nb = div_up(n > 0 ? n : 1, SCAN_CHUNK);
    return align_up(sizeof(long long) * (size_t)(nb + 1), 256);
}

// The total is written to *total (device) even when it overflows int32; callers
// check it before trusting out[].
gm_status exclusive_scan(const int32_t* in, int32_t* out, int64_t n, long long* total, void* ws,
                         hipStream_t stream)
{
    if (n <= SCAN1_MAX) {
        k_scan_single<<<1, SCAN1_THREADS, 0, stream>>>(in, n, out, total);
        GM_LAUNCH_CHECK();
        return GM_OK;
    }
    int64_t nb = div_up(n, SCAN_CHUNK);
    long long* sums = (long long*)ws;
    k_scan_block_sums<<<(unsigned)nb, SCAN_THREADS, 0, stream>>>(in, n, sums);
    GM_LAUNCH_CHECK();
    if (nb <= SCAN2_MAX_BLOCKS) {
        k_scan_apply_self<<<(unsigned)nb, SCAN_THREADS, 0, stream>>>(in, n, sums, total, out);
        GM_LAUNCH_CHECK();
        return GM_OK;
    }
    k_scan_sums<<<1, 1024, 0, stream>>>(sums, nb, total);
    GM_LAUNCH_CHECK();
    k_scan_apply<<<(unsigned)nb, SCAN_THREADS, 0, stream>>>(in, n, sums, total, out);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

// ---------------------------------------------------------------------------
// mip pyramid (box filter)
// ---------------------------------------------------------------------------
__global__ void k_mip_level(const float* __restrict__ src, int s, float* __restrict__ dst)
{
    const int h = s >> 1;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= h * h * 3) return;
    const int c = i % 3, x = (i / 3) % h, y = i / (3 * h);
    const float a = src[((2 * y) * s + 2 * x) * 3 + c];
    const float b = src[((2 * y) * s + 2 * x + 1) * 3 + c];
    const float d = src[((2 * y + 1) * s + 2 * x) * 3 + c];
    const float e = src[((2 * y + 1) * s + 2 * x + 1) * 3 + c];
    dst[i] = 0.25f * ((a + b) + (d + e));
}

}  // namespace gm

using namespace gm;

extern "C" {

const char* gm_last_error(void) { return g_err; }

int32_t gm_version(void) { return 100; }

size_t gm_mipmaps_floats(int32_t S)
{
    size_t n = 0;
    for (int32_t s = S; s >= 1; s >>= 1) n += (size_t)s * s * 3;
    return n;
}

gm_status gm_build_mipmaps(const float* tex, int32_t S, float* mips, hipStream_t stream)
{
    clear_error();
    GM_ARG_CHECK(tex && mips, "texture or mip buffer is NULL");
    GM_ARG_CHECK(S > 0 && (S & (S - 1)) == 0 && S <= 16384, "texture side %d is not a power of two", S);
    GM_HIP_CHECK(hipMemcpyAsync(mips, tex, sizeof(float) * (size_t)S * S * 3, hipMemcpyDeviceToDevice,
                                stream));
    float* src = mips;
    for (int s = S; s > 1; s >>= 1) {
        float* dst = src + (size_t)s * s * 3;
        int n = (s / 2) * (s / 2) * 3;
        k_mip_level<<<(unsigned)div_up(n, 256), 256, 0, stream>>>(src, s, dst);
        GM_LAUNCH_CHECK();
        src = dst;
    }
    return GM_OK;
}

}  // extern "C"
