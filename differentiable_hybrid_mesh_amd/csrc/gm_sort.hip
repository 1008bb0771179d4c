// Per-tile Gaussian lists in centre-depth order with the occlusion cull
// (gmesh README, "Design Details > Hybrid rendering": composited "in the usual
// sorted 3DGS order"; cull_occluded drops Gaussians certainly hidden behind the
// mesh in fully covered 16x16 tiles without changing the result).
//
// Strategy: stable LSD radix sort of the visible Gaussians by the bits of their
// fp32 depth (ties keep id order), one pass that counts the surviving tiles of
// every Gaussian in that order, a scan, one pass that emits (tile, id) pairs in
// that order, and a stable LSD radix sort of the pairs by tile.  Stability keeps
// every tile's list in (depth, id) order.  The radix passes rank keys inside a
// block with wave64 ballots (8 ballots give each lane the mask of lanes holding
// the same digit), so the scatter is stable without any sorting network.
#include <algorithm>

#include "gm_internal.h"

namespace gm {

constexpr int RS_THREADS = 256;
constexpr int RS_WAVES = RS_THREADS / 64;
constexpr int RS_ITEMS = 16;  // keys per thread of the pair sort (4096 per block)
constexpr int DS_ITEMS = 8;   // of the depth sort: 2048 per block, about 490 blocks for 1M keys (4096 per
                              // block left fewer blocks than CUs: 0.21 -> 0.19 ms; 1024: 0.206 ms)
constexpr int RS_RADIX = 256;

__global__ void k_sort_init(int32_t* __restrict__ ranges, int64_t n2, long long* __restrict__ n_keys)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n2) ranges[i] = 0;
    if (i == 0) *n_keys = 0;
}

// Live key count of a pass.  A count above the buffers' capacity means the
// emitting pass wrote nothing, so there is nothing to sort.
__device__ inline long long live_count(const long long* __restrict__ d_count, long long n_max)
{
    const long long c = *d_count;
    return c > n_max ? 0 : c;
}

// ---------------------------------------------------------------------------
// stable LSD radix sort pass over a digit of BITS <= 8 bits
// ---------------------------------------------------------------------------
// The top-byte pass of the 32-bit depth sort is skipped on the device when every
// listed key (not all ones) has the same top byte and none has all ones in its low 24
// bits: after the three low-byte passes the order is then already the final one (the
// unlisted keys, all ones, sort after every listed one on their low 24 bits, in index
// order).  The first pass's histogram blocks record, per block, the OR and the AND of
// the listed keys' top bytes, whether a listed key has a low 24 bits of all ones, and
// the unlisted count; block 0 of the second pass's histogram reduces them to the skip
// flag and the listed count, which the last pass's kernels read.
struct TopSkip {
    int4* stats_out = nullptr;       // first pass: per-block record
    const int4* stats_in = nullptr;  // second pass: the records ...
    int32_t* flag_out = nullptr;     // ... reduced by block 0 to {skip, listed count}
    const int32_t* flag = nullptr;   // last pass: skip when flag[0]; flag[1] = listed count
    int32_t* count_out = nullptr;    // last pass, skipped: where the listed count is read
};

__device__ __forceinline__ void block_reduce4(int4& v, int4* s_tmp)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        v.x |= __shfl_xor(v.x, o, 64);
        v.y &= __shfl_xor(v.y, o, 64);
        v.z |= __shfl_xor(v.z, o, 64);
        v.w += __shfl_xor(v.w, o, 64);
    }
    if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    v = make_int4(0, 0xff, 0, 0);
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) {
        v.x |= s_tmp[w].x;
        v.y &= s_tmp[w].y;
        v.z |= s_tmp[w].z;
        v.w += s_tmp[w].w;
    }
}

__device__ __forceinline__ void top_stats_add(int4& st, uint32_t key)
{
    const bool listed = key != 0xffffffffu;
    const int top = (int)(key >> 24);
    st.x |= listed ? top : 0;
    st.y &= listed ? top : 0xff;
    st.z |= (listed && (key & 0xffffffu) == 0xffffffu) ? 1 : 0;
    st.w += listed ? 0 : 1;
}

// Logical index of block b when the first nlive blocks of the grid hold keys.
// Blocks are dispatched to the eight XCDs in turn (block b on XCD b % 8); among
// the live blocks XCD x takes the contiguous logical range from x q + min(x, r)
// (q = nlive / 8, r = nlive % 8), so blocks with consecutive logical indices
// (adjacent key ranges, histogram columns and digit runs) share one L2 and fill
// its lines together instead of writing parts of them from several XCDs.  Blocks
// past the live ones keep their index (their histogram columns are zeros).  A
// bijection on the grid.
__device__ __forceinline__ int xcd_block(int b, int nlive)
{
    if (b >= nlive) return b;
    const int q = nlive >> 3, r = nlive & 7, x = b & 7, i = b >> 3;
    return x * q + min(x, r) + i;
}

template <int BITS, typename KT, int ITEMS>
__global__ void __launch_bounds__(RS_THREADS)
k_radix_hist(const KT* __restrict__ keys, const long long* __restrict__ d_count, long long n_max,
             int shift, int nblocks, int32_t* __restrict__ hist, unsigned long long* __restrict__ scan_clear,
             int64_t scan_words, TopSkip ts)
{
    if (ts.flag && ts.flag[0]) return;  // uniform: the pass is skipped (so is its scan)
    constexpr int R = 1 << BITS;
    // four histograms per wave (lanes l and l + 4 share one), a word of padding each so
    // that equal digits of different copies fall in different banks: fewer colliding
    // LDS atomics
    constexpr int HC = RS_WAVES * 4, HS = RS_RADIX + 1;
    __shared__ int32_t h[HC][HS];
    __shared__ int4 s_st[RS_WAVES];
    const long long n = live_count(d_count, n_max);
    const int hc = (threadIdx.x >> 6) * 4 + (threadIdx.x & 3);
    if (ts.stats_in && blockIdx.x == 0) {  // second pass: the skip decision
        int4 st = make_int4(0, 0xff, 0, 0);
        for (int b = threadIdx.x; b < nblocks; b += RS_THREADS) {
            const int4 r = ts.stats_in[b];
            st.x |= r.x;
            st.y &= r.y;
            st.z |= r.z;
            st.w += r.w;
        }
        block_reduce4(st, s_st);
        if (threadIdx.x == 0) {
            ts.flag_out[0] = st.x == st.y && st.z == 0 ? 1 : 0;
            ts.flag_out[1] = (int32_t)(n - st.w);
        }
    }
    int4 st = make_int4(0, 0xff, 0, 0);  // first pass: this block's record
    {  // the status words of the single-launch scan that follows
        const int64_t gid = (int64_t)blockIdx.x * RS_THREADS + threadIdx.x;
        if (gid < scan_words) scan_clear[gid] = 0ull;
    }
    for (int i = threadIdx.x; i < HC * HS; i += RS_THREADS) (&h[0][0])[i] = 0;
    __syncthreads();
    // thread t counts the ITEMS consecutive keys from e0, read with 16-byte loads
    // (keys are 256-byte aligned and e0 is a multiple of ITEMS): all of a block's
    // loads are in flight together, where one key per load left it latency-bound
    constexpr int CHUNK = RS_THREADS * ITEMS;
    const int lb = xcd_block(blockIdx.x, (int)((n + CHUNK - 1) / CHUNK));
    const long long e0 = (long long)lb * CHUNK + (long long)threadIdx.x * ITEMS;
    if (e0 + ITEMS <= n) {
        static_assert(ITEMS * sizeof(KT) % 16 == 0, "whole 16-byte loads per thread");
        constexpr int NV = ITEMS * (int)sizeof(KT) / 16;
        constexpr int PER = 16 / (int)sizeof(KT);  // keys per 16-byte load
        uint4 q[NV];
        const uint4* src = reinterpret_cast<const uint4*>(keys + e0);
#pragma unroll
        for (int v = 0; v < NV; ++v) q[v] = src[v];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t w4[4] = {q[v].x, q[v].y, q[v].z, q[v].w};
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const uint32_t key = sizeof(KT) == 2 ? (w4[k >> 1] >> (16 * (k & 1))) & 0xffffu : w4[k];
                atomicAdd(&h[hc][(key >> shift) & (R - 1)], 1);
                if (ts.stats_out) top_stats_add(st, key);
            }
        }
    } else {
        for (int k = 0; k < ITEMS; ++k)
            if (e0 + k < n) {
                const uint32_t key = (uint32_t)keys[e0 + k];
                atomicAdd(&h[hc][(key >> shift) & (R - 1)], 1);
                if (ts.stats_out) top_stats_add(st, key);
            }
    }
    if (ts.stats_out) {
        __syncthreads();  // s_st may still be read by the decision above
        block_reduce4(st, s_st);
        if (threadIdx.x == 0) ts.stats_out[lb] = st;
    }
    __syncthreads();
    if (threadIdx.x < R) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < HC; ++w) c += h[w][threadIdx.x];
        hist[threadIdx.x * nblocks + lb] = c;
    }
}

// Stable scatter of one LSD pass over a block of RS_THREADS * ITEMS keys.  Wave w
// ranks its own 64 * ITEMS consecutive keys in ITEMS rounds of 64 without block
// barriers: BITS ballots
// give each lane the lanes holding the same digit, and a per-wave running count per
// digit in LDS carries the rank across rounds (a wave's LDS operations complete in
// program order).  One block scan then turns the per-wave counts into bases, keys
// are placed in LDS in digit order, and each digit's run leaves the block as
// contiguous stores.
template <int BITS, typename KT, int ITEMS>
__global__ void __launch_bounds__(RS_THREADS)
k_radix_scatter(const KT* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                const long long* __restrict__ d_count, long long n_max, int shift, int nblocks,
                const int32_t* __restrict__ offs, KT* __restrict__ keys_out, int32_t* __restrict__ vals_out,
                TopSkip ts)
{
    if (ts.flag && ts.flag[0]) {  // uniform: the order is final; move the values to the output
        const long long n = live_count(d_count, n_max);
        for (long long i = (long long)blockIdx.x * RS_THREADS + threadIdx.x; i < n;
             i += (long long)gridDim.x * RS_THREADS)
            vals_out[i] = vals_in[i];
        if (blockIdx.x == 0 && threadIdx.x == 0) *ts.count_out = ts.flag[1];
        return;
    }
    constexpr int CHUNK = RS_THREADS * ITEMS;
    __shared__ KT s_k[CHUNK];
    __shared__ int32_t s_v[CHUNK];
    __shared__ int32_t s_wc[RS_WAVES][RS_RADIX];  // running counts per wave, then per-wave bases
    __shared__ int32_t s_lstart[RS_RADIX], s_goff[RS_RADIX];
    __shared__ int32_t s_wsum[RS_WAVES];
    constexpr int R = 1 << BITS;
    const long long n = live_count(d_count, n_max);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int lb = xcd_block(blockIdx.x, (int)((n + CHUNK - 1) / CHUNK));
    const long long base = (long long)lb * CHUNK;
    if (base >= n) return;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) s_wc[w][t] = 0;
    if (t < R) s_goff[t] = offs[t * nblocks + lb];
    __syncthreads();
    uint32_t key[ITEMS];  // KT widened
    int32_t val[ITEMS];
    int rank[ITEMS];
    const long long wbase = base + (long long)wave * (CHUNK / RS_WAVES);
    const bool full = base + CHUNK <= n;  // uniform: every block but the last
    if (full) {
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            key[r] = keys_in[wbase + r * 64 + lane];
            val[r] = vals_in[wbase + r * 64 + lane];
        }
    } else {
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            const long long e = wbase + r * 64 + lane;
            const bool act = e < n;
            key[r] = act ? keys_in[e] : 0u;
            val[r] = act ? vals_in[e] : 0;
        }
    }
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const bool act = full || wbase + r * 64 + lane < n;
        const int d = (key[r] >> shift) & (R - 1);
        // lanes whose digit differs in some bit: for bit b, sgn is all ones where
        // the lane's bit is set, and ballot ^ sgn marks the lanes that disagree
        unsigned long long miss = ~__ballot(act);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            const int sgn = (int)((uint32_t)d << (31 - b)) >> 31;
            const unsigned long long bb = __ballot(sgn != 0);
            miss |= bb ^ (unsigned long long)(long long)sgn;
        }
        const unsigned long long peers = ~miss;
        const int before = s_wc[wave][d];
        rank[r] = before + __popcll(peers & lt);
        if (act && (peers >> lane) == 1ull) s_wc[wave][d] = before + __popcll(peers);  // last lane of the group
    }
    __syncthreads();
    // digit t: per-wave counts -> block-local start of the digit and per-wave bases
    int cw[RS_WAVES];
    int c = 0;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) {
        cw[w] = s_wc[w][t];
        c += cw[w];
    }
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    int wo = 0;
    for (int w = 0; w < wave; ++w) wo += s_wsum[w];
    const int lstart = wo + x - c;
    s_lstart[t] = lstart;
    int run = lstart;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) {
        s_wc[w][t] = run;
        run += cw[w];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        if (wbase + r * 64 + lane < n) {
            const int pos = s_wc[wave][(key[r] >> shift) & (R - 1)] + rank[r];
            s_k[pos] = (KT)key[r];
            s_v[pos] = val[r];
        }
    }
    __syncthreads();
    const int nvalid = (int)min((long long)CHUNK, n - base);
    for (int p = t; p < nvalid; p += RS_THREADS) {
        const KT k = s_k[p];
        const int d = (k >> shift) & (R - 1);
        const int g = s_goff[d] + (p - s_lstart[d]);
        keys_out[g] = k;
        vals_out[g] = s_v[p];
    }
}

static int radix_passes(int nbits) { return nbits <= 0 ? 1 : (nbits + 7) / 8; }

size_t radix_ws_bytes(int64_t n, int items)
{
    const int64_t nb = div_up(n > 0 ? n : 1, (int64_t)RS_THREADS * items);
    return 2 * align_up(sizeof(int32_t) * (size_t)(RS_RADIX * nb + 1), 256) + scan_ws_bytes(RS_RADIX * nb) +
           align_up(sizeof(long long), 256) + align_up(sizeof(int4) * (size_t)nb + 4 * sizeof(int32_t), 256);
}

template <int BITS, typename KT, int ITEMS>
static gm_status radix_pass(const KT* kin, const int32_t* vin, KT* kout, int32_t* vout, int shift,
                            const long long* d_count, int64_t n_max, int nb, int32_t* hist, int32_t* offs,
                            long long* tot, void* scan_ws, const TopSkip& ts, hipStream_t stream)
{
    const int64_t nscan = (int64_t)(1 << BITS) * nb;
    k_radix_hist<BITS, KT, ITEMS><<<nb, RS_THREADS, 0, stream>>>(kin, d_count, n_max, shift, nb, hist,
                                                                  (unsigned long long*)scan_ws,
                                                                  scan_lb_clear_words(nscan), ts);
    GM_LAUNCH_CHECK();
    if (gm_status s = exclusive_scan_lb(hist, offs, nscan, tot, scan_ws, stream, ts.flag)) return s;
    k_radix_scatter<BITS, KT, ITEMS><<<nb, RS_THREADS, 0, stream>>>(kin, vin, d_count, n_max, shift, nb, offs, kout,
                                                                     vout, ts);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

// Offsets ([digit][block], exclusive) of the last pass of a radix sort over at most
// n_max keys, `items` per thread, where radix_sort leaves them in its workspace.
static int32_t* radix_last_offsets(void* ws, int64_t n_max, int items)
{
    const int64_t nb = div_up(n_max > 0 ? n_max : 1, (int64_t)RS_THREADS * items);
    return (int32_t*)((char*)ws + align_up(sizeof(int32_t) * (size_t)(RS_RADIX * nb + 1), 256));
}

// Sorts n_max-bounded (keys, vals) by key bits [0, nbits) with LSD passes of at most 8
// bits, split as evenly as possible (fewer digit values per pass than 256 give longer
// runs of equal digits and so longer contiguous stores); the live count is *d_count
// (device), zero when above n_max.  Ping-pongs between (ka, va) and (kb, vb): an even
// number of passes ends in (ka, va), an odd one in (kb, vb).  The last pass's
// offsets stay in ws (radix_last_offsets) until the workspace is used again.
template <typename KT, int ITEMS>
static gm_status radix_sort(KT* ka, int32_t* va, KT* kb, int32_t* vb, int nbits,
                            const long long* d_count, int64_t n_max, void* ws, hipStream_t stream)
{
    const int nb = (int)div_up(n_max > 0 ? n_max : 1, (int64_t)RS_THREADS * ITEMS);
    char* w = (char*)ws;
    int32_t* hist = (int32_t*)w;
    int32_t* offs = radix_last_offsets(ws, n_max, ITEMS);
    w = (char*)offs + align_up(sizeof(int32_t) * (size_t)(RS_RADIX * nb + 1), 256);
    long long* tot = (long long*)w;
    w += align_up(sizeof(long long), 256);
    void* scan_ws = w;
    w += scan_ws_bytes((int64_t)RS_RADIX * nb);
    int4* ts_stats = (int4*)w;
    int32_t* ts_flag = (int32_t*)(ts_stats + nb);
    KT* kin = ka;
    int32_t* vin = va;
    KT* kout = kb;
    int32_t* vout = vb;
    const int npass = radix_passes(nbits);
    // the skippable top byte: 32-bit keys in four 8-bit passes with the multi-block scan
    const bool topskip = sizeof(KT) == 4 && nbits == 32 && npass == 4 && scan_lb_clear_words((int64_t)RS_RADIX * nb) > 0;
    int shift = 0;
    for (int p = 0; p < npass; ++p) {
        const int bits = (nbits - shift + (npass - p) - 1) / (npass - p);  // ceil(remaining / passes left)
        TopSkip ts;
        if (topskip && p == 0) ts.stats_out = ts_stats;
        if (topskip && p == 1) {
            ts.stats_in = ts_stats;
            ts.flag_out = ts_flag;
        }
        if (topskip && p == 3) {
            ts.flag = ts_flag;
            ts.count_out = offs + (size_t)(RS_RADIX - 1) * nb;
        }
        gm_status s = GM_OK;
        switch (bits) {
        case 1: s = radix_pass<1, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 2: s = radix_pass<2, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 3: s = radix_pass<3, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 4: s = radix_pass<4, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 5: s = radix_pass<5, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 6: s = radix_pass<6, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        case 7: s = radix_pass<7, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        default: s = radix_pass<8, KT, ITEMS>(kin, vin, kout, vout, shift, d_count, n_max, nb, hist, offs, tot, scan_ws, ts, stream); break;
        }
        if (s) return s;
        shift += bits;
        KT* tk = kin;
        int32_t* tv = vin;
        kin = kout;
        vin = vout;
        kout = tk;
        vout = tv;
    }
    return GM_OK;
}

// ---------------------------------------------------------------------------
// depth keys
// ---------------------------------------------------------------------------
// Key of Gaussian i: the bits of its fp32 z_c when it is listed (z_c > 0, so the bits
// order like the values and the top byte is below 0x80), all ones otherwise; the
// stable sort then puts the listed Gaussians first in (z_c, id) order, and the last
// pass's offset of top byte 0xff is their number.
__global__ void k_depth_keys(int N, const float* __restrict__ rec, uint32_t* __restrict__ keys,
                             int32_t* __restrict__ vals, long long* __restrict__ d_n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) *d_n = N;  // the key count of the sort that follows
    if (i >= N) return;
    const bool vis = __float_as_int(rec[(size_t)i * GM_REC + 15]) > 0;
    keys[i] = vis ? __float_as_uint(rec[(size_t)i * GM_REC + 9]) : 0xffffffffu;
    vals[i] = i;
}

// ---------------------------------------------------------------------------
// occlusion cull (fp32); identical code in the counting and the emitting pass
// ---------------------------------------------------------------------------
struct CullParams {
    const float* tile_dmax;  // nullptr: no culling
    float softness;
};

// f must reach (1/255)(1 - 1e-3) / min(0.99, o) for the pair to matter anywhere;
// the matching split value is s_crit = Phi^-1(that) = -sqrt(2) erfcinv(2 that), once
// per Gaussian (+inf when even f = 1 cannot reach it).
__device__ inline float cull_scrit(float o)
{
    const float amax = fminf(o, 0.99f);
    const float y = (1.0f / 255.0f) * (1.0f - 1e-3f) / amax;
    if (!(y < 1.0f)) return INFINITY;
    return -1.41421356237309515f * erfcinvf(2.0f * y);
}

// Pair (tile, Gaussian) is dropped when the tile is fully covered and
// min(0.99, o) Phi((Dmax + 1e-5 |Dmax| - zmin) / (sigma softness)) < (1/255)(1 - 1e-3),
// evaluated as Dmax + 1e-5 |Dmax| - zmin < s_crit sigma softness (sigma softness > 0;
// rounding only moves decisions inside the threshold's 1e-3 margin).  zmin is the
// conditional depth's minimum over the four corner pixel centres of the tile.
__device__ inline bool culled(const DevCamera& cam, float softness, float dmax, int tx, int ty, float u, float v,
                              float zc, float g0, float g1, float sig_soft, float scrit)
{
    // evaluated whatever dmax is (so its operands load alongside dmax); an uncovered
    // tile (dmax = +inf) keeps the pair
    const bool covered = dmax < INFINITY;
    // the tile's first and last pixel centres, in float (exact: integers + 1/2 below
    // 2^24); the last is clipped to the image's last pixel centre
    const float xa = (float)(tx * GM_TILE) + 0.5f, ya = (float)(ty * GM_TILE) + 0.5f;
    const float xb = fminf(xa + (float)(GM_TILE - 1), (float)cam.width - 0.5f);
    const float yb = fminf(ya + (float)(GM_TILE - 1), (float)cam.height - 0.5f);
    const float ax = g0 * (xa - u), bx = g0 * (xb - u);
    const float ay = g1 * (ya - v), by = g1 * (yb - v);
    const float zmin = zc + (fminf(ax, bx) + fminf(ay, by));
    const float lim = dmax + 1e-5f * fabsf(dmax);
    if (softness > 0.0f) return covered && lim - zmin < scrit * sig_soft;
    return covered && (!(zmin < lim) || scrit == INFINITY);
}

// Pairs of the visible Gaussians in depth order: a counting pass, a scan of the
// per-chunk counts, an emitting pass.
//
// A wave takes a chunk of 64 consecutive Gaussians (one per lane), prefix-sums the
// tile counts of their rects and treats the chunk's (Gaussian, tile) pairs as one
// flat sequence, 64 per step.  Lane l of a step owns flat index f = f0 + l; its
// Gaussian is the last one whose range starts at or before f: the one carried over
// from the previous step, unless one of the few Gaussians starting inside the step
// (a ballot) starts at or before f (a binary search over the starts in LDS when
// many start there).  The tile is f - start of the rect (row-major, the row from a
// reciprocal multiply) and the cull reads tile_dmax from LDS.
//
// The counting pass takes every cull decision, stores each step's ballot of
// surviving pairs (the first PW_WORDS steps of a chunk) and the chunk's count.  The
// emitting pass skips steps whose ballot is empty, reuses the stored decisions for
// the others (recomputing them only past PW_WORDS steps) and writes each chunk's
// pairs as one contiguous run in (depth, id, tile) order.
constexpr int PW_WAVES = 8;              // waves per 512-thread block
constexpr int PW_LDS_MAX_TILES = 10240;  // tile_dmax staged in LDS up to this many tiles
constexpr int PW_WORDS = 64;             // stored step ballots per chunk (4096 pairs)
constexpr int PW_COUNT_BLOCKS = 512;     // grid of the counting pass (two blocks per CU with tile_dmax in LDS)
constexpr int PW_EMIT_BLOCKS = 1024;     // grid of the emitting pass (no tile_dmax in LDS: four blocks per CU)

struct ChunkCtx {
    int wave, lane, total, start, nt;
    unsigned long long lt;
};

// Owner Gaussian (lane index in the chunk) of flat index f = f0 + lane, given the
// owner of f0 - 1 (carry); returns the owner of f0 + 63 in carry.
__device__ __forceinline__ int step_owner(const int4 (*s_gi)[64], const ChunkCtx& c, int f0, int& carry)
{
    const int f = f0 + c.lane;
    // three comparison masks ANDed (a combined bool would be turned into a vector
    // value and back)
    unsigned long long m = __ballot(c.nt > 0) & __ballot(c.start >= f0) & __ballot(c.start < f0 + 64);
    int g = carry;
    if (__popcll(m) <= 6) {
        while (m) {
            const int h = __builtin_ctzll(m);
            m &= m - 1;
            if (f >= __builtin_amdgcn_readlane(c.start, h)) g = h;
        }
    } else {
        int lo = 0, hi = 63;
        while (lo < hi) {  // last g with start[g] <= f
            const int mid = (lo + hi + 1) >> 1;
            if (s_gi[c.wave][mid].x <= f) lo = mid;
            else hi = mid - 1;
        }
        g = lo;
    }
    carry = __builtin_amdgcn_readlane(g, 63);
    return g;
}

// Owner of f0 + 63 when the step itself is skipped: the last Gaussian starting in
// the step, else the carried one.
__device__ __forceinline__ void skip_owner(const ChunkCtx& c, int f0, int& carry)
{
    const unsigned long long m = __ballot(c.nt > 0) & __ballot(c.start >= f0) & __ballot(c.start < f0 + 64);
    if (m) carry = 63 - __builtin_clzll(m);
}

// LDS: tile_dmax is staged in LDS (a compile-time choice, so the cull's read is a
// plain LDS load rather than a generic one through a pointer picked at run time).
// The counting pass also clears the tile ranges (n2 ints; grid-stride), which
// only the range kernel at the end writes again (one launch fewer).
template <bool EMIT, bool LDS, typename KT>
__global__ void __launch_bounds__(64 * PW_WAVES)
k_pairs(DevCamera cam, CullParams cp, const int32_t* __restrict__ d_nvis, int nchunks,
        const int32_t* __restrict__ order, const float* __restrict__ rec, int32_t* __restrict__ chunk_cnt,
        const int32_t* __restrict__ chunk_off, unsigned long long* __restrict__ bits,
        int2* __restrict__ crect, const long long* __restrict__ d_total, long long cap, KT* __restrict__ tkeys,
        int32_t* __restrict__ tvals, int32_t* __restrict__ ranges, int64_t n2)
{
    if (!EMIT)
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n2; i += (int64_t)gridDim.x * blockDim.x)
            ranges[i] = 0;
    extern __shared__ float s_dmax[];       // tile_dmax when LDS
    __shared__ int4 s_gi[PW_WAVES][64];     // first flat index in the chunk, rect lo, rect hi, id
    __shared__ float4 s_ga[PW_WAVES][64];   // u, v, z_c, g0
    __shared__ float4 s_gb[PW_WAVES][64];   // g1, sigma softness, s_crit
    __shared__ int s_next;                  // next chunk of the block, in grid strides
    ChunkCtx c;
    c.lane = threadIdx.x & 63;
    c.wave = threadIdx.x >> 6;
    c.lt = (1ull << c.lane) - 1ull;
    const int lane = c.lane, wave = c.wave;
    const int nvis = *d_nvis;
    if (EMIT && *d_total > cap) return;  // over capacity: nothing is written (uniform)
    const int T = cam.tx * cam.ty;
    if (threadIdx.x == 0) s_next = 0;
    if (LDS)
        for (int i = threadIdx.x; i < T; i += blockDim.x) s_dmax[i] = cp.tile_dmax[i];
    __syncthreads();
    // tile and id of the pair at flat index f0 + lane (owner g), and its keep
    // decision when `decide` (otherwise it is already known)
    // Straight-line: a lane past the chunk's pairs computes with t = 0, reads tile 0
    // and returns false, so the keep decision stays a comparison mask for the ballot.
    auto keep_of = [&](int f0, int g, int& tile, int& id, bool decide) -> bool {
        const int f = f0 + lane;
        const bool in = f < c.total;
        const int4 gi = s_gi[wave][g];
        const int t = in ? f - gi.x : 0;
        const int rlo = gi.y, rhi = gi.z;
        const int x0 = rlo & 0xffff, y0 = rlo >> 16, w = (rhi & 0xffff) - x0;
        // row = floor(t / w): the quotient's fraction is at least 1/(2w) away from an
        // integer and t < 2^20, so one reciprocal multiply is exact enough
        const int q = (int)(((float)t + 0.5f) * __builtin_amdgcn_rcpf((float)w));
        const int ty = y0 + q, tx = x0 + (t - (int)__umul24(q, w));  // 24-bit products: full rate
        // a lane past the chunk's pairs may have an owner whose rect this wave never
        // wrote (a chunk past the listed Gaussians, or a trailing lane found by the
        // binary search): its tile is then garbage, so it reads tile 0 instead
        tile = in ? (int)__umul24(ty, cam.tx) + tx : 0;
        id = gi.w;
        if (!decide || !cp.tile_dmax) return in;  // uniform
        const float4 ga = s_ga[wave][g], gb = s_gb[wave][g];
        const float dmax = LDS ? s_dmax[tile] : cp.tile_dmax[tile];
        return in & !culled(cam, cp.softness, dmax, tx, ty, ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z);
    };
    // Block b owns chunks b, b + grid, b + 2 grid, ...; its waves take them in turn
    // from an LDS counter.  Chunk pair counts vary with the Gaussians' rects: a fixed
    // chunk per wave left the busiest wave at 1.5x the mean load (1.16x this way), and
    // one global counter serialised on its address.
    for (;;) {
        int k = 0;
        if (lane == 0) k = atomicAdd(&s_next, 1);
        const int chunk = (int)blockIdx.x + __builtin_amdgcn_readfirstlane(k) * (int)gridDim.x;
        if (chunk >= nchunks) break;
        const int jl = chunk * 64 + lane;
        int nt = 0;
        // the counting pass reads the records (the cull needs them) and keeps each
        // Gaussian's rect in depth order (crect); the emitting pass reads that instead
        // of gathering 64-byte records again
        auto stage_cull = [&](int id) {
            const float4* r = reinterpret_cast<const float4*>(rec + (size_t)id * GM_REC);
            const float4 a = r[0], b = r[1], cc = r[2], d = r[3];
            s_ga[wave][lane] = make_float4(a.x, a.y, cc.y, cc.z);
            s_gb[wave][lane] = make_float4(cc.w, d.x * cp.softness, cull_scrit(b.y), 0.0f);
            return make_int2(__float_as_int(d.y), __float_as_int(d.z));
        };
        int id = 0;
        if (jl < nvis) {
            id = order[jl];
            const int2 lh = EMIT ? crect[jl] : stage_cull(id);
            if (!EMIT) crect[jl] = lh;
            const int lo = lh.x, hi = lh.y;
            nt = ((hi & 0xffff) - (lo & 0xffff)) * ((hi >> 16) - (lo >> 16));
            s_gi[wave][lane].y = lo;
            s_gi[wave][lane].z = hi;
            s_gi[wave][lane].w = id;
        }
        int P = nt;
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) {
            const int y = __shfl_up(P, k, 64);
            if (lane >= k) P += y;
        }
        c.nt = nt;
        c.start = P - nt;
        s_gi[wave][lane].x = c.start;
        c.total = __builtin_amdgcn_readlane(P, 63);
        // a chunk longer than the stored ballots takes the cull again past them: the
        // emitting pass then needs the records' cull fields (uniform per chunk)
        if (EMIT && c.total > PW_WORDS * 64 && jl < nvis) (void)stage_cull(id);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        unsigned long long* cbits = bits + (size_t)chunk * PW_WORDS;
        int carry = 0;
        if (!EMIT) {
            int cnt = 0;
            for (int f0 = 0, st = 0; f0 < c.total; f0 += 64, ++st) {
                const int g = step_owner(s_gi, c, f0, carry);
                int tile, id;
                const unsigned long long km = __ballot(keep_of(f0, g, tile, id, true));
                if (st < PW_WORDS && lane == 0) cbits[st] = km;
                cnt += __popcll(km);
            }
            if (lane == 0) chunk_cnt[chunk] = cnt;
        } else {
            int p = chunk_off[chunk];
            // the counting pass's decisions, one step per lane, read once per chunk
            const int nsteps = (c.total + 63) >> 6;
            const unsigned long long myword = lane < min(nsteps, PW_WORDS) ? cbits[lane] : 0ull;
            for (int f0 = 0, st = 0; f0 < c.total; f0 += 64, ++st) {
                unsigned long long km;
                int g, tile = 0, id = 0;
                if (st < PW_WORDS) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)myword, st);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(myword >> 32), st);
                    km = (unsigned long long)lo | ((unsigned long long)hi << 32);
                    if (km == 0ull) {
                        skip_owner(c, f0, carry);
                        continue;
                    }
                    g = step_owner(s_gi, c, f0, carry);
                    if ((km >> lane) & 1ull) keep_of(f0, g, tile, id, false);
                } else {
                    g = step_owner(s_gi, c, f0, carry);
                    km = __ballot(keep_of(f0, g, tile, id, true));
                }
                if ((km >> lane) & 1ull) {
                    const int q = p + __popcll(km & c.lt);
                    tkeys[q] = (KT)tile;
                    tvals[q] = id;
                }
                p += __popcll(km);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// Tile ranges from the tile-sorted keys, TR_KEYS consecutive keys per thread read
// with 16-byte loads (KT: 16-bit tile ids when the image has at most 65536 tiles,
// else 32-bit).  Key k starts its tile's range when key k - 1 differs and ends it
// when key k + 1 differs.
constexpr int TR_KEYS = 16;
template <typename KT>
__global__ void k_tile_ranges(const KT* __restrict__ keys, const long long* __restrict__ d_count,
                              long long n_max, int32_t* __restrict__ ranges)
{
    const long long K = live_count(d_count, n_max);
    const long long k0 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * TR_KEYS;
    if (k0 >= K) return;
    uint32_t v[TR_KEYS + 2];  // keys k0 - 1 .. k0 + TR_KEYS, all ones outside [0, K)
    v[0] = k0 > 0 ? keys[k0 - 1] : 0xffffffffu;
    if (k0 + TR_KEYS <= K) {  // k0 % TR_KEYS == 0, buffer 256-B aligned: whole vector loads
        constexpr int NV = TR_KEYS * (int)sizeof(KT) / 16, PER = 16 / (int)sizeof(KT);
        const uint4* src = reinterpret_cast<const uint4*>(keys + k0);
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const uint4 w = src[q];
            const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < PER; ++k)
                v[1 + q * PER + k] = sizeof(KT) == 2 ? (w4[k >> 1] >> (16 * (k & 1))) & 0xffffu : w4[k];
        }
    } else {
#pragma unroll
        for (int i = 0; i < TR_KEYS; ++i) v[1 + i] = k0 + i < K ? keys[k0 + i] : 0xffffffffu;
    }
    v[TR_KEYS + 1] = k0 + TR_KEYS < K ? keys[k0 + TR_KEYS] : 0xffffffffu;
#pragma unroll
    for (int i = 0; i < TR_KEYS; ++i) {
        const long long k = k0 + i;
        const uint32_t t = v[1 + i];
        if (k < K) {
            if (v[i] != t) ranges[2 * t] = (int32_t)k;
            if (v[2 + i] != t) ranges[2 * t + 1] = (int32_t)(k + 1);
        }
    }
}

struct SortWs {
    int32_t *cnt, *off;            // per-chunk pair counts and their exclusive prefix
    unsigned long long* bits;      // per-chunk step ballots of the counting pass
    int2* crect;                   // the listed Gaussians' rects in depth order (counting pass)
    uint32_t *dka, *dkb;
    int32_t *dva, *dvb;
    uint32_t *tka, *tkb;
    int32_t* tva;
    long long* n;
    void* scan;  // scan of the chunk counts
    void* aux;   // radix histograms and their scans
};

static size_t sort_layout(int64_t N, int64_t cap, int64_t T, char* base, SortWs* w)
{
    const int64_t n1 = N > 0 ? N : 1, c1 = cap > 0 ? cap : 1;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + o : nullptr;
        o += align_up(bytes, 256);
        return p;
    };
    SortWs s;
    const int64_t nch = div_up(n1, 64);
    s.cnt = (int32_t*)take(4 * nch);
    s.off = (int32_t*)take(4 * (nch + 1));
    s.bits = (unsigned long long*)take(8 * (size_t)nch * PW_WORDS);
    s.crect = (int2*)take(8 * (size_t)nch * 64);
    s.dka = (uint32_t*)take(4 * n1);
    s.dkb = (uint32_t*)take(4 * n1);
    s.dva = (int32_t*)take(4 * n1);
    s.dvb = (int32_t*)take(4 * n1);
    s.tka = (uint32_t*)take(4 * c1);
    s.tkb = (uint32_t*)take(4 * c1);
    s.tva = (int32_t*)take(4 * c1);
    s.n = (long long*)take(8);
    const int64_t m = std::max<int64_t>(std::max<int64_t>(n1, c1), T);
    s.scan = take(scan_ws_bytes(nch));
    s.aux = take(std::max(radix_ws_bytes(n1, DS_ITEMS), radix_ws_bytes(m, RS_ITEMS)));
    if (w) *w = s;
    return o;
}

// Host checks shared by the sort calls; fills the workspace layout.
static gm_status sort_args(const gm_camera* cam, int32_t N, const float* rec, int64_t cap, void* ws,
                           size_t ws_bytes, DevCamera* dc, SortWs* w)
{
    if (gm_status s = check_camera(cam)) return s;
    GM_ARG_CHECK(N >= 0, "N = %d is negative", N);
    GM_ARG_CHECK(ws, "ws is NULL");
    GM_ARG_CHECK(N == 0 || rec, "rec is NULL");
    GM_ARG_CHECK(cap >= 0, "cap negative");
    *dc = dev_camera(*cam);
    const int64_t T = (int64_t)dc->tx * dc->ty;
    const size_t need = sort_layout(N, cap, T, nullptr, nullptr);
    GM_ARG_CHECK(ws_bytes >= need, "workspace %zu bytes, %zu needed", ws_bytes, need);
    sort_layout(N, cap, T, (char*)ws, w);
    return GM_OK;
}

// 1. stable sort of all Gaussians by depth key; the listed ones come first.  The
// order stays in (w.dka, w.dva), the histogram offsets of the last pass in w.aux.
static gm_status sort_depth(const DevCamera& dc, int32_t N, const float* rec, const SortWs& w, hipStream_t stream)
{
    if (N == 0) return GM_OK;
    k_depth_keys<<<(unsigned)div_up(N, 256), 256, 0, stream>>>(N, rec, w.dka, w.dva, w.n);
    GM_LAUNCH_CHECK();
    return radix_sort<uint32_t, DS_ITEMS>(w.dka, w.dva, w.dkb, w.dvb, 32, w.n, N, w.aux, stream);
}

// Emission of the (tile, id) pairs with tile keys of type KT, their stable sort by
// tile and the tile ranges.
template <typename KT>
static gm_status emit_and_sort(const DevCamera& dc, const CullParams& cp, const int32_t* d_nvis, int nchunks,
                               unsigned gW, const int32_t* order, const float* rec, long long* total, int64_t kcap,
                               int64_t T, int32_t* sorted_ids, int32_t* tile_ranges, const SortWs& w,
                               hipStream_t stream)
{
    int tbits = 0;
    while (tbits < 31 && ((T - 1) >> tbits)) ++tbits;
    const int npass = radix_passes(tbits);
    KT* ka = reinterpret_cast<KT*>(w.tka);
    KT* kb = reinterpret_cast<KT*>(w.tkb);
    int32_t* va = (npass % 2 == 0) ? sorted_ids : w.tva;
    int32_t* vb = (npass % 2 == 0) ? w.tva : sorted_ids;
    k_pairs<true, false, KT><<<gW, 64 * PW_WAVES, 0, stream>>>(dc, cp, d_nvis, nchunks, order, rec, nullptr, w.off,
                                                               w.bits, w.crect, total, kcap, ka, va, nullptr, 0);
    GM_LAUNCH_CHECK();
    if (gm_status s = radix_sort<KT, RS_ITEMS>(ka, va, kb, vb, tbits, total, kcap, w.aux, stream)) return s;
    const KT* kfin = (npass % 2 == 0) ? ka : kb;
    k_tile_ranges<KT><<<(unsigned)div_up(div_up(kcap, TR_KEYS), 256), 256, 0, stream>>>(kfin, total, kcap,
                                                                                        tile_ranges);
    GM_LAUNCH_CHECK();
    return GM_OK;
}

// 2.-5. after sort_depth: pairs per chunk of 64 Gaussians in depth order (count, scan,
// emit), stable sort by tile, tile ranges.
static gm_status sort_tiles(const DevCamera& dc, int32_t N, const float* rec, const float* tile_dmax,
                            float softness, int32_t* tile_ranges, int32_t* sorted_ids, int64_t cap,
                            long long* total, const SortWs& w, hipStream_t stream)
{
    const int64_t T = (int64_t)dc.tx * dc.ty;
    if (N == 0) {  // no lists: empty ranges, no keys
        k_sort_init<<<(unsigned)div_up(2 * T, 256), 256, 0, stream>>>(tile_ranges, 2 * T, total);
        GM_LAUNCH_CHECK();
        return GM_OK;
    }
    const int32_t* order = w.dva;  // 4 passes (a skipped top-byte pass copies): back in the first buffer pair
    // number of listed Gaussians = offset of top byte 0xff in the depth sort's last
    // pass, block 0 (written there by a skipped pass too); valid until the tile sort
    // below reuses the histogram buffers
    const int32_t* d_nvis = radix_last_offsets(w.aux, N, DS_ITEMS) +
                            (size_t)(RS_RADIX - 1) * div_up(N, (int64_t)RS_THREADS * DS_ITEMS);
    const bool lds = tile_dmax && T <= PW_LDS_MAX_TILES;
    CullParams cp{tile_dmax, softness};
    const size_t shm = lds ? sizeof(float) * (size_t)T : 0;
    const int nchunks = (int)div_up(N, 64);
    const unsigned gW = (unsigned)std::min<int64_t>(div_up(nchunks, PW_WAVES), PW_COUNT_BLOCKS);
    const unsigned gE = (unsigned)std::min<int64_t>(div_up(nchunks, PW_WAVES), PW_EMIT_BLOCKS);
    auto count = lds ? k_pairs<false, true, uint16_t> : k_pairs<false, false, uint16_t>;  // no keys written
    count<<<gW, 64 * PW_WAVES, shm, stream>>>(dc, cp, d_nvis, nchunks, order, rec, w.cnt, nullptr, w.bits, w.crect,
                                              nullptr, 0, nullptr, nullptr, tile_ranges, 2 * T);  // also clears the ranges
    GM_LAUNCH_CHECK();
    if (gm_status s = exclusive_scan(w.cnt, w.off, nchunks, total, w.scan, stream)) return s;
    // 3. emit (tile, id) in depth order; 4. stable sort by tile; 5. tile ranges.
    //    Every kernel from here on compares the total with cap on the device and
    //    writes nothing above it.
    const int64_t kcap = std::min<int64_t>(cap, INT32_MAX);
    if (kcap == 0) return GM_OK;
    if (T <= 65536)  // 16-bit tile keys: 12 instead of 16 bytes per key and pass
        return emit_and_sort<uint16_t>(dc, cp, d_nvis, nchunks, gE, order, rec, total, kcap, T, sorted_ids,
                                       tile_ranges, w, stream);
    return emit_and_sort<uint32_t>(dc, cp, d_nvis, nchunks, gE, order, rec, total, kcap, T, sorted_ids, tile_ranges,
                                   w, stream);
}

}  // namespace gm

using namespace gm;

extern "C" {

size_t gm_sort_tile_keys_ws(int32_t N, int64_t cap, int32_t width, int32_t height)
{
    const int64_t T = div_up(width, GM_TILE) * div_up(height, GM_TILE);
    return sort_layout(N, cap, T, nullptr, nullptr);
}

gm_status gm_sort_depth(const gm_camera* cam, int32_t N, const float* rec, int64_t cap, void* ws, size_t ws_bytes,
                        hipStream_t stream)
{
    clear_error();
    DevCamera dc;
    SortWs w;
    if (gm_status s = sort_args(cam, N, rec, cap, ws, ws_bytes, &dc, &w)) return s;
    return sort_depth(dc, N, rec, w, stream);
}

gm_status gm_project_sort_depth(const gm_camera* cam, int32_t N, const float* means, const float* quats,
                                const float* scales, const float* opacity, const float* sh, int32_t sh_degree,
                                float* rec, int64_t cap, void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (gm_status s = check_project_args(cam, N, means, quats, scales, opacity, sh, sh_degree, rec)) return s;
    DevCamera dc;
    SortWs w;
    if (gm_status s = sort_args(cam, N, rec, cap, ws, ws_bytes, &dc, &w)) return s;
    if (N == 0) return GM_OK;
    if (gm_status s = launch_project_keys(dc, N, means, quats, scales, opacity, sh, sh_degree, rec, w.dka, w.dva,
                                          w.n, stream))
        return s;
    return radix_sort<uint32_t, DS_ITEMS>(w.dka, w.dva, w.dkb, w.dvb, 32, w.n, N, w.aux, stream);
}

gm_status gm_sort_tiles(const gm_camera* cam, int32_t N, const float* rec, const float* tile_dmax, float softness,
                        int32_t* tile_ranges, int32_t* sorted_ids, int64_t cap, int64_t* n_keys, void* ws,
                        size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    DevCamera dc;
    SortWs w;
    if (gm_status s = sort_args(cam, N, rec, cap, ws, ws_bytes, &dc, &w)) return s;
    GM_ARG_CHECK(softness >= 0.0f, "softness must be >= 0");
    GM_ARG_CHECK(tile_ranges && n_keys, "tile_ranges / n_keys is NULL");
    GM_ARG_CHECK(cap == 0 || sorted_ids, "sorted_ids is NULL");
    return sort_tiles(dc, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap,
                      reinterpret_cast<long long*>(n_keys), w, stream);
}

gm_status gm_sort_tile_keys(const gm_camera* cam, int32_t N, const float* rec, const float* tile_dmax,
                            float softness, int32_t* tile_ranges, int32_t* sorted_ids, int64_t cap,
                            int64_t* n_keys, void* ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    DevCamera dc;
    SortWs w;
    if (gm_status s = sort_args(cam, N, rec, cap, ws, ws_bytes, &dc, &w)) return s;
    GM_ARG_CHECK(softness >= 0.0f, "softness must be >= 0");
    GM_ARG_CHECK(tile_ranges && n_keys, "tile_ranges / n_keys is NULL");
    GM_ARG_CHECK(cap == 0 || sorted_ids, "sorted_ids is NULL");
    if (gm_status s = sort_depth(dc, N, rec, w, stream)) return s;
    return sort_tiles(dc, N, rec, tile_dmax, softness, tile_ranges, sorted_ids, cap,
                      reinterpret_cast<long long*>(n_keys), w, stream);
}

}  // extern "C"
