// Scatter-map construction for BEV pooling on gfx950.
//
// "Accelerating BEV Pooling on NVIDIA GPUs for Physical AI Applications"
// names the five INT32 arrays of the map (section "Remove redundant scatter
// traffic") and has the map prepared in advance of the pooling kernel
// (section "Implement the interval-owned scatter-reduce"), but does not say
// how it is built.  Here it is a stable sort of the kept frustum points by
// cell, so points of one cell stay in increasing frustum index p: the order
// (cell, p) is total and the map is therefore unique.
//
// Pipeline (all integer work, once per geometry, outside the timed path):
//   1. LSD radix sort by cell, 8 bits or fewer per pass.  The first pass
//      also compacts away dropped points (cell -1) and counts out-of-range
//      cells.  Each pass: per-tile digit histograms -> exclusive scan over
//      (digit, tile) -> stable scatter.  Stability inside a tile comes from
//      wave ballots (lanes with the same digit, in lane order) plus per-wave
//      counts in LDS, processed in element order.
//   2. Emit ranks_bev / ranks_depth / ranks_feat from the sorted (cell, p)
//      pairs; the feature row of p is computed here, once, by division, so
//      the pooling kernel never divides.
//   3. Interval starts are the positions where the cell changes (a scan of
//      change flags gives each its interval number); lengths are differences
//      of consecutive starts.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bevpool_internal.h"

namespace bevpool {
namespace {

constexpr int kBlock = 256;           // threads per block (4 waves of 64)
constexpr int kItems = 8;             // elements per thread per tile
constexpr int kTile = kBlock * kItems;
constexpr int kMaxBins = 256;         // at most 8 radix bits per pass

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ----------------------------------------------------------------- scans
__device__ inline int wave_inclusive_scan(int v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive scan across a 256-thread block; returns the thread's exclusive
// prefix and writes the block total to *total.
__device__ inline int block_exclusive_scan(int v, int *total)
{
    __shared__ int wsum[kBlock / 64];
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    int inc = wave_inclusive_scan(v);
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i) {
        before += (i < w) ? wsum[i] : 0;
        all += wsum[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kBlock) void scan_reduce_tiles(const int *in, const int *n_dev,
                                                            int n_max, int *partials)
{
    const int n = n_dev ? *n_dev : n_max;
    const int base = blockIdx.x * kTile;
    int s = 0;
    for (int r = 0; r < kItems; ++r) {
        int i = base + r * kBlock + threadIdx.x;
        if (i < n) s += in[i];
    }
    int total;
    block_exclusive_scan(s, &total);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

// One block of 1024 threads: exclusive scan of the tile partials in place.
__global__ __launch_bounds__(1024) void scan_partials(int *partials, int nb, int *total_out)
{
    __shared__ int wsum[16];
    const int chunk = (nb + 1023) / 1024;
    const int lo = min(nb, int(threadIdx.x) * chunk), hi = min(nb, lo + chunk);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += partials[i];
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    int inc = wave_inclusive_scan(s);
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < 16; ++i) {
        before += (i < w) ? wsum[i] : 0;
        all += wsum[i];
    }
    int run = before + inc - s;
    for (int i = lo; i < hi; ++i) {
        int v = partials[i];
        partials[i] = run;
        run += v;
    }
    if (threadIdx.x == 0 && total_out) *total_out = all;
}

// Exclusive scan of one tile plus its scanned partial; may run in place.
__global__ __launch_bounds__(kBlock) void scan_tiles(const int *in, int *out, const int *n_dev,
                                                     int n_max, const int *partials)
{
    const int n = n_dev ? *n_dev : n_max;
    const int base = blockIdx.x * kTile + threadIdx.x * kItems;
    int v[kItems];
    int s = 0;
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        v[r] = (base + r < n) ? in[base + r] : 0;
        s += v[r];
    }
    int total;
    int run = block_exclusive_scan(s, &total) + partials[blockIdx.x];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        if (base + r < n) out[base + r] = run;
        run += v[r];
    }
}

// Exclusive scan of in[0, n) into out (in place allowed).  n is *n_dev when
// n_dev is given, else n_max; n_max bounds the grid.  total_out gets the sum.
hipError_t exclusive_scan(const int *in, int *out, const int *n_dev, int n_max, int *partials,
                          int *total_out, hipStream_t s)
{
    const int nb = int((int64_t(n_max) + kTile - 1) / kTile);   // n_max may be 2^31 - 1
    if (nb == 0) return hipSuccess;
    scan_reduce_tiles<<<nb, kBlock, 0, s>>>(in, n_dev, n_max, partials);
    scan_partials<<<1, 1024, 0, s>>>(partials, nb, total_out);
    scan_tiles<<<nb, kBlock, 0, s>>>(in, out, n_dev, n_max, partials);
    return hipGetLastError();
}

// ------------------------------------------------------------ radix passes
// Pass 1 reads point_cell directly (value = index p) and keeps cells in
// [0, n_cells); later passes read the previous pass's (key, value) pairs.
__device__ inline bool load_element(const int *keys, const int *vals, int idx, int n,
                                    bool first, int64_t n_cells, int &key, int &val)
{
    if (idx >= n) return false;
    key = keys[idx];
    val = first ? idx : vals[idx];
    return !first || (key >= 0 && key < n_cells);
}

__global__ __launch_bounds__(kBlock) void radix_histogram(const int *keys, const int *n_dev,
                                                          int n_max, int64_t n_cells, int first,
                                                          int shift, int bits, int *hist, int nb,
                                                          int *bad_cells)
{
    __shared__ int h[kMaxBins];
    const int nbins = 1 << bits, mask = nbins - 1;
    for (int d = threadIdx.x; d < nbins; d += kBlock) h[d] = 0;
    __syncthreads();
    const int n = n_dev ? *n_dev : n_max;
    const int base = blockIdx.x * kTile;
    int bad = 0;
    for (int r = 0; r < kItems; ++r) {
        const int idx = base + r * kBlock + threadIdx.x;
        if (idx >= n) break;
        const int key = keys[idx];
        const bool ok = !first || (key >= 0 && key < n_cells);
        if (first && (key < -1 || key >= n_cells)) ++bad;
        if (ok) atomicAdd(&h[(key >> shift) & mask], 1);
    }
    if (first && bad) atomicAdd(bad_cells, bad);
    __syncthreads();
    for (int d = threadIdx.x; d < nbins; d += kBlock) hist[d * nb + blockIdx.x] = h[d];
}

__global__ __launch_bounds__(kBlock) void radix_scatter(const int *keys, const int *vals,
                                                        const int *n_dev, int n_max,
                                                        int64_t n_cells, int first, int shift,
                                                        int bits, const int *offsets, int nb,
                                                        int *keys_out, int *vals_out)
{
    __shared__ int run_cnt[kMaxBins];
    __shared__ int wave_cnt[kBlock / 64][kMaxBins];
    const int n = n_dev ? *n_dev : n_max;
    const int base = blockIdx.x * kTile;
    if (base >= n) return;                               // uniform per block
    const int nbins = 1 << bits, mask = nbins - 1;
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1;    // lanes before this one
    for (int d = threadIdx.x; d < nbins; d += kBlock) run_cnt[d] = 0;

    for (int r = 0; r < kItems; ++r) {
        for (int j = threadIdx.x; j < (kBlock / 64) * nbins; j += kBlock)
            wave_cnt[j / nbins][j % nbins] = 0;
        __syncthreads();
        int idx = base + r * kBlock + threadIdx.x, key = 0, val = 0;
        bool ok = load_element(keys, vals, idx, n, first, n_cells, key, val);
        int digit = ok ? (key >> shift) & mask : 0;
        // lanes of this wave holding the same digit
        uint64_t peers = __ballot(ok);
        for (int b = 0; b < bits; ++b) {
            uint64_t m = __ballot((digit >> b) & 1);
            peers &= ((digit >> b) & 1) ? m : ~m;
        }
        const int rank = __popcll(peers & below);
        if (ok && rank == 0) wave_cnt[w][digit] = __popcll(peers);
        __syncthreads();
        if (ok) {
            int pos = run_cnt[digit] + rank;
            for (int v = 0; v < w; ++v) pos += wave_cnt[v][digit];
            const int dst = offsets[digit * nb + blockIdx.x] + pos;
            keys_out[dst] = key;
            vals_out[dst] = val;
        }
        __syncthreads();
        for (int d = threadIdx.x; d < nbins; d += kBlock) {
            int add = 0;
            for (int v = 0; v < kBlock / 64; ++v) add += wave_cnt[v][d];
            run_cnt[d] += add;
        }
        __syncthreads();
    }
}

// Zeroes the build's counters: a kernel rather than a memset, so the
// sequence holds kernels only.
__global__ __launch_bounds__(64) void clear_counters(int *counters, int n)
{
    if (int(threadIdx.x) < n) counters[threadIdx.x] = 0;
}

// ---------------------------------------------------------------- emission
__device__ inline bool starts_interval(const int *keys, int t)
{
    return t == 0 || keys[t - 1] != keys[t];
}

__global__ __launch_bounds__(kBlock) void emit_ranks(const int *keys, const int *vals,
                                                     const int *counters, int capacity, int DHW,
                                                     int HW, int *ranks_depth, int *ranks_feat,
                                                     int *ranks_bev, int *flags)
{
    const int n = counters[0];
    const int t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= n) return;
    const int key = keys[t], p = vals[t];
    flags[t] = starts_interval(keys, t) ? 1 : 0;
    if (n <= capacity) {
        ranks_bev[t] = key;
        ranks_depth[t] = p;
        ranks_feat[t] = (p / DHW) * HW + p % HW;   // image row block, then (h, w)
    }
}

__global__ __launch_bounds__(kBlock) void emit_starts(const int *keys, const int *ivx,
                                                      const int *counters, int capacity,
                                                      int *interval_starts)
{
    const int n = counters[0];
    const int t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= n || n > capacity) return;
    if (starts_interval(keys, t)) interval_starts[ivx[t]] = t;
}

__global__ __launch_bounds__(kBlock) void emit_lengths(const int *counters, int capacity,
                                                       const int *interval_starts,
                                                       int *interval_lengths)
{
    const int n = counters[0], I = counters[1];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= I || n > capacity) return;
    const int end = (i + 1 < I) ? interval_starts[i + 1] : n;
    interval_lengths[i] = end - interval_starts[i];
}

struct Workspace {
    int *keys[2], *vals[2], *hist, *flags, *partials, *counters;
    int nb_tiles;
};

Workspace carve(void *base, int64_t P)
{
    Workspace w{};
    char *p = static_cast<char *>(base);
    const size_t arr = align256(size_t(P) * sizeof(int));
    const int nb = int((P + kTile - 1) / kTile);
    for (int i = 0; i < 2; ++i) {
        w.keys[i] = reinterpret_cast<int *>(p); p += arr;
        w.vals[i] = reinterpret_cast<int *>(p); p += arr;
    }
    w.flags = reinterpret_cast<int *>(p); p += arr;
    w.hist = reinterpret_cast<int *>(p); p += align256(size_t(kMaxBins) * nb * sizeof(int));
    w.partials = reinterpret_cast<int *>(p);
    p += align256((size_t(kMaxBins) * nb / kTile + size_t(P) / kTile + 64) * sizeof(int));
    w.counters = reinterpret_cast<int *>(p);
    w.nb_tiles = nb;
    return w;
}

}  // namespace

size_t map_workspace_bytes(int64_t P)
{
    const int64_t nb = (P + kTile - 1) / kTile;
    const size_t arr = align256(size_t(P) * sizeof(int));
    return 5 * arr + align256(size_t(kMaxBins) * nb * sizeof(int)) +
           align256((size_t(kMaxBins) * nb / kTile + size_t(P) / kTile + 64) * sizeof(int)) +
           align256(16 * sizeof(int));
}

hipError_t run_build_map(const MapParams &mp, int32_t h_counts[3], hipStream_t s)
{
    Workspace w = carve(mp.workspace, mp.P);
    const int P = mp.P, nb = w.nb_tiles;
    int *counters = w.counters;   // [0] kept, [1] intervals, [2] bad cells, [3] spare total
    clear_counters<<<1, 64, 0, s>>>(counters, 16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // bits needed for the largest cell index
    int nbits = 1;
    while (nbits < 63 && (int64_t(1) << nbits) < mp.n_cells) ++nbits;
    const int npass = (nbits + 7) / 8;
    const int per = (nbits + npass - 1) / npass;

    const int *kin = mp.point_cell, *vin = nullptr;
    int src = 0;
    for (int pass = 0; pass < npass; ++pass) {
        const int shift = pass * per, bits = min(per, nbits - shift);
        const int first = pass == 0;
        const int *n_dev = first ? nullptr : counters;
        radix_histogram<<<nb, kBlock, 0, s>>>(kin, n_dev, P, mp.n_cells, first, shift, bits,
                                              w.hist, nb, counters + 2);
        // scanning all (digit, tile) counts; the first pass's total is the kept count
        e = exclusive_scan(w.hist, w.hist, nullptr, (1 << bits) * nb, w.partials,
                           first ? counters : counters + 3, s);
        if (e != hipSuccess) return e;
        radix_scatter<<<nb, kBlock, 0, s>>>(kin, vin, n_dev, P, mp.n_cells, first, shift, bits,
                                            w.hist, nb, w.keys[src], w.vals[src]);
        kin = w.keys[src];
        vin = w.vals[src];
        src ^= 1;
    }

    // Grid sizes are rounded up in 64 bits (P may be 2^31 - 1).  In the kernels
    // no index passes 2^31 - 1: tiles of kTile and blocks of kBlock elements
    // divide 2^31, so the last tile or block ends at or below it.
    const int grid = int((int64_t(P) + kBlock - 1) / kBlock);
    emit_ranks<<<grid, kBlock, 0, s>>>(kin, vin, counters, mp.capacity, mp.DHW, mp.HW,
                                       mp.ranks_depth, mp.ranks_feat, mp.ranks_bev, w.flags);
    e = exclusive_scan(w.flags, w.flags, counters, P, w.partials, counters + 1, s);
    if (e != hipSuccess) return e;
    emit_starts<<<grid, kBlock, 0, s>>>(kin, w.flags, counters, mp.capacity, mp.interval_starts);
    emit_lengths<<<grid, kBlock, 0, s>>>(counters, mp.capacity, mp.interval_starts,
                                         mp.interval_lengths);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(h_counts, counters, 3 * sizeof(int), hipMemcpyDeviceToHost, s)) !=
        hipSuccess)
        return e;
    return hipStreamSynchronize(s);
}

// ------------------------------------------------ workspace without allocation
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid hipMalloc), bevpool_build_map_no_alloc takes its
// workspace from this array instead of the caller.  Each device the library
// runs on holds its own copy from the module's load until the process ends.
// In host code the name stands for a host-side shadow, not a device address:
// kernels get the device address that hipGetSymbolAddress returns, looked up
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kMapScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t map_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace bevpool
