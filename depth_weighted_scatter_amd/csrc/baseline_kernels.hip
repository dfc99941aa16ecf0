// Baseline traversal orders for comparison with the interval-owned kernel.
//
// "Accelerating BEV Pooling on NVIDIA GPUs for Physical AI Applications"
// (sections "How BEVPoolV3 lowers latency" and "Remove redundant scatter
// traffic", Table 1) measures two earlier kernels:
//   * V2: channel tiles are iterated outside the scatter loop, so every tile
//     re-reads the same scatter indices (10 times for C=80 and 8-channel
//     tiles);
//   * V2+DO ("depth-outer"): each interval is visited once and all of its
//     channels are accumulated in that visit.
// Neither kernel's source is in the article; these are our own plain HIP
// versions of the two loop orders, with the same inputs and outputs as
// bevpool_forward, for measuring the ladder on MI355X.  One thread owns one
// (interval, 16-byte channel tile) pair and walks the interval's points; the
// output is zero-filled first and each owned cell is then stored once.
//   tile-outer : thread id = tile * I + interval  (a tile's pass streams all
//                indices; the next tile's pass streams them again)
//   depth-outer: thread id = interval * tiles + tile (the tiles of one
//                interval are neighbouring threads, so each index is fetched
//                once per interval and shared)
#include <hip/hip_runtime.h>

#include "bevpool_internal.h"

namespace bevpool {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 256;

template <int FT> struct Tile;   // elements of one 16-byte tile
template <> struct Tile<kF32> { static constexpr int kElems = 4; };
template <> struct Tile<kF16> { static constexpr int kElems = 8; };
template <> struct Tile<kE4M3> { static constexpr int kElems = 16; };

template <int DT> __device__ inline float depth_at(const void *d, int i)
{
    if constexpr (DT == kF32) return static_cast<const float *>(d)[i];
    else return static_cast<float>(static_cast<const _Float16 *>(d)[i]);
}

template <int FT> __device__ inline void tile_fma(float *acc, float d, u32x4 v)
{
    if constexpr (FT == kF32) {
        const f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(d, f[e], acc[e]);
    } else if constexpr (FT == kF16) {
        const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(d, static_cast<float>(h[e]), acc[e]);
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[w]), false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[w]), true);
            acc[4 * w + 0] = __builtin_fmaf(d, lo[0], acc[4 * w + 0]);
            acc[4 * w + 1] = __builtin_fmaf(d, lo[1], acc[4 * w + 1]);
            acc[4 * w + 2] = __builtin_fmaf(d, hi[0], acc[4 * w + 2]);
            acc[4 * w + 3] = __builtin_fmaf(d, hi[1], acc[4 * w + 3]);
        }
    }
}

__global__ __launch_bounds__(kBlock) void baseline_zero(f32x4 *out, int n4)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < n4; i += gridDim.x * kBlock) out[i] = z;
}

template <int DT, int FT, bool TILE_OUTER>
__global__ __launch_bounds__(kBlock) void baseline_scatter(FwdParams p, int tiles)
{
    constexpr int E = Tile<FT>::kElems;
    const int64_t id = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (id >= int64_t(p.n_intervals) * tiles) return;
    const int iv = TILE_OUTER ? int(id % p.n_intervals) : int(id / tiles);
    const int tile = TILE_OUTER ? int(id / p.n_intervals) : int(id % tiles);
    const int start = p.interval_starts[iv], len = p.interval_lengths[iv];
    const u32x4 *feat = static_cast<const u32x4 *>(p.feat);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int t = start; t < start + len; ++t) {
        const float d = depth_at<DT>(p.depth, p.ranks_depth[t]);
        tile_fma<FT>(acc, d, feat[p.ranks_feat[t] * tiles + tile]);
    }
    const float scale = FT == kE4M3 ? p.feat_scale : 1.f;
    f32x4 *o = reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) +
                                         int64_t(p.ranks_bev[start]) * p.C + tile * E);
#pragma unroll
    for (int e = 0; e < E; e += 4)
        o[e / 4] = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]} * scale;
}

template <int DT, int FT>
hipError_t launch(const FwdParams &p, bool tile_outer, hipStream_t s)
{
    const int n4 = p.n_cells * (p.C / 4);
    baseline_zero<<<min((n4 + kBlock - 1) / kBlock, 8192), kBlock, 0, s>>>(
        reinterpret_cast<f32x4 *>(p.out), n4);
    const int tiles = p.C / Tile<FT>::kElems;
    const int64_t threads = int64_t(p.n_intervals) * tiles;
    if (threads > 0) {
        const int blocks = int((threads + kBlock - 1) / kBlock);
        if (tile_outer) baseline_scatter<DT, FT, true><<<blocks, kBlock, 0, s>>>(p, tiles);
        else baseline_scatter<DT, FT, false><<<blocks, kBlock, 0, s>>>(p, tiles);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t run_forward_baseline(const FwdParams &p, bool tile_outer, hipStream_t s)
{
    if (p.depth_dtype == kF32 && p.feat_dtype == kF32) return launch<kF32, kF32>(p, tile_outer, s);
    if (p.depth_dtype == kF16 && p.feat_dtype == kF16) return launch<kF16, kF16>(p, tile_outer, s);
    if (p.depth_dtype == kF16 && p.feat_dtype == kE4M3) return launch<kF16, kE4M3>(p, tile_outer, s);
    return hipErrorInvalidValue;
}

}  // namespace bevpool
