// Interval-owned, depth-weighted scatter-reduce (BEV pooling) for gfx950.
//
// What is computed ("Accelerating BEV Pooling on NVIDIA GPUs for Physical AI
// Applications", section "Remove redundant scatter traffic"):
//     out[ranks_bev[t], c] += depth[ranks_depth[t]] * feat[ranks_feat[t], c]
// How the work is owned (section "Implement the interval-owned
// scatter-reduce"): each interval of points sharing one cell has a single
// owner that walks its points, loads each point's depth once, accumulates
// every channel locally and writes the cell once -- no atomics, and the map
// arrays carry explicit indices so nothing is divided at run time.
//
// CDNA4 mapping (our design, not the pages'):
//   * One 64-lane wavefront owns one interval.  A feature row is split into
//     G = rowbytes/16 chunks of 16 bytes; lane (g, k) = g*G + k loads chunk k
//     of point slot g, so one wave instruction gathers PPW = 64/G rows with
//     dwordx4 loads (C=80 fp16: G=10, six rows per instruction).
//   * Map indices of up to 64 points are read with one coalesced load per
//     array (non-temporal: they are read once), the depth value of each point
//     is gathered once by the lane that read its index, and both are handed
//     to the lanes of slot g with ds_bpermute.
//   * fp16 features feed v_fma_mix_f32 directly; e4m3 features go through the
//     native OCP-fp8 v_cvt_pk_f32_fp8; accumulation is fp32 in registers.
//   * The PPW partial rows are summed through a per-wave LDS slice, and the
//     owner writes the cell with non-temporal 16-byte stores so the output
//     stream does not evict feature rows from L2 (the pages' cache-streaming
//     output stores, section "Map the algorithm to hardware").
//   * Cells without points: intervals come in increasing cell order, so the
//     owner of interval i also zeroes the cells between the previous
//     interval's cell and its own, and the last owner zeroes the tail.  Every
//     output element is stored exactly once and no memset is needed.
//   * Blocks are renumbered so each of the 8 XCDs (own L2 each) takes a
//     contiguous run of intervals, i.e. a spatially coherent patch of cells.
#include <hip/hip_runtime.h>

#include "bevpool_internal.h"

namespace bevpool {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kXcds = 8;

// Element types of one 16-byte chunk.
template <int FT> struct Chunk;
template <> struct Chunk<kF32> { static constexpr int kElems = 4; };
template <> struct Chunk<kF16> { static constexpr int kElems = 8; };
template <> struct Chunk<kE4M3> { static constexpr int kElems = 16; };

// Depth values are gathered in their storage type and widened at first use,
// so the gather can stay in flight while other work issues.
template <int DT> struct DepthT;
template <> struct DepthT<kF32> { using type = float; };
template <> struct DepthT<kF16> { using type = _Float16; };

// acc[e] += d * value(e) for the elements of one 16-byte chunk.
template <int FT> __device__ inline void accumulate(float *acc, float d, u32x4 v);
template <> __device__ inline void accumulate<kF32>(float *acc, float d, u32x4 v)
{
    const f32x4 f = __builtin_bit_cast(f32x4, v);   // whole-vector cast
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(d, f[e], acc[e]);
}
template <> __device__ inline void accumulate<kF16>(float *acc, float d, u32x4 v)
{
    const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(d, static_cast<float>(h[e]), acc[e]);
}
template <> __device__ inline void accumulate<kE4M3>(float *acc, float d, u32x4 v)
{
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

// Block index -> work index such that XCD x (blocks x, x+8, x+16, ... under
// round-robin dispatch) receives one contiguous range of work indices.
__device__ inline int xcd_contiguous_block(int bid, int nblocks)
{
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int x = bid % kXcds, slot = bid / kXcds;
    return x * q + min(x, r) + slot;
}

__device__ inline void zero_cells(float *out, int C, int cell_lo, int cell_hi, int lane)
{
    if (cell_hi <= cell_lo) return;
    f32x4 *o = reinterpret_cast<f32x4 *>(out);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const int q0 = cell_lo * (C / 4), q1 = cell_hi * (C / 4);
    for (int q = q0 + lane; q < q1; q += kWave) __builtin_nontemporal_store(z, o + q);
}

// Lane i reads the map indices of point t0 + min(i, n - 1), 1 <= n <= 64:
// lanes past the batch repeat its last point, so every address derived from
// them stays in bounds and no lane needs an exec-masked branch.
__device__ inline void load_indices(const FwdParams &p, int t0, int n, int lane, int &row,
                                    int &didx)
{
    const int t = t0 + min(lane, n - 1);
    row = __builtin_nontemporal_load(p.ranks_feat + t);
    didx = __builtin_nontemporal_load(p.ranks_depth + t);
}

// G_CT > 0: lanes per point fixed at compile time; G_CT == 0: p.chunks.
template <int DT, int FT, int G_CT>
__global__ __launch_bounds__(kBlock) void bev_pool_fwd(FwdParams p)
{
    constexpr int E = Chunk<FT>::kElems;
    constexpr int PPW_CT = G_CT > 0 ? kWave / G_CT : 1;
    // sub-iterations (PPW rows each) whose feature loads are in flight together:
    // a whole 64-point batch when it fits in 16 loads of 16 bytes per lane
    constexpr int NS_FULL = (kWave + PPW_CT - 1) / PPW_CT;
    constexpr int SUB = G_CT > 0 ? (NS_FULL > 16 ? 16 : NS_FULL) : 4;
    constexpr int CH = 4;   // sub-iterations per branch-free chunk
    __shared__ __attribute__((aligned(16))) float red[kWavesPerBlock][kWave * E];

    const int G = G_CT > 0 ? G_CT : p.chunks;
    const int PPW = G_CT > 0 ? PPW_CT : kWave / G;
    const int lane = __lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int iv = xcd_contiguous_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
    if (iv >= p.n_intervals) return;

    const int C = p.C;
    const int start = p.interval_starts[iv];
    const int len = p.interval_lengths[iv];

    const int g = lane / G;
    const int k = lane - g * G;
    const bool slot_ok = g < PPW;
    const u32x4 *feat = static_cast<const u32x4 *>(p.feat);

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;

    using DRaw = typename DepthT<DT>::type;
    const DRaw *depth = static_cast<const DRaw *>(p.depth);

    // Points are walked in batches of 64.  For batch b the feature rows are
    // requested first (they need only the row indices), then the batch's
    // depth values (their indices are already here), then the indices of
    // batch b+1; accumulation waits for all of it.  Nothing is in flight
    // across the loop edge, so a batch costs one memory round trip once its
    // indices are known, and the first batch two.
    const int n_batches = (len + kWave - 1) / kWave;
    int row0, didx0;
    load_indices(p, start, min(kWave, len), lane, row0, didx0);

    for (int b = 0; b < n_batches; ++b) {
        const int nb = min(kWave, len - b * kWave);
        const bool more = b + 1 < n_batches;                  // wave-uniform
        const int my_chunk = row0 * G;
        DRaw draw = DRaw(0);
        int row1 = 0, didx1 = 0;
        for (int s0 = 0; s0 < nb; s0 += SUB * PPW) {
            u32x4 v[SUB];
            // Chunks of CH sub-iterations are branch-free: every lane loads an
            // in-bounds row (lanes past the batch repeat its last point, k < G),
            // slots without a point are zeroed by select at first use, so the
            // shuffles and loads of a chunk issue back to back.  Only the chunk
            // guard, which is wave-uniform, branches.
#pragma unroll
            for (int c = 0; c < SUB; c += CH) {
                if (s0 + c * PPW < nb) {
#pragma unroll
                    for (int u = c; u < c + CH && u < SUB; ++u) {
                        const int j = s0 + u * PPW + g;
                        const int row = __shfl(my_chunk, j & (kWave - 1));
                        v[u] = feat[row + k];
                    }
                }
            }
            if (s0 == 0) {
                draw = depth[didx0];
                if (more)
                    load_indices(p, start + (b + 1) * kWave, min(kWave, len - (b + 1) * kWave),
                                 lane, row1, didx1);
            }
            // depth values and the validity selects are first needed here
            const float my_d = static_cast<float>(draw);
#pragma unroll
            for (int c = 0; c < SUB; c += CH) {
                if (s0 + c * PPW < nb) {
#pragma unroll
                    for (int u = c; u < c + CH && u < SUB; ++u) {
                        const int j = s0 + u * PPW + g;
                        const float d = __shfl(my_d, j & (kWave - 1));
                        const bool ok = slot_ok && j < nb;
                        accumulate<FT>(acc, ok ? d : 0.f, ok ? v[u] : u32x4{0u, 0u, 0u, 0u});
                    }
                }
            }
        }
        row0 = row1;
        didx0 = didx1;
    }
    if (FT == kE4M3) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= p.feat_scale;
    }

    // sum the PPW partial rows: red[w][g*C + k*E + e]
    float *r = red[wv];
    if (slot_ok) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
            *reinterpret_cast<f32x4 *>(r + g * C + k * E + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int bev = p.ranks_bev[start];
    const int prev_bev = iv > 0 ? p.ranks_bev[start - 1] : -1;
    f32x4 *o = reinterpret_cast<f32x4 *>(p.out);
    const int C4 = C / 4;
    for (int q = lane; q < C4; q += kWave) {
        f32x4 s = *reinterpret_cast<const f32x4 *>(r + 4 * q);
        for (int gg = 1; gg < PPW; ++gg) s += *reinterpret_cast<const f32x4 *>(r + gg * C + 4 * q);
        __builtin_nontemporal_store(s, o + bev * C4 + q);
    }

    zero_cells(p.out, C, prev_bev + 1, bev, lane);
    if (iv == p.n_intervals - 1) zero_cells(p.out, C, bev + 1, p.n_cells, lane);
}

__global__ __launch_bounds__(kBlock) void zero_fill(f32x4 *out, int n4)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < n4; i += gridDim.x * kBlock)
        __builtin_nontemporal_store(z, out + i);
}

template <int DT, int FT>
hipError_t launch_typed(const FwdParams &p, hipStream_t s)
{
    const int blocks = (p.n_intervals + kWavesPerBlock - 1) / kWavesPerBlock;
#define BEVPOOL_CASE(GV)                                                    \
    case GV: bev_pool_fwd<DT, FT, GV><<<blocks, kBlock, 0, s>>>(p); break;
    switch (p.chunks) {
        BEVPOOL_CASE(1) BEVPOOL_CASE(2) BEVPOOL_CASE(4) BEVPOOL_CASE(5) BEVPOOL_CASE(8)
        BEVPOOL_CASE(10) BEVPOOL_CASE(16) BEVPOOL_CASE(20) BEVPOOL_CASE(32) BEVPOOL_CASE(64)
    default: bev_pool_fwd<DT, FT, 0><<<blocks, kBlock, 0, s>>>(p); break;
    }
#undef BEVPOOL_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t run_forward(const FwdParams &p, hipStream_t s)
{
    if (p.n_intervals == 0) {
        const int n4 = p.n_cells * (p.C / 4);
        const int blocks = min((n4 + kBlock - 1) / kBlock, 4096);
        zero_fill<<<blocks, kBlock, 0, s>>>(reinterpret_cast<f32x4 *>(p.out), n4);
        return hipGetLastError();
    }
    if (p.depth_dtype == kF32 && p.feat_dtype == kF32) return launch_typed<kF32, kF32>(p, s);
    if (p.depth_dtype == kF16 && p.feat_dtype == kF16) return launch_typed<kF16, kF16>(p, s);
    if (p.depth_dtype == kF16 && p.feat_dtype == kE4M3) return launch_typed<kF16, kE4M3>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace bevpool
