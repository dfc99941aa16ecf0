// Internal launch interface between the C ABI (bevpool_api.cpp) and the
// gfx950 kernels (map_kernels.hip, forward_kernels.hip).  Not installed.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace bevpool {

// ---- map build -------------------------------------------------------------
struct MapParams {
    const int32_t *point_cell;   // [P]
    int32_t P;                   // n_img * D * H * W (< 2^31)
    int32_t DHW, HW;             // D*H*W and H*W, for the feature-row of point p
    int64_t n_cells;
    int32_t capacity;            // min(capacity, INT32_MAX) of the five output arrays
    int32_t *ranks_depth, *ranks_feat, *ranks_bev, *interval_starts, *interval_lengths;
    void *workspace;
    size_t workspace_bytes;
};

// Device workspace for a frustum of P points (256-byte aligned sub-buffers).
size_t map_workspace_bytes(int64_t P);

// Enqueue the map build; on return the three counters (kept points,
// intervals, out-of-range cells) sit at h_counts after a stream sync.
hipError_t run_build_map(const MapParams &p, int32_t h_counts[3], hipStream_t stream);

// Size of the per-device static workspace of bevpool_build_map_no_alloc
// (BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES in bevpool.h).
constexpr size_t kMapScratchBytes = size_t(80) << 20;

// Device address of the current device's static map workspace (looked up
// once per device).
hipError_t map_scratch(void **ptr);

// ---- forward -----------------------------------------------------------------
enum DType : int32_t { kF32 = 0, kF16 = 1, kE4M3 = 2, kBF16 = 3 };

struct FwdParams {
    const void *depth;
    const void *feat;            // [rows, C], 16-byte aligned
    float feat_scale;
    int32_t C;
    int32_t chunks;              // 16-byte chunks per feature row (= G lanes per point)
    const int32_t *ranks_depth, *ranks_feat, *ranks_bev, *interval_starts, *interval_lengths;
    int32_t n_points, n_intervals;
    int32_t n_long_blocks;       // blocks in the long-interval role (set by run_forward)
    int32_t xcd_run;             // short-role blocks per XCD run (set by run_forward; 1 = plain order)
    int32_t first_short;         // first short-role block of a launch (set by run_forward)
    int32_t short_base;          // logical short-role block of that block (set by run_forward)
    int64_t table_bytes;         // feature-table bytes (n_feat_rows * row bytes)
    void *out;                   // [n_cells, C] of out_dtype, 16-byte aligned
    int32_t out_dtype;           // kF32, kF16 or kBF16
    int32_t n_cells;
    int32_t depth_dtype, feat_dtype;
};

hipError_t run_forward(const FwdParams &p, hipStream_t stream);

// Segment mode of the same kernel: interval_starts holds n_intervals + 1
// offsets, cell i is segment i, depth (nullable) holds one weight per point,
// and ranks_depth / ranks_bev / interval_lengths are unused.
hipError_t run_segment_reduce(const FwdParams &p, hipStream_t stream);

// The article's earlier loop orders (comparison baselines, baseline_kernels.hip).
hipError_t run_forward_baseline(const FwdParams &p, bool tile_outer, hipStream_t stream);

}  // namespace bevpool
