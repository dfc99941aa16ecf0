// C ABI of the BEV-pooling library: host-side validation, then dispatch to
// the gfx950 kernels.  Declarations and the contract live in bevpool.h.
#include "bevpool.h"

#include <climits>
#include <cstdint>

#include "bevpool_internal.h"

namespace {

constexpr int64_t kInt32Limit = int64_t(INT32_MAX);   // sizes must stay below 2^31
// Feature rows are addressed as a table base plus a 32-bit unsigned byte
// offset, below the range the kernels keep for empty batch slots.
constexpr int64_t kTableBytesLimit = int64_t(BEVPOOL_MAX_TABLE_BYTES);

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Frustum points n_img * D * H * W for positive factors, saturated just past
// the INT32 limit: each step multiplies a value at most 2^31 by a factor
// below 2^31, so no int64 product overflows however large the factors are.
int64_t frustum_points(int32_t n_img, int32_t D, int32_t H, int32_t W)
{
    int64_t p = n_img;
    for (const int32_t f : {D, H, W}) {
        p *= f;
        if (p > kInt32Limit) return kInt32Limit + 1;
    }
    return p;
}

int elem_bytes(int32_t dtype)
{
    switch (dtype) {
    case BEVPOOL_F32: return 4;
    case BEVPOOL_F16: return 2;
    case BEVPOOL_FP8_E4M3: return 1;
    default: return 0;   // bf16 is an output type only
    }
}

}  // namespace

extern "C" {

const char *bevpool_status_string(int status)
{
    switch (status) {
    case BEVPOOL_OK: return "ok";
    case BEVPOOL_ERR_INVALID_ARG: return "invalid argument";
    case BEVPOOL_ERR_UNSUPPORTED: return "unsupported dtype / channel combination";
    case BEVPOOL_ERR_OVERFLOW: return "size exceeds the INT32 index contract";
    case BEVPOOL_ERR_WORKSPACE: return "workspace too small or misaligned";
    case BEVPOOL_ERR_CAPACITY: return "map arrays too small for the kept points";
    case BEVPOOL_ERR_BAD_CELL: return "point_cell holds a value outside [-1, n_cells)";
    case BEVPOOL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int bevpool_version(void) { return 10000; }

size_t bevpool_build_map_workspace_size(int32_t n_img, int32_t D, int32_t H, int32_t W,
                                        int64_t n_cells)
{
    if (n_img <= 0 || D <= 0 || H <= 0 || W <= 0 || n_cells <= 0 || n_cells > kInt32Limit)
        return 0;
    const int64_t P = frustum_points(n_img, D, H, W);
    if (P > kInt32Limit) return 0;
    return bevpool::map_workspace_bytes(P);
}

int bevpool_build_map(const int32_t *point_cell, int32_t n_img, int32_t D, int32_t H, int32_t W,
                      int64_t n_cells,
                      int32_t *ranks_depth, int32_t *ranks_feat, int32_t *ranks_bev,
                      int32_t *interval_starts, int32_t *interval_lengths, int64_t capacity,
                      int32_t *h_n_points, int32_t *h_n_intervals,
                      void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!point_cell || !ranks_depth || !ranks_feat || !ranks_bev || !interval_starts ||
        !interval_lengths || !h_n_points || !h_n_intervals || !workspace)
        return BEVPOOL_ERR_INVALID_ARG;
    if (n_img <= 0 || D <= 0 || H <= 0 || W <= 0 || n_cells <= 0 || capacity < 0)
        return BEVPOOL_ERR_INVALID_ARG;
    const int64_t P = frustum_points(n_img, D, H, W);
    if (P > kInt32Limit || n_cells > kInt32Limit) return BEVPOOL_ERR_OVERFLOW;
    if (!aligned(workspace, 256) || workspace_bytes < bevpool::map_workspace_bytes(P))
        return BEVPOOL_ERR_WORKSPACE;

    bevpool::MapParams mp{};
    mp.point_cell = point_cell;
    mp.P = int32_t(P);
    mp.DHW = int32_t(int64_t(D) * H * W);
    mp.HW = int32_t(int64_t(H) * W);
    mp.n_cells = n_cells;
    mp.capacity = int32_t(capacity < kInt32Limit ? capacity : kInt32Limit);
    mp.ranks_depth = ranks_depth;
    mp.ranks_feat = ranks_feat;
    mp.ranks_bev = ranks_bev;
    mp.interval_starts = interval_starts;
    mp.interval_lengths = interval_lengths;
    mp.workspace = workspace;
    mp.workspace_bytes = workspace_bytes;

    int32_t counts[3] = {0, 0, 0};
    if (bevpool::run_build_map(mp, counts, stream) != hipSuccess) return BEVPOOL_ERR_HIP;
    *h_n_points = counts[0];
    *h_n_intervals = counts[1];
    if (counts[2] != 0) return BEVPOOL_ERR_BAD_CELL;
    if (counts[0] > capacity) return BEVPOOL_ERR_CAPACITY;
    return BEVPOOL_OK;
}

int bevpool_build_map_no_alloc(const int32_t *point_cell, int32_t n_img, int32_t D, int32_t H,
                               int32_t W, int64_t n_cells,
                               int32_t *ranks_depth, int32_t *ranks_feat, int32_t *ranks_bev,
                               int32_t *interval_starts, int32_t *interval_lengths,
                               int64_t capacity, int32_t *h_n_points, int32_t *h_n_intervals,
                               hipStream_t stream)
{
    // the size checks come first, so an oversized frustum is refused before
    // any HIP call; the remaining checks are bevpool_build_map's
    if (n_img > 0 && D > 0 && H > 0 && W > 0) {
        const int64_t P = frustum_points(n_img, D, H, W);
        if (P <= kInt32Limit && bevpool::map_workspace_bytes(P) > bevpool::kMapScratchBytes)
            return BEVPOOL_ERR_WORKSPACE;
    }
    if (!point_cell || !ranks_depth || !ranks_feat || !ranks_bev || !interval_starts ||
        !interval_lengths || !h_n_points || !h_n_intervals)
        return BEVPOOL_ERR_INVALID_ARG;
    if (n_img <= 0 || D <= 0 || H <= 0 || W <= 0 || n_cells <= 0 || capacity < 0)
        return BEVPOOL_ERR_INVALID_ARG;
    if (frustum_points(n_img, D, H, W) > kInt32Limit || n_cells > kInt32Limit)
        return BEVPOOL_ERR_OVERFLOW;
    void *ws = nullptr;
    if (bevpool::map_scratch(&ws) != hipSuccess) return BEVPOOL_ERR_HIP;
    return bevpool_build_map(point_cell, n_img, D, H, W, n_cells, ranks_depth, ranks_feat,
                             ranks_bev, interval_starts, interval_lengths, capacity, h_n_points,
                             h_n_intervals, ws, bevpool::kMapScratchBytes, stream);
}

}  // extern "C"

namespace {

// Host-side validation shared by the forward entry points; fills p.
int validate_forward(const void *depth, int32_t depth_dtype, int64_t n_depth, const void *feat,
                     int32_t feat_dtype, int64_t n_feat_rows, int32_t C, float feat_scale,
                     const int32_t *ranks_depth, const int32_t *ranks_feat,
                     const int32_t *ranks_bev, const int32_t *interval_starts,
                     const int32_t *interval_lengths, int32_t n_points, int32_t n_intervals,
                     void *out, int32_t out_dtype, int64_t n_cells, bool tiles16,
                     bevpool::FwdParams &p)
{
    if (out_dtype != BEVPOOL_F32 && out_dtype != BEVPOOL_F16 && out_dtype != BEVPOOL_BF16)
        return BEVPOOL_ERR_UNSUPPORTED;
    if (!out || n_cells <= 0 || C <= 0 || n_points < 0 || n_intervals < 0 ||
        n_intervals > n_points)
        return BEVPOOL_ERR_INVALID_ARG;
    if (n_intervals > 0 && (!depth || !feat || !ranks_depth || !ranks_feat || !ranks_bev ||
                            !interval_starts || !interval_lengths || n_depth <= 0 ||
                            n_feat_rows <= 0))
        return BEVPOOL_ERR_INVALID_ARG;

    const int fe = elem_bytes(feat_dtype);
    const bool pair_ok = (depth_dtype == BEVPOOL_F32 && feat_dtype == BEVPOOL_F32) ||
                         (depth_dtype == BEVPOOL_F16 && feat_dtype == BEVPOOL_F16) ||
                         (depth_dtype == BEVPOOL_F16 && feat_dtype == BEVPOOL_FP8_E4M3);
    if (!pair_ok || fe == 0) return BEVPOOL_ERR_UNSUPPORTED;
    // a row is split into 16-byte lane chunks (the kernels may take 8-byte
    // ones for e4m3 rows of up to 512 bytes), at most 64 per row
    const int64_t row_bytes = int64_t(C) * fe;
    const bool e4m3_small = !tiles16 && feat_dtype == BEVPOOL_FP8_E4M3 && row_bytes <= 512;
    if (row_bytes % (e4m3_small ? 8 : 16) != 0 || row_bytes > 1024) return BEVPOOL_ERR_UNSUPPORTED;

    // each count is bounded before it is multiplied, so no product overflows
    if (n_cells > kInt32Limit || n_feat_rows > kInt32Limit || n_depth > kInt32Limit ||
        n_cells * C > kInt32Limit || n_feat_rows * C > kInt32Limit ||
        n_feat_rows * row_bytes > kTableBytesLimit)
        return BEVPOOL_ERR_OVERFLOW;
    if (!aligned(out, out_dtype == BEVPOOL_F32 ? 16 : 8) || (feat && !aligned(feat, 16)) ||
        (depth && !aligned(depth, uintptr_t(elem_bytes(depth_dtype)))))
        return BEVPOOL_ERR_INVALID_ARG;

    p = bevpool::FwdParams{};
    p.depth = depth;
    p.feat = feat;
    p.feat_scale = feat_scale;
    p.C = C;
    p.chunks = int32_t(row_bytes / 16);
    p.ranks_depth = ranks_depth;
    p.ranks_feat = ranks_feat;
    p.ranks_bev = ranks_bev;
    p.interval_starts = interval_starts;
    p.interval_lengths = interval_lengths;
    p.n_points = n_points;
    p.n_intervals = n_intervals;
    p.table_bytes = n_feat_rows * row_bytes;
    p.out = out;
    p.out_dtype = out_dtype;
    p.n_cells = int32_t(n_cells);
    p.depth_dtype = depth_dtype;
    p.feat_dtype = feat_dtype;
    return BEVPOOL_OK;
}

}  // namespace

extern "C" {

int bevpool_forward_ex(const void *depth, int32_t depth_dtype, int64_t n_depth,
                       const void *feat, int32_t feat_dtype, int64_t n_feat_rows, int32_t C,
                       float feat_scale,
                       const int32_t *ranks_depth, const int32_t *ranks_feat,
                       const int32_t *ranks_bev,
                       const int32_t *interval_starts, const int32_t *interval_lengths,
                       int32_t n_points, int32_t n_intervals,
                       void *out, int32_t out_dtype, int64_t n_cells, hipStream_t stream)
{
    bevpool::FwdParams p;
    const int st = validate_forward(depth, depth_dtype, n_depth, feat, feat_dtype, n_feat_rows, C,
                                    feat_scale, ranks_depth, ranks_feat, ranks_bev,
                                    interval_starts, interval_lengths, n_points, n_intervals,
                                    out, out_dtype, n_cells, false, p);
    if (st != BEVPOOL_OK) return st;
    return bevpool::run_forward(p, stream) == hipSuccess ? BEVPOOL_OK : BEVPOOL_ERR_HIP;
}

int bevpool_forward(const void *depth, int32_t depth_dtype, int64_t n_depth,
                    const void *feat, int32_t feat_dtype, int64_t n_feat_rows, int32_t C,
                    float feat_scale,
                    const int32_t *ranks_depth, const int32_t *ranks_feat,
                    const int32_t *ranks_bev,
                    const int32_t *interval_starts, const int32_t *interval_lengths,
                    int32_t n_points, int32_t n_intervals,
                    float *out, int64_t n_cells, hipStream_t stream)
{
    return bevpool_forward_ex(depth, depth_dtype, n_depth, feat, feat_dtype, n_feat_rows, C,
                              feat_scale, ranks_depth, ranks_feat, ranks_bev, interval_starts,
                              interval_lengths, n_points, n_intervals, out, BEVPOOL_F32, n_cells,
                              stream);
}

int bevpool_forward_baseline(int32_t order, const void *depth, int32_t depth_dtype,
                             int64_t n_depth, const void *feat, int32_t feat_dtype,
                             int64_t n_feat_rows, int32_t C, float feat_scale,
                             const int32_t *ranks_depth, const int32_t *ranks_feat,
                             const int32_t *ranks_bev, const int32_t *interval_starts,
                             const int32_t *interval_lengths, int32_t n_points,
                             int32_t n_intervals, float *out, int64_t n_cells,
                             hipStream_t stream)
{
    if (order != BEVPOOL_ORDER_TILE_OUTER && order != BEVPOOL_ORDER_DEPTH_OUTER)
        return BEVPOOL_ERR_INVALID_ARG;
    bevpool::FwdParams p;
    const int st = validate_forward(depth, depth_dtype, n_depth, feat, feat_dtype, n_feat_rows, C,
                                    feat_scale, ranks_depth, ranks_feat, ranks_bev,
                                    interval_starts, interval_lengths, n_points, n_intervals,
                                    out, BEVPOOL_F32, n_cells, true, p);
    if (st != BEVPOOL_OK) return st;
    return bevpool::run_forward_baseline(p, order == BEVPOOL_ORDER_TILE_OUTER, stream) ==
                   hipSuccess
               ? BEVPOOL_OK
               : BEVPOOL_ERR_HIP;
}

int bevpool_segment_reduce(const void *weights, int32_t weight_dtype, const void *table,
                           int32_t table_dtype, int64_t n_rows, int32_t C, float table_scale,
                           const int32_t *indices, const int32_t *offsets, int32_t n_segments,
                           int32_t n_points, float *out, hipStream_t stream)
{
    if (n_segments < 0 || n_points < 0 || C <= 0) return BEVPOOL_ERR_INVALID_ARG;
    if (n_segments == 0) return BEVPOOL_OK;
    if (!table || !indices || !offsets || !out || n_rows <= 0) return BEVPOOL_ERR_INVALID_ARG;
    const int fe = elem_bytes(table_dtype);
    const bool pair_ok = (weight_dtype == BEVPOOL_F32 && table_dtype == BEVPOOL_F32) ||
                         (weight_dtype == BEVPOOL_F16 && table_dtype == BEVPOOL_F16) ||
                         (weight_dtype == BEVPOOL_F16 && table_dtype == BEVPOOL_FP8_E4M3);
    if (!pair_ok || fe == 0) return BEVPOOL_ERR_UNSUPPORTED;
    const int64_t row_bytes = int64_t(C) * fe;
    const bool e4m3_small = table_dtype == BEVPOOL_FP8_E4M3 && row_bytes <= 512;
    if (row_bytes % (e4m3_small ? 8 : 16) != 0 || row_bytes > 1024) return BEVPOOL_ERR_UNSUPPORTED;
    if (n_rows > kInt32Limit || int64_t(n_segments) * C > kInt32Limit || n_rows * C > kInt32Limit ||
        n_rows * row_bytes > kTableBytesLimit)
        return BEVPOOL_ERR_OVERFLOW;
    if (!aligned(out, 16) || !aligned(table, 16) ||
        (weights && !aligned(weights, uintptr_t(elem_bytes(weight_dtype)))))
        return BEVPOOL_ERR_INVALID_ARG;

    bevpool::FwdParams p{};
    p.depth = weights;
    p.feat = table;
    p.feat_scale = table_scale;
    p.C = C;
    p.chunks = int32_t(row_bytes / 16);
    p.ranks_feat = indices;
    p.interval_starts = offsets;
    p.n_points = n_points;
    p.n_intervals = n_segments;
    p.table_bytes = n_rows * row_bytes;
    p.out = out;
    p.out_dtype = bevpool::kF32;
    p.n_cells = n_segments;
    p.depth_dtype = weight_dtype;
    p.feat_dtype = table_dtype;
    return bevpool::run_segment_reduce(p, stream) == hipSuccess ? BEVPOOL_OK : BEVPOOL_ERR_HIP;
}

}  // extern "C"
