/*
 * bevpool.h -- C ABI of the MI355X (gfx950) BEV-pooling library.
 *
 * BEV pooling lifts multi-camera image features into a top-down grid: every
 * frustum point weights its image feature row by its depth probability and
 * the weighted rows are summed into the BEV cell the point falls in
 * ("Accelerating BEV Pooling on NVIDIA GPUs for Physical AI Applications",
 * introduction and section "Remove redundant scatter traffic"):
 *
 *     out[ranks_bev[t], c] += depth[ranks_depth[t]] * feat[ranks_feat[t], c]
 *
 * bevpool_build_map turns a per-point cell index into the five-array INT32
 * scatter map of that section (ranks_depth, ranks_feat, ranks_bev,
 * interval_starts, interval_lengths), once per geometry.  bevpool_forward runs
 * the interval-owned scatter-reduce of section "Implement the interval-owned
 * scatter-reduce": each interval of points sharing one cell has a single
 * owner that accumulates all channels and writes the cell once; no atomics,
 * no runtime index division.  bevpool_forward_ex adds fp16/bf16 output cells,
 * bevpool_segment_reduce applies the same owner kernel to a weighted
 * segmented gather-reduce (an embedding bag), and bevpool_forward_baseline
 * runs the article's two earlier loop orders for comparison.
 *
 * Conventions (all calls):
 *   - Pointers without an h_ prefix are device pointers (HBM of the current
 *     device); h_ pointers are host pointers.  The caller owns all memory;
 *     the library allocates nothing and frees nothing (the one device array
 *     it holds, the workspace of bevpool_build_map_no_alloc, is static).
 *   - Every call returns a bevpool_status; no C++ exception crosses the ABI.
 *     Arguments are validated on the host before any HIP call, so a failed
 *     validation touches neither the GPU nor any output.
 *   - Work is enqueued on `stream` (NULL = the null stream).
 *   - Sizes follow the article's INT32 map contract: point counts, cell
 *     counts times C, and feature rows times C must stay below 2^31.
 */
#ifndef BEVPOOL_H
#define BEVPOOL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bevpool_status {
    BEVPOOL_OK = 0,
    BEVPOOL_ERR_INVALID_ARG = -1,  /* null pointer, negative or zero size, misalignment, inconsistent counts */
    BEVPOOL_ERR_UNSUPPORTED = -2,  /* no kernel for this (depth dtype, feat dtype, C) */
    BEVPOOL_ERR_OVERFLOW = -3,     /* a size breaks the INT32 index contract */
    BEVPOOL_ERR_WORKSPACE = -4,    /* workspace smaller than bevpool_build_map_workspace_size() */
    BEVPOOL_ERR_CAPACITY = -5,     /* more kept points than the map arrays' capacity */
    BEVPOOL_ERR_BAD_CELL = -6,     /* point_cell holds a value outside [-1, n_cells) */
    BEVPOOL_ERR_HIP = -7           /* the HIP runtime reported an error */
} bevpool_status;

/* Element types.  FP8_E4M3 is the OCP 8-bit float E4M3 ("FN": bias 7, max
 * 448, no infinities, NaN = S.1111.111), decoded in-kernel by gfx950's
 * native conversion and multiplied by a per-tensor fp32 scale. */
typedef enum bevpool_dtype {
    BEVPOOL_F32 = 0,
    BEVPOOL_F16 = 1,
    BEVPOOL_FP8_E4M3 = 2,
    BEVPOOL_BF16 = 3   /* output type of bevpool_forward_ex only */
} bevpool_dtype;

/* Largest feature table (or segment-reduce table) in bytes, 2^32 - 4096.
 * Rows are addressed by 32-bit byte offsets from the table base; the kernels
 * keep the top 4 KB of that range for the slots of a batch that hold no
 * point, which read as zeros. */
#define BEVPOOL_MAX_TABLE_BYTES 4294963200u

/* Human-readable name of a status code (static storage; never NULL). */
const char *bevpool_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int bevpool_version(void);

/*
 * Bytes of device workspace bevpool_build_map needs for a frustum of
 * n_img*D*H*W points and n_cells cells.  Returns 0 for invalid sizes.
 */
size_t bevpool_build_map_workspace_size(int32_t n_img, int32_t D, int32_t H, int32_t W,
                                        int64_t n_cells);

/*
 * bevpool_build_map -- the five-array INT32 scatter map, prepared once per
 * geometry ahead of the forward calls (section "Implement the interval-owned
 * scatter-reduce"; the arrays are named in section "Remove redundant scatter
 * traffic").
 *
 * Input
 *   point_cell [n_img*D*H*W] int32, device: for frustum point
 *       p = ((img*D + d)*H + h)*W + w  its BEV cell in [0, n_cells), or -1
 *       when the point is dropped (outside the grid, culled).  Batched frames
 *       are folded into img and into the cell index by the caller.
 *   n_img, D, H, W: images (frames x cameras), depth bins, feature rows and
 *       columns; depth is laid out [n_img, D, H, W] and feat [n_img, H, W, C].
 *   n_cells: number of BEV cells (>= 1).
 * Output (device, capacity >= kept points each; only the first n_points /
 * n_intervals entries are written):
 *   ranks_depth[t] = p, ranks_feat[t] = img*H*W + h*W + w,
 *   ranks_bev[t] = point_cell[p] for the kept points, ordered by
 *       (cell, p) -- a total order, so the map is unique and bit-exact;
 *   interval_starts[i], interval_lengths[i]: maximal runs of equal
 *       ranks_bev, in increasing cell; every length >= 1.
 *   h_n_points, h_n_intervals (host): kept point and interval counts.  They
 *       are also reported with BEVPOOL_ERR_CAPACITY so the caller can size
 *       the arrays and call again.
 * workspace: device memory of at least bevpool_build_map_workspace_size()
 *   bytes, 256-byte aligned, caller-owned; contents on entry are ignored.
 * Blocking: returns after the map is complete (one stream synchronisation
 *   to read the two counts back).  Not for use under stream capture.
 * Errors: INVALID_ARG, OVERFLOW (n_img*D*H*W >= 2^31), WORKSPACE, CAPACITY,
 *   BAD_CELL (a cell outside [-1, n_cells); the arrays are then undefined),
 *   HIP.
 */
int bevpool_build_map(const int32_t *point_cell, int32_t n_img, int32_t D, int32_t H, int32_t W,
                      int64_t n_cells,
                      int32_t *ranks_depth, int32_t *ranks_feat, int32_t *ranks_bev,
                      int32_t *interval_starts, int32_t *interval_lengths, int64_t capacity,
                      int32_t *h_n_points, int32_t *h_n_intervals,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the static device workspace of bevpool_build_map_no_alloc: 80 MiB
 * per device, enough for frustums of up to 4,091,520 points. */
#define BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES (80u << 20)

/*
 * bevpool_build_map_no_alloc -- bevpool_build_map for callers that cannot
 * allocate device memory (harnesses that forbid hipMalloc, serving loops
 * that must not allocate): the workspace is a static device array of the
 * library (BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES on each device the library
 * runs on, held until the process ends) instead of a caller argument.  It
 * calls no allocating routine.  The caller still passes the point_cell input
 * and the five map arrays.
 *
 * Arguments, outputs, blocking behaviour and errors are those of
 * bevpool_build_map without workspace / workspace_bytes, except:
 *   BEVPOOL_ERR_WORKSPACE when bevpool_build_map_workspace_size() of the
 *       frustum exceeds BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES (checked first, on
 *       the host, before any HIP call);
 *   BEVPOOL_ERR_HIP also when the workspace's device address cannot be
 *       looked up on the current device.
 * Every call on one device uses that device's one array: calls that overlap
 * on a device (other host threads, or other streams of the same device) race
 * and must be serialised by the caller.  The array keeps the previous call's
 * contents; the build clears what it needs.
 */
int bevpool_build_map_no_alloc(const int32_t *point_cell, int32_t n_img, int32_t D, int32_t H,
                               int32_t W, int64_t n_cells,
                               int32_t *ranks_depth, int32_t *ranks_feat, int32_t *ranks_bev,
                               int32_t *interval_starts, int32_t *interval_lengths,
                               int64_t capacity, int32_t *h_n_points, int32_t *h_n_intervals,
                               hipStream_t stream);

/*
 * bevpool_forward -- the depth-weighted, interval-owned scatter-reduce
 * (section "Remove redundant scatter traffic" for the formula; section
 * "Implement the interval-owned scatter-reduce" for the owner loop):
 *
 *   out[cell, c] = sum over the points t of the interval whose cell it is of
 *                  depth[ranks_depth[t]] * feat[ranks_feat[t], c] (* feat_scale)
 *
 * accumulated in fp32 registers and written once; cells without an interval
 * are written as 0.  Every element of out is written, so out needs no
 * clearing.
 *
 *   depth [n_depth] (device): depth probabilities, read flat through
 *       ranks_depth; depth_dtype BEVPOOL_F32 or BEVPOOL_F16.
 *   feat [n_feat_rows, C] (device, 16-byte aligned): channel-last feature
 *       rows; feat_dtype BEVPOOL_F32, BEVPOOL_F16 or BEVPOOL_FP8_E4M3.
 *   feat_scale: dequantisation scale applied to FP8_E4M3 features (ignored
 *       for the other types).
 *   Supported pairs: (F32 depth, F32 feat); (F16 depth, F16 feat);
 *       (F16 depth, FP8_E4M3 feat).  Channels: C % 4 == 0 and C <= 256 for
 *       F32; C % 8 == 0 and C <= 512 for F16; for FP8_E4M3, C % 8 == 0 up to
 *       C = 512 and C % 16 == 0 up to C = 1024.  Anything else returns
 *       BEVPOOL_ERR_UNSUPPORTED.
 *   ranks_*, interval_*: a map as produced by bevpool_build_map for this
 *       geometry (n_points, n_intervals entries).  The kernel trusts the map:
 *       indices outside depth / feat / out are undefined behaviour.
 *   out [n_cells, C] fp32 (device, 16-byte aligned), overwritten.
 * Sizes: n_cells*C and n_feat_rows*C below 2^31 elements, n_depth below 2^31,
 *   and the feature table at most BEVPOOL_MAX_TABLE_BYTES (n_feat_rows*C*
 *   element bytes; this binds for F32 features, and for F16 ones only within
 *   4 KB of 2^32 bytes); else BEVPOOL_ERR_OVERFLOW.
 * Asynchronous: enqueues on `stream` and returns; never synchronises or
 * allocates, so it may be captured into a HIP graph.  One kernel launch, or
 * several in stream order for more than 2^24 intervals.
 * Errors: INVALID_ARG, UNSUPPORTED, OVERFLOW, HIP (launch failure).
 */
int bevpool_forward(const void *depth, int32_t depth_dtype, int64_t n_depth,
                    const void *feat, int32_t feat_dtype, int64_t n_feat_rows, int32_t C,
                    float feat_scale,
                    const int32_t *ranks_depth, const int32_t *ranks_feat,
                    const int32_t *ranks_bev,
                    const int32_t *interval_starts, const int32_t *interval_lengths,
                    int32_t n_points, int32_t n_intervals,
                    float *out, int64_t n_cells, hipStream_t stream);

/*
 * bevpool_forward_ex -- bevpool_forward with a choice of output type, for
 * callers whose output traffic is the larger share of a DRAM-bound call.
 * The article's FP8 path halves the output bytes as well as the feature bytes
 * (Figure 4, and the section on classifying the memory regime: when the
 * working set spills out of L2, fewer bytes is the target).
 *
 * Accumulation stays fp32 in registers; each finished fp32 sum is rounded
 * once, to nearest-even, to out_dtype at the store:
 *   out_dtype BEVPOOL_F32  -- identical to bevpool_forward;
 *   out_dtype BEVPOOL_F16  -- IEEE binary16 (sums beyond 65504 become inf);
 *   out_dtype BEVPOOL_BF16 -- bfloat16 (fp32's exponent range, 8-bit
 *                             significand).
 *   out [n_cells, C] of out_dtype (device; 16-byte aligned for F32, 8-byte
 *       aligned for F16/BF16), overwritten, empty cells 0.
 * Every other argument, the supported combinations and the behaviour are
 * those of bevpool_forward.  Errors: as bevpool_forward; UNSUPPORTED for an
 * out_dtype other than the three above.
 */
int bevpool_forward_ex(const void *depth, int32_t depth_dtype, int64_t n_depth,
                       const void *feat, int32_t feat_dtype, int64_t n_feat_rows, int32_t C,
                       float feat_scale,
                       const int32_t *ranks_depth, const int32_t *ranks_feat,
                       const int32_t *ranks_bev,
                       const int32_t *interval_starts, const int32_t *interval_lengths,
                       int32_t n_points, int32_t n_intervals,
                       void *out, int32_t out_dtype, int64_t n_cells, hipStream_t stream);

/*
 * bevpool_segment_reduce -- the interval-owned kernel applied to a generic
 * weighted segmented gather-reduce (an embedding bag with per-point weights).
 * The article names sparse embeddings and segmented reductions as the same
 * workload shape as BEV pooling (sections "Map the algorithm to hardware" and
 * "Getting started"):
 *
 *   out[s, c] = sum over t in [offsets[s], offsets[s+1]) of
 *               weights[t] * table[indices[t], c] (* table_scale for e4m3)
 *
 * with one owner per segment, fp32 accumulation and one write per output
 * element; empty segments are written as 0.  For wide rows (fp32: C a
 * multiple of 16 and at least 64; fp16 and e4m3: C a multiple of 32 and at
 * least 128, and of 64 past 512 for e4m3) a segment of over 384 points gets
 * four owners, one per quarter of the channels, each writing its quarter once.
 *
 *   weights [n_points] (device; NULL = all ones), weight_dtype as the depth
 *       dtype of bevpool_forward.
 *   table [n_rows, C] (device, 16-byte aligned), table_dtype and the
 *       supported (weight, table, C) combinations as bevpool_forward.
 *   indices [n_points] int32 rows of table; offsets [n_segments + 1] int32,
 *       non-decreasing, offsets[n_segments] <= n_points.  Row reads are
 *       bounded by the table's byte size, so no index reads memory outside
 *       the table: an index from n_rows up to 2^32 / row_bytes, or a small
 *       negative one (index * row_bytes >= -4096), reads a zero row; any
 *       other index outside [0, n_rows) reads zeros or an unspecified row.
 *       Offsets are trusted (values outside the arrays are undefined
 *       behaviour).
 *   out [n_segments, C] fp32 (device, 16-byte aligned), overwritten.
 * Sizes: n_segments*C and n_rows*C below 2^31, table at most
 * BEVPOOL_MAX_TABLE_BYTES.
 * Asynchronous, no allocation.  n_segments == 0 is a no-op.  Errors:
 * INVALID_ARG, UNSUPPORTED, OVERFLOW, HIP.
 */
int bevpool_segment_reduce(const void *weights, int32_t weight_dtype, const void *table,
                           int32_t table_dtype, int64_t n_rows, int32_t C, float table_scale,
                           const int32_t *indices, const int32_t *offsets, int32_t n_segments,
                           int32_t n_points, float *out, hipStream_t stream);

/* Loop orders of bevpool_forward_baseline. */
typedef enum bevpool_order {
    BEVPOOL_ORDER_TILE_OUTER = 0,   /* V2-style: channel tiles outside the scatter loop */
    BEVPOOL_ORDER_DEPTH_OUTER = 1   /* V2+DO-style: each interval visited once, all channels */
} bevpool_order;

/*
 * bevpool_forward_baseline -- the two earlier traversal orders the article
 * compares against (sections "How BEVPoolV3 lowers latency" and "Remove
 * redundant scatter traffic", Table 1), for measuring on the same hardware
 * what the interval-owned kernel gains.  Not a fast path.
 *
 * One thread owns one (interval, 16-byte channel tile) pair and walks the
 * interval's points, loading its indices and depth value per tile; the output
 * is zero-filled by a first kernel and each occupied cell stored once by a
 * second.  With BEVPOOL_ORDER_TILE_OUTER the tiles are the slowest-varying
 * thread index (every tile re-reads all indices); with
 * BEVPOOL_ORDER_DEPTH_OUTER the tiles of one interval are neighbouring
 * threads (each index fetched once per interval).
 *
 * Arguments, layouts and results are those of bevpool_forward (same
 * tolerance), except that a feature row must be a multiple of 16 bytes for
 * every dtype.  Asynchronous, no allocation.  Errors: as bevpool_forward, and
 * INVALID_ARG for an unknown order.
 */
int bevpool_forward_baseline(int32_t order, const void *depth, int32_t depth_dtype,
                             int64_t n_depth, const void *feat, int32_t feat_dtype,
                             int64_t n_feat_rows, int32_t C, float feat_scale,
                             const int32_t *ranks_depth, const int32_t *ranks_feat,
                             const int32_t *ranks_bev, const int32_t *interval_starts,
                             const int32_t *interval_lengths, int32_t n_points,
                             int32_t n_intervals, float *out, int64_t n_cells,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BEVPOOL_H */
