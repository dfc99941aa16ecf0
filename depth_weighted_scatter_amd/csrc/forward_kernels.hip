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
// CDNA4 mapping (our design, not the article's):
//   * A feature row is split into G chunks of 16 bytes (8 bytes for narrow
//     e4m3 rows); lane (g, k) = g*G + k loads chunk k of point slot g,
//     so one wave instruction gathers PPW = 64/G rows (C=80 fp16 or e4m3:
//     G=10, six rows per instruction).  Row loads are raw buffer loads with a
//     32-bit per-lane byte offset; a slot that holds no point reads at an
//     offset past the table, which returns zeros, with weight zero, so slots
//     are never masked one by one (the owner waves' scalar issue is the
//     contended resource, and per-slot exec-mask branches are scalar work).
//   * The map indices of up to 64 points come in with one coalesced load per
//     array; each point's depth is gathered once by the lane that read its
//     index and handed to the lanes of its slot with ds_bpermute.
//   * fp16 features feed v_fma_mix_f32; e4m3 features go through gfx950's
//     OCP-fp8 v_cvt_pk_f32_fp8; accumulation is fp32 in registers.
//   * The PPW slot accumulators of a wave are folded through LDS and the cell
//     is written with non-temporal 16-byte stores, so the output stream does
//     not evict feature rows from L2 (the article's cache-streaming stores,
//     section "Map the algorithm to hardware").
//   * Cells without points: intervals come in increasing cell order, so the
//     owner of interval i also zeroes the cells between the previous
//     interval's cell and its own.  Long empty runs are shared out so no
//     single wave writes them: the head and tail of the grid are sliced over
//     the first and last 64 owners, and aligned chunks of 256 cells that lie
//     inside a gap are zeroed by chunk checks run on the long-interval blocks.
//     Every output element is stored exactly once and no memset is needed.
//
// The kernel is not bandwidth-bound on a single frame (a 209K-point frame
// moves ~19 MB through HBM in ~6 us): its time is waves waiting on short chains
// of dependent loads, so the launch is shaped for memory-level parallelism:
//   * Short intervals (<= 96 points, ~99% of them at 209K points) get one
//     wave each, in blocks of four, with a small register budget (about 18
//     points' rows in flight per request round) so seven or eight waves fit
//     per SIMD.
//   * Long intervals (cells near the cameras, clustered in cell order) would
//     each pin one wave for many round trips.  The first n_long_blocks blocks
//     therefore own them instead: block b takes the long intervals b, b+n,
//     b+2n, ... (so a cluster spreads over many blocks), its four waves split
//     each one's points, and the partial rows are summed through LDS in wave
//     order before the single write.  These blocks are dispatched first, so
//     the long intervals overlap the short ones.
//   * Blocks go out to the eight XCDs round-robin.  When the feature table is
//     much larger than one XCD's 4 MB L2 (a batch of frames), each XCD is
//     instead given one contiguous eighth of the short intervals, so its L2
//     holds the rows of its own cells (one frame's rows, for a batch) rather
//     than every XCD streaming the whole table.  Below that size the plain
//     order is kept: contiguous eighths of one frame are unequal in work
//     (dense cells near the cameras).
//   * Segment reductions (embedding bags) can hold segments of thousands of
//     points.  With rows of 16 or more chunks, a segment over kPartMin points
//     is split by channels into four parts, worked by four blocks at once:
//     the owning long-interval block and one block from each of three
//     channel-part groups dispatched after the long-interval blocks.  Each
//     part is written once, so no cross-block combine is needed.  Waves of a
//     long segment of unsplit rows stage a few more row loads per round
//     straight into LDS (global_load_lds), so more rows are in flight without
//     registers, which are allocated per kernel and would cost the short role
//     its occupancy.
//   * One launch holds at most kMaxShortBlocks short-role blocks (its grid of
//     work-items must stay below 2^32); more intervals take further launches
//     of short-role blocks only.
#include <hip/hip_runtime.h>

#include "bevpool.h"
#include "bevpool_internal.h"

namespace bevpool {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kShortMax = 96;   // longest interval a single wave owns
constexpr int kRoundPoints = 18; // points per row-request round of a wave
constexpr int kLongScan = 16;    // intervals scanned per long-interval block
constexpr int kPartScan = 256;   // segments scanned per channel-part block
constexpr int kPartMin = 384;    // segments longer than this are split by channels
// short-role blocks per launch at most (a multiple of 8); more intervals take
// further launches of short-role blocks only, which keeps every grid's
// work-item count below 2^32
constexpr int kMaxShortBlocks = 1 << 22;
constexpr int64_t kContiguousTableBytes = int64_t(8) << 20;   // two XCD L2s

// A lane's share of a feature row: CB bytes (16, or 8 for e4m3 rows under
// 256 bytes -- 128 for segments -- which keeps them on the same row geometry
// as fp16 rows of the same channel count; dispatch() picks it).
template <int CB> struct ChunkVec;
template <> struct ChunkVec<16> { using type = u32x4; };
template <> struct ChunkVec<8> { using type = u32x2; };
constexpr int elem_bytes(int ft) { return ft == kF32 ? 4 : ft == kF16 ? 2 : 1; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }
// Row loads a wave stages in LDS per round when it works a long segment of
// unsplit rows: enough for about kStagePoints points per round with the SUB
// register-held loads, at most kMaxStaged (3 KB of LDS per wave).
constexpr int kStagePoints = 48;
constexpr int kMaxStaged = 3;
constexpr int staged_loads(int ppw, int sub)
{
    return cmin(kMaxStaged, (kStagePoints + ppw - 1) / ppw - sub > 0 ? (kStagePoints + ppw - 1) / ppw - sub : 0);
}

// Depth values are gathered in their storage type and widened at first use.
template <int DT> struct DepthT;
template <> struct DepthT<kF32> { using type = float; };
template <> struct DepthT<kF16> { using type = _Float16; };

// acc[e] += d * value(e) for the elements of one chunk.
template <int FT, int CB> struct Accum;
template <> struct Accum<kF32, 16> {
    __device__ static inline void run(float *acc, float d, u32x4 v)
    {
        const f32x4 f = __builtin_bit_cast(f32x4, v);   // whole-vector cast
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(d, f[e], acc[e]);
    }
};
template <> struct Accum<kF16, 16> {
    __device__ static inline void run(float *acc, float d, u32x4 v)
    {
        const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(d, static_cast<float>(h[e]), acc[e]);
    }
};
template <int CB> struct Accum<kE4M3, CB> {
    template <class V> __device__ static inline void run(float *acc, float d, V v)
    {
#pragma unroll
        for (int w = 0; w < CB / 4; ++w) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[w]), false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[w]), true);
            acc[4 * w + 0] = __builtin_fmaf(d, lo[0], acc[4 * w + 0]);
            acc[4 * w + 1] = __builtin_fmaf(d, lo[1], acc[4 * w + 1]);
            acc[4 * w + 2] = __builtin_fmaf(d, hi[0], acc[4 * w + 2]);
            acc[4 * w + 3] = __builtin_fmaf(d, hi[1], acc[4 * w + 3]);
        }
    }
};

// Stores output elements 4q .. 4q+3 (a float4 of the row-major [cells, C]
// output) in the output type, non-temporally.  The 16-bit conversions round
// to nearest-even (gfx950 converts fp32 pairs to bf16 natively).
__device__ inline void store4(void *out, int out_dtype, int q, f32x4 v)
{
    if (out_dtype == kF32) {
        __builtin_nontemporal_store(v, static_cast<f32x4 *>(out) + q);
        return;
    }
    u32x2 w;
    if (out_dtype == kF16) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        w[0] = __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1])});
        w[1] = __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])});
    } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        w[0] = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])});
        w[1] = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])});
    }
    __builtin_nontemporal_store(w, static_cast<u32x2 *>(out) + q);
}

// Zeroes cells [cell_lo, cell_hi) of out with non-temporal stores; `lane`
// and `lanes` give this thread's position among the cooperating threads.
__device__ inline void zero_cells(void *out, int out_dtype, int C, int cell_lo, int cell_hi,
                                  int lane, int lanes)
{
    if (cell_hi <= cell_lo) return;
    const int q0 = cell_lo * (C / 4), q1 = cell_hi * (C / 4);
    if (out_dtype == kF32) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int q = q0 + lane; q < q1; q += lanes)
            __builtin_nontemporal_store(z, static_cast<f32x4 *>(out) + q);
    } else {
        const u32x2 z = {0u, 0u};
        for (int q = q0 + lane; q < q1; q += lanes)
            __builtin_nontemporal_store(z, static_cast<u32x2 *>(out) + q);
    }
}

// The empty cells before the first interval's cell (the head) and after the
// last one's (the tail) can be long runs -- a grid wider than the sensing
// range, or a region no camera sees.  They are cut into up to 64 slices of at
// least kSliceCells cells: slice s of the head is zeroed by the owner of
// interval s, slice s of the tail by the owner of interval I - 1 - s.  Both
// ends are known from ranks_bev[0] and ranks_bev[N - 1], so no owner waits on
// another.  The gaps between intervals are zeroed by the owner of the
// interval that follows them.
constexpr int kSliceCells = 64;

struct Slice { int lo, hi; };

// Slice s of the cells [lo, hi) shared by `owners` owners.
__device__ inline Slice end_slice(int lo, int hi, int s, int owners)
{
    const int size = hi - lo;
    const int k = max(1, min(min(kWave, owners), (size + kSliceCells - 1) / kSliceCells));
    if (s >= k || size <= 0) return {0, 0};
    const int len = (size + k - 1) / k;
    return {min(hi, lo + s * len), min(hi, lo + (s + 1) * len)};
}

// This owner's slices of the head and tail.
__device__ inline void zero_end_slices(const FwdParams &p, int od, int C, int iv, int lane,
                                       int lanes)
{
    if (iv < kWave) {
        const Slice h = end_slice(0, p.ranks_bev[0], iv, p.n_intervals);
        zero_cells(p.out, od, C, h.lo, h.hi, lane, lanes);
    }
    const int s_tail = p.n_intervals - 1 - iv;
    if (s_tail < kWave) {
        const Slice t = end_slice(p.ranks_bev[p.n_points - 1] + 1, p.n_cells, s_tail, p.n_intervals);
        zero_cells(p.out, od, C, t.lo, t.hi, lane, lanes);
    }
}

// Empty cells between two intervals (an interior gap) are zeroed by the owner
// of the interval that follows the gap, except for the aligned chunks of
// kChunkCells cells that lie wholly inside the gap: the long-interval blocks,
// after their own intervals, check every chunk (zero_chunk_if_empty) and
// zero the empty ones, so a long interior gap is spread over many waves and
// an owner zeroes at most two partial chunks.
constexpr int kChunkCells = 256;

__device__ inline void zero_interior_gap(const FwdParams &p, int od, int C, int lo, int hi,
                                         int lane, int lanes)
{
    if (hi - lo >= kChunkCells) {          // may hold whole chunks: those are the workers'
        const int kf = (lo + kChunkCells - 1) / kChunkCells, kl = hi / kChunkCells;
        if (kf < kl) {
            zero_cells(p.out, od, C, lo, kf * kChunkCells, lane, lanes);
            lo = kl * kChunkCells;
        }
    }
    zero_cells(p.out, od, C, lo, hi, lane, lanes);
}

// Chunk check: zeroes cells [c0, c0 + kChunkCells) if no point falls in
// them and they lie between the first and the last occupied cell.  The first
// point whose cell is >= c0 is found by a 64-way search over ranks_bev, which
// is sorted by cell.
__device__ inline void zero_chunk_if_empty(const FwdParams &p, int od, int C, int chunk, int lane)
{
    const int c0 = chunk * kChunkCells, c1 = min(p.n_cells, c0 + kChunkCells);
    const int N = p.n_points;
    const int first = p.ranks_bev[0], last = p.ranks_bev[N - 1];
    if (c1 <= first || c0 > last) return;          // head or tail: sliced elsewhere
    // the first t with ranks_bev[t] >= c0 lies in [lo, hi]; hv = ranks_bev[hi]
    // (INT32_MAX while hi = N, i.e. no such point yet)
    int lo = 0, hi = N, hv = INT32_MAX;
    while (lo < hi) {
        const int step = (hi - lo + kWave - 1) / kWave;
        const int t = lo + lane * step;
        const bool valid = t < hi;
        const int v = valid ? p.ranks_bev[t] : INT32_MAX;   // probes past hi count as >= c0
        const uint64_t ge = __ballot(v >= c0);
        const int j = ge ? __builtin_ctzll(ge) : kWave;
        // the answer is in (t_(j-1), min(t_j, hi)], with t_(-1) = lo - 1
        const int new_lo = j == 0 ? lo : lo + (j - 1) * step + 1;
        if (j < kWave && lo + j * step < hi) {
            hi = lo + j * step;
            hv = __builtin_amdgcn_readlane(v, j);
        }
        lo = new_lo;
    }
    if (hv >= c1) zero_cells(p.out, od, C, c0, c1, lane, kWave);   // no point in [c0, c1)
}

// Lane i reads the map indices of point t0 + min(i, n - 1), 1 <= n <= 64:
// lanes past the batch repeat its last point, so the index and depth loads
// stay in bounds without an exec-masked branch.
// In segment mode (SEG) the weight of point t is read directly at t.
// These are ordinary (cached) loads: the map is reused by every call for the
// same geometry, and streaming loads that keep it out of the caches measured
// 3-21% slower (the larger figure on the 1.6M-point batched workload).
template <bool SEG>
__device__ inline void load_indices(const FwdParams &p, int t0, int n, int lane, int &row,
                                    int &didx)
{
    const int t = t0 + min(lane, n - 1);
    row = p.ranks_feat[t];
    didx = SEG ? t : p.ranks_depth[t];
}

// Channel parts a long segment of a segment reduction is split into: 4 for
// rows of 16 or more chunks (a multiple of 4), else 1 (whole rows; also when
// the chunk count is known only at run time).  Rows of 16 chunks take four
// points per load instruction whole and sixteen per part; rows of 8 chunks
// measured slower split in two or four.  BEV pooling keeps whole rows: with
// its few, moderately long intervals the extra blocks cost more than they save.
template <bool SEG>
__host__ __device__ constexpr int channel_parts(int g)
{
    return SEG && g >= 16 && g % 4 == 0 ? 4 : 1;
}

// Blocks in each channel-part group after the first.
__host__ __device__ inline int part_blocks(int n_intervals)
{
    return max(1, (n_intervals + kPartScan - 1) / kPartScan);
}

// Lane geometry of a wave: lane (g, k) = g*G + k holds chunk k of slot g.
struct Slots {
    int G, PPW, g, k, lane;
    bool ok;     // g < PPW (the last 64 mod G lanes idle)
    int row_G;   // chunks per feature row (G unless one channel part is worked)
    int coff;    // first chunk of the part worked (0 for whole rows)
};

typedef __attribute__((address_space(3))) char lds_char;

// Byte offset a slot without a point reads its row at: past every table the
// C ABI accepts (and at most 1 KB + 16 below 2^32 with a lane's chunk added),
// so the raw buffer load there is out of range and returns zeros.
constexpr uint32_t kEmptySlotOffset = BEVPOOL_MAX_TABLE_BYTES;

// Word 3 of a raw buffer descriptor on gfx9-family chips: 32-bit data format
// (untyped buffer loads need a valid one), no swizzle, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;

template <int CB>
__device__ inline typename ChunkVec<CB>::type load_chunk(__amdgpu_buffer_rsrc_t rows, uint32_t off)
{
    if constexpr (CB == 16)
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rows, int(off), 0, 0));
    else
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rows, int(off), 0, 0));
}

// Accumulates points [t0, t0 + n) (n >= 1) into this lane's acc, in batches
// of at most 64 points.  For each batch the loads go out in this order, and
// accumulation waits for all of them:
//   BEV:      depth values, feature rows, the indices of the next batch
//             (depth first measured 0.5-1 % faster than after the rows);
//   segments: feature rows, weights, the indices of the next batch (weights
//             first, or fetched with the indices, measured up to 30 % slower
//             on some segment mixes).
// Rows of a batch are requested SUB register-held loads plus LST loads
// staged in LDS at `stage` ((SUB + LST) * PPW points) per round.
//
// With PPWC (points per wave) known at compile time and rounds of at most 64
// points (ZERO), a batch is a whole number of rounds, so a slot's point index
// never wraps past lane 63, and the slots without a point read a zero row
// (kEmptySlotOffset) with weight zero: every lane accumulates without a
// branch, exactly (0 * 0 adds +0 whatever the table holds).  Staged loads
// past the table write zeros to LDS the same way.  Every slot group of a
// round is then requested and accumulated unguarded, the last round's empty
// groups included: with a wave-uniform test per group the compiler could
// not pair each load with its accumulation across the round loop, and at
// four or more groups per round it waited for each load before issuing the
// next (one round trip per group); without the tests the kernels also lose
// about 90 scalar instructions (3-5 % on the 209K-point frames, up to 8 % on
// embedding bags).  Otherwise (PPWC == 0: G
// known at run time; rounds over 64 points; staged rounds under 48 points,
// which measured faster in 64-point batches than in whole rounds) the lanes
// past the batch repeat its last point and empty slots are skipped by exec
// mask.  Only wave-uniform guards branch in either case.
template <int DT, int FT, int CB, int SUB, bool SEG, int PPWC, int LST = 0>
__device__ inline void accumulate_points(const FwdParams &p, int t0, int n, const Slots &s,
                                         float *acc, lds_char *stage = nullptr)
{
    constexpr int ROUND = (SUB + LST) * (PPWC > 0 ? PPWC : kWave);
    constexpr bool ZERO = PPWC > 0 && ROUND <= kWave && (LST == 0 || ROUND >= 48);
    // Staged rounds of 48 or more points take batches of one round, so no
    // round trip is spent on a batch's short remainder.
    constexpr int BATCH = ZERO ? kWave / ROUND * ROUND
                               : LST > 0 && ROUND >= 48 && ROUND <= kWave ? ROUND : kWave;
    using V = typename ChunkVec<CB>::type;
    using DRaw = typename DepthT<DT>::type;
    const DRaw *depth = static_cast<const DRaw *>(p.depth);
    const char *feat = static_cast<const char *>(p.feat);
    // Range of the raw buffer: segment indices come from the caller, so their
    // rows are bounded by the real table size (an index past the table reads
    // zeros rather than memory beyond it).  BEV maps come from
    // bevpool_build_map; their kernels keep the constant bound, which the
    // compiler folds (the table size as a kernel argument made it re-issue a
    // descriptor word before every row load: six scalar instructions per wave).
    const __amdgpu_buffer_rsrc_t rows_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(feat), 0, SEG ? int(uint32_t(p.table_bytes)) : int(kEmptySlotOffset),
        kRawBufferWord3);
    int row0, didx0;
    load_indices<SEG>(p, t0, min(BATCH, n), s.lane, row0, didx0);
    if constexpr (ZERO) {
        if (LST == 0 && n <= ROUND) {                 // (staged rounds take the loop)
            // One batch of one round (most short intervals: 80 % have 13-18
            // points at C=80): every slot group is requested unguarded (the
            // empty ones read zeros) and no next batch exists, so the round
            // carries no scalar bookkeeping.
            const bool live = s.lane < n;
            const int my_row = int(live ? uint32_t(row0 * s.row_G + s.coff) * uint32_t(CB)
                                        : kEmptySlotOffset);
            DRaw draw = SEG ? DRaw(0) : depth[didx0];
            V v[SUB];
#pragma unroll
            for (int u = 0; u < SUB; ++u)
                v[u] = load_chunk<CB>(rows_rsrc, uint32_t(__shfl(my_row, (u * s.PPW + s.g) & (kWave - 1))) +
                                                     uint32_t(s.k * CB));
            if (SEG) draw = depth ? depth[didx0] : DRaw(1);
            const float my_d = live ? static_cast<float>(draw) : 0.f;
#pragma unroll
            for (int u = 0; u < SUB; ++u)
                Accum<FT, CB>::run(acc, __shfl(my_d, (u * s.PPW + s.g) & (kWave - 1)), v[u]);
            return;
        }
    }
    for (int base = 0; base < n; base += BATCH) {
        const int nb = min(BATCH, n - base);
        const bool more = base + BATCH < n;                // wave-uniform
        const bool live = s.lane < nb;                     // this lane's point is in the batch
        // ZERO: byte offset of the lane's row (its part's first chunk);
        // else the index of that chunk
        const int my_row = ZERO ? int(live ? uint32_t(row0 * s.row_G + s.coff) * uint32_t(CB)
                                           : kEmptySlotOffset)
                                : row0 * s.row_G + s.coff;
        DRaw draw = SEG ? DRaw(0) : depth[didx0];
        int row1 = 0, didx1 = 0;
        for (int s0 = 0; s0 < nb; s0 += (SUB + LST) * s.PPW) {
            int rows[SUB + LST];
#pragma unroll
            for (int u = 0; u < SUB + LST; ++u)
                rows[u] = __shfl(my_row, (s0 + u * s.PPW + s.g) & (kWave - 1));
            V v[SUB];
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                if (ZERO || s0 + u * s.PPW < nb) {
                    if constexpr (ZERO)
                        v[u] = load_chunk<CB>(rows_rsrc, uint32_t(rows[u]) + uint32_t(s.k * CB));
                    else if constexpr (SEG)
                        v[u] = load_chunk<CB>(rows_rsrc, uint32_t(rows[u] + s.k) * uint32_t(CB));
                    else
                        v[u] = *reinterpret_cast<const V *>(feat + uint32_t(rows[u] + s.k) * uint32_t(CB));
                }
            }
            // further rows of the round go straight to LDS: lane i's 16 bytes
            // of staged instruction j at stage + 1024 j + 16 i
#pragma unroll
            for (int u = SUB; u < SUB + LST; ++u) {
                if (ZERO || s0 + u * s.PPW < nb) {
                    if constexpr (ZERO)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rows_rsrc, (__attribute__((address_space(3))) void *)(stage + (u - SUB) * 1024), 16,
                            uint32_t(rows[u]) + uint32_t(s.k * CB), 0, 0, 0);
                    else   // (staged loads are segment mode only)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rows_rsrc, (__attribute__((address_space(3))) void *)(stage + (u - SUB) * 1024), 16,
                            uint32_t(rows[u] + s.k) * uint32_t(CB), 0, 0, 0);
                }
            }
            if (s0 == 0) {
                const bool weighted = !SEG || depth;              // segments may be unweighted
                if (SEG) draw = weighted ? depth[didx0] : DRaw(1);
                if (more)
                    load_indices<SEG>(p, t0 + base + BATCH, min(BATCH, n - base - BATCH), s.lane,
                                      row1, didx1);
                // Without this pin the compiler may convert the weight right
                // after its load, so the wait for it holds back the loads
                // issued after it: for segments the next batch's indices
                // until this batch's rows are in (13-20 % on long segments);
                // for BEV depth, requested first, the rows themselves (+22 %
                // on the headline frame in a build with 24-point rounds).
                // e4m3 BEV rows measured 3 % faster without it.
                if ((SEG && weighted) || (!SEG && FT != kE4M3)) asm volatile("" : "+v"(draw));
            }
            const float my_d = ZERO && !live ? 0.f : static_cast<float>(draw);
            float ds[SUB + LST];
#pragma unroll
            for (int u = 0; u < SUB + LST; ++u) ds[u] = __shfl(my_d, (s0 + u * s.PPW + s.g) & (kWave - 1));
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                if (ZERO || s0 + u * s.PPW < nb) {
                    if (ZERO || (s.ok && s0 + u * s.PPW + s.g < nb)) Accum<FT, CB>::run(acc, ds[u], v[u]);
                }
                // e4m3: decode one slot group at a time.  Unguarded, the
                // compiler decoded all groups of a round first (64 live fp32
                // values for four 16-byte groups): 113 VGPRs at C=256 against
                // 77, four waves per SIMD instead of six, +11 % on that frame.
                // (In the one-round path the same barrier measured 2 % slower.)
                if constexpr (FT == kE4M3) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = SUB; u < SUB + LST; ++u) {
                if (ZERO || s0 + u * s.PPW < nb) {
                    typedef __attribute__((address_space(3))) const V lds_v;
                    const V x = *reinterpret_cast<lds_v *>(stage + (u - SUB) * 1024 + s.lane * 16);
                    if (ZERO || (s.ok && s0 + u * s.PPW + s.g < nb)) Accum<FT, CB>::run(acc, ds[u], x);
                }
            }
        }
        row0 = row1;
        didx0 = didx1;
    }
}

// Folds the PPW slot accumulators of a wave through its LDS scratch r (64*E
// floats) and hands float4 q of the C-float row sum to emit(q, sum) on lane q
// (mod 64).  Every lane writes its E sums unmasked: the idle lanes (g == PPW,
// k < 64 - PPW*G) land in [PPW*C, 64*E), which the fold does not read.
template <int E, class Emit>
__device__ inline void fold_slots(float *r, const float *acc, const Slots &s, int C, Emit emit)
{
#pragma unroll
    for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4 *>(r + s.g * C + s.k * E + e) =
            f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_assume(s.lane >= 0 && s.lane < kWave);   // one pass while C <= 256
    for (int q = s.lane; q < C / 4; q += kWave) {
        f32x4 sum = *reinterpret_cast<const f32x4 *>(r + 4 * q);
        for (int gg = 1; gg < s.PPW; ++gg) sum += *reinterpret_cast<const f32x4 *>(r + gg * C + 4 * q);
        emit(q, sum);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// CB: bytes per lane chunk.  G_CT > 0: lanes per point (chunks per row)
// fixed at compile time; G_CT < 0: p.chunks lanes per point and -G_CT points
// per wave (the rows of other widths keep the compile-time wave geometry:
// unrolled rounds, zero-row padding, the one-round path); G_CT == 0: both
// from p.chunks.  OD: the output type, fixed at
// compile time so the stores and zero fills carry no type branches (they
// measured 1-2 % of the call in scalar instructions).
//
// SEG: segment mode (bevpool_segment_reduce): interval i is segment i, with
// start offsets[i] (interval_starts) and length offsets[i+1] - offsets[i]
// (possibly 0), cell i, and the weight of point t read at t (or 1).
template <int DT, int FT, int CB, int G_CT, bool SEG, int OD>
__global__ __launch_bounds__(kBlock) void bev_pool_fwd(FwdParams p)
{
    constexpr int E = CB / elem_bytes(FT);   // row elements per lane
    constexpr int PPW_CT = G_CT > 0 ? kWave / G_CT : G_CT < 0 ? -G_CT : 1;
    constexpr int PPW_RT = G_CT != 0 ? PPW_CT : 0;   // 0: known at run time only
    // rows in flight per lane: about kRoundPoints points per request round,
    // which keeps the common kernels near 64 VGPRs (up to eight waves per SIMD);
    // rows of 16 or more chunks (at most four points per instruction) take
    // four instructions per round, which measured faster than more rows in
    // flight at half the occupancy (C = 128 and 256)
    constexpr int SUB_RAW = G_CT != 0 ? (kRoundPoints + PPW_CT - 1) / PPW_CT : 4;
    constexpr bool WIDE = G_CT >= 16 || (G_CT < 0 && PPW_CT <= 4);   // 13 or more chunks
    constexpr int SUB = WIDE ? (SUB_RAW > 4 ? 4 : SUB_RAW)
                                   : SUB_RAW > 8 ? 8 : (SUB_RAW > 5 && E == 16 ? 5 : SUB_RAW);
    // A channel part of a long segment (segment reductions, rows split by
    // channels) mostly misses L2 (tables larger than it), so its waves request
    // about 64 rows per round (at most 8 instructions) instead of
    // kRoundPoints.  Whole rows keep SUB: registers are allocated per kernel,
    // and more rows in flight there cost the short role its occupancy.
    constexpr int KP = channel_parts<SEG>(G_CT);
    constexpr int PPW_PART = G_CT > 0 ? kWave / (G_CT / KP) : 1;
    constexpr int SUB_LP = !SEG || G_CT <= 0 ? SUB : cmin(8, (kWave + PPW_PART - 1) / PPW_PART);
    constexpr int PPW_PART_RT = G_CT > 0 ? PPW_PART : 0;
    // Long segments of unsplit rows: their waves also stage LST row loads per
    // round in LDS (the wave's fold buffer, free while it accumulates), which
    // adds rows in flight without the registers that would cost the short
    // role its occupancy.
    constexpr int LST = SEG && KP == 1 && CB == 16 && G_CT > 0 ? staged_loads(PPW_CT, SUB) : 0;
    constexpr int RED = kWave * E > LST * 256 ? kWave * E : LST * 256;   // floats per wave
    __shared__ __attribute__((aligned(16))) float red[kWavesPerBlock][RED];
    extern __shared__ __attribute__((aligned(16))) float part[];   // [kWavesPerBlock][C]

    // with a compile-time chunk count the channel count is compile-time too
    const int C = G_CT > 0 ? G_CT * E : p.C, C4 = C / 4;
    const int lane = __lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    Slots s;
    s.G = G_CT > 0 ? G_CT : p.chunks;
    s.PPW = G_CT != 0 ? PPW_CT : kWave / s.G;
    s.g = lane / s.G;
    s.k = lane - s.g * s.G;
    s.lane = lane;
    s.ok = s.g < s.PPW;
    s.row_G = s.G;
    s.coff = 0;
    const float scale = FT == kE4M3 ? p.feat_scale : 1.f;
    constexpr int od = OD;
    float acc[E];

    const int first_short = p.first_short;
    if (int(blockIdx.x) >= first_short) {
        // ---- short-interval role: one wave, one interval ----
        // Logical block j of this role runs on XCD (j + first_short) mod 8
        // (short_base is a multiple of 8); with xcd_run > 1 XCD x takes the
        // logical blocks [x * run, (x + 1) * run).
        const int j = int(blockIdx.x) - first_short + p.short_base;
        const int lj = p.xcd_run == 1 ? j : ((j + first_short) % 8) * p.xcd_run + j / 8;
        const int iv = lj * kWavesPerBlock + wv;
        if (iv >= p.n_intervals) return;
        const int start = p.interval_starts[iv];
        const int len = SEG ? p.interval_starts[iv + 1] - start : p.interval_lengths[iv];
        // Both header words are wave-uniform (scalar loads); without this the
        // compiler sinks the start load below the length test, so a wave
        // would wait for two scalar round trips instead of one.
        asm volatile("" ::"s"(start), "s"(len));
        if (len > kShortMax) {                              // owned by a long-interval block
            if (!SEG) zero_end_slices(p, od, C, iv, lane, kWave);
            return;
        }
        // lane 0: the cell before this interval, other lanes: its own cell
        const int cells = SEG ? iv - 1 + min(lane, 1) : p.ranks_bev[max(start - 1 + min(lane, 1), 0)];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        if (!SEG || len > 0) accumulate_points<DT, FT, CB, SUB, SEG, PPW_RT>(p, start, len, s, acc);
        const int bev = __builtin_amdgcn_readlane(cells, 1);
        fold_slots<E>(red[wv], acc, s, C, [&](int q, f32x4 sum) {
            if (FT == kE4M3) sum *= scale;
            store4(p.out, od, bev * C4 + q, sum);
        });
        if (!SEG) {
            if (iv > 0) zero_interior_gap(p, od, C, __builtin_amdgcn_readlane(cells, 0) + 1, bev, lane, kWave);
            zero_end_slices(p, od, C, iv, lane, kWave);
        }
        return;
    }

    // ---- long-interval role ----
    // Group 0 (the first n_long_blocks blocks): block b owns the long
    // intervals b, b + n_long_blocks, ...  With KP > 1 a segment over kPartMin
    // points is split by channels into KP parts: group 0 works part 0, and
    // group j (n_part blocks each, after group 0) works part j, its block b
    // taking the segments b, b + n_part, ...  Every part is written once.
    const int n_part = KP > 1 ? part_blocks(p.n_intervals) : 0;
    const int grp = KP == 1 || int(blockIdx.x) < p.n_long_blocks
                        ? 0 : 1 + (int(blockIdx.x) - p.n_long_blocks) / n_part;
    const int nl = grp == 0 ? p.n_long_blocks : n_part;
    const int b0 = grp == 0 ? int(blockIdx.x) : (int(blockIdx.x) - p.n_long_blocks) % n_part;
    const int min_len = grp == 0 ? kShortMax : kPartMin;
    Slots sp = s;                                           // lane geometry of one part
    if (KP > 1) {
        sp.G = s.G / KP;
        sp.PPW = kWave / sp.G;
        sp.g = lane / sp.G;
        sp.k = lane - sp.g * sp.G;
        sp.ok = sp.g < sp.PPW;
        sp.coff = grp * sp.G;
    }
    const int Cp = C / KP, Cp4 = Cp / 4;
    for (int base = b0; base < p.n_intervals; base += nl * kWave) {
        const int cand = base + lane * nl;
        int cand_len = 0;
        if (cand < p.n_intervals)
            cand_len = SEG ? p.interval_starts[cand + 1] - p.interval_starts[cand]
                           : p.interval_lengths[cand];
        uint64_t todo = __ballot(cand_len > min_len);      // same in every wave of the block
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int iv = base + j * nl;
            const int len = __builtin_amdgcn_readlane(cand_len, j);
            const bool split = KP > 1 && len > kPartMin;
            const Slots &ss = split ? sp : s;
            const int Cw = split ? Cp : C, Cw4 = split ? Cp4 : C4;
            const int c4off = split ? grp * Cp4 : 0;
            const int start = p.interval_starts[iv];
            // the four waves take consecutive quarters of the points
            const int quarter = (len + kWavesPerBlock - 1) / kWavesPerBlock;
            const int lo = min(len, wv * quarter), hi = min(len, lo + quarter);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = 0.f;
            if (lo < hi) {
                if constexpr (LST > 0) {
                    accumulate_points<DT, FT, CB, SUB, SEG, PPW_RT, LST>(
                        p, start + lo, hi - lo, s, acc,
                        (lds_char *)(__attribute__((address_space(3))) void *)red[wv]);
                } else if (split) {
                    accumulate_points<DT, FT, CB, SUB_LP, SEG, PPW_PART_RT>(p, start + lo, hi - lo, sp, acc);
                } else {
                    accumulate_points<DT, FT, CB, SUB, SEG, PPW_RT>(p, start + lo, hi - lo, s, acc);
                }
            }
            fold_slots<E>(red[wv], acc, ss, Cw, [&](int q, f32x4 sum) {
                *reinterpret_cast<f32x4 *>(part + wv * Cw + 4 * q) = sum;
            });
            __syncthreads();
            const int bev = SEG ? iv : p.ranks_bev[start];
            const int prev_bev = SEG ? iv - 1 : (iv > 0 ? p.ranks_bev[start - 1] : -1);
            for (int q = threadIdx.x; q < Cw4; q += kBlock) {
                f32x4 sum = *reinterpret_cast<const f32x4 *>(part + 4 * q);
#pragma unroll
                for (int w = 1; w < kWavesPerBlock; ++w)
                    sum += *reinterpret_cast<const f32x4 *>(part + w * Cw + 4 * q);
                if (FT == kE4M3) sum *= scale;
                store4(p.out, od, bev * C4 + c4off + q, sum);
            }
            if (!SEG && iv > 0) zero_interior_gap(p, od, C, prev_bev + 1, bev, threadIdx.x, kBlock);
            __syncthreads();                                // part is reused
        }
    }
    // then each wave checks its share of the cell chunks for interior gaps
    if (!SEG) {
        const int n_chunks = (p.n_cells + kChunkCells - 1) / kChunkCells;
        for (int c = blockIdx.x * kWavesPerBlock + wv; c < n_chunks; c += nl * kWavesPerBlock)
            zero_chunk_if_empty(p, od, C, c, lane);
    }
}

// Zero output for a map with no intervals: a pure write stream, so plain
// stores (they measured faster than non-temporal ones for bulk writes), four
// per thread, one thread per four groups of four elements.
constexpr int kFillPer = 4;

template <class T>
__global__ __launch_bounds__(kBlock) void zero_fill(T *out, int n4)
{
    const int i0 = blockIdx.x * (kBlock * kFillPer) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kFillPer; ++u) {
        const int i = i0 + u * kBlock;
        if (i < n4) out[i] = T{};
    }
}

// The launches of one call: the first holds the long-interval blocks, the
// channel-part groups (segment reductions with rows split into parts) and up
// to kMaxShortBlocks short-role blocks; any further ones hold short-role
// blocks only.
template <int DT, int FT, int CB, int G, bool SEG, int OD>
void launch_g(FwdParams p, int n_short, size_t lds, hipStream_t s)
{
    constexpr int kp = channel_parts<SEG>(G);
    const int role_blocks = p.n_long_blocks + (kp > 1 ? (kp - 1) * part_blocks(p.n_intervals) : 0);
    for (int base = 0; base < n_short; base += kMaxShortBlocks) {
        p.first_short = base == 0 ? role_blocks : 0;
        p.short_base = base;
        const int blocks = p.first_short + min(kMaxShortBlocks, n_short - base);
        bev_pool_fwd<DT, FT, CB, G, SEG, OD><<<blocks, kBlock, lds, s>>>(p);
    }
}

// Chunk counts with a kernel of their own (others take the run-time-G one,
// which measured 23-25 % slower at C=48, 96 and 192 fp16 before 6, 12 and 24
// got theirs).  e4m3 rows only arrive in 8-byte chunks up to 248 bytes and in
// 16-byte chunks from 128 bytes (segments) or 256 bytes (BEV); see dispatch().
template <int FT, int CB, bool SEG>
constexpr bool compiled_g(int g)
{
    return FT != kE4M3 || (CB == 8 ? g < 32 : g >= (SEG ? 8 : 16));
}

// Rows whose chunk count has no kernel of its own: the kernel for their
// points per wave (64 / chunks: 1, 2, 3, 4, 5, 7, 9 or 21 for the counts
// that reach here).  A run-time wave geometry measured 23-25 % slower.
template <int DT, int FT, int CB, bool SEG, int OD>
void launch_ppw(FwdParams p, int n_short, size_t lds, hipStream_t s)
{
    switch (kWave / p.chunks) {
    case 1: launch_g<DT, FT, CB, -1, SEG, OD>(p, n_short, lds, s); break;
    case 2: launch_g<DT, FT, CB, -2, SEG, OD>(p, n_short, lds, s); break;
    case 3: launch_g<DT, FT, CB, -3, SEG, OD>(p, n_short, lds, s); break;
    case 4: launch_g<DT, FT, CB, -4, SEG, OD>(p, n_short, lds, s); break;
    case 5: launch_g<DT, FT, CB, -5, SEG, OD>(p, n_short, lds, s); break;
    case 7: launch_g<DT, FT, CB, -7, SEG, OD>(p, n_short, lds, s); break;
    case 9: launch_g<DT, FT, CB, -9, SEG, OD>(p, n_short, lds, s); break;
    case 21: launch_g<DT, FT, CB, -21, SEG, OD>(p, n_short, lds, s); break;
    default: launch_g<DT, FT, CB, 0, SEG, OD>(p, n_short, lds, s); break;
    }
}

template <int DT, int FT, int CB, bool SEG, int OD>
hipError_t launch_typed(FwdParams p, hipStream_t s)
{
    // long-interval blocks: about kLongScan intervals scanned per block
    p.n_long_blocks = min(2048, max(1, (p.n_intervals + kLongScan - 1) / kLongScan));
    // short-role blocks: contiguous eighths per XCD for BEV tables over 8 MB
    // (segment rows follow no cell order, so segments keep the plain order)
    const int short_blocks = (p.n_intervals + kWavesPerBlock - 1) / kWavesPerBlock;
    p.xcd_run = !SEG && p.table_bytes > kContiguousTableBytes ? (short_blocks + 7) / 8 : 1;
    const int n_short = p.xcd_run == 1 ? short_blocks : 8 * p.xcd_run;
    const size_t lds = size_t(kWavesPerBlock) * p.C * sizeof(float);
#define BEVPOOL_CASE(GV)                                                              \
    case GV:                                                                          \
        if constexpr (compiled_g<FT, CB, SEG>(GV)) launch_g<DT, FT, CB, GV, SEG, OD>(p, n_short, lds, s); \
        else launch_ppw<DT, FT, CB, SEG, OD>(p, n_short, lds, s);                     \
        break;
    switch (p.chunks) {
        BEVPOOL_CASE(1) BEVPOOL_CASE(2) BEVPOOL_CASE(4) BEVPOOL_CASE(5) BEVPOOL_CASE(8)
        BEVPOOL_CASE(6) BEVPOOL_CASE(10) BEVPOOL_CASE(12) BEVPOOL_CASE(16) BEVPOOL_CASE(20)
        BEVPOOL_CASE(24) BEVPOOL_CASE(32) BEVPOOL_CASE(64)
    default: launch_ppw<DT, FT, CB, SEG, OD>(p, n_short, lds, s); break;
    }
#undef BEVPOOL_CASE
    return hipGetLastError();
}

// The output type as a template argument (segment reductions write fp32 only).
template <int DT, int FT, int CB, bool SEG>
hipError_t launch_out(const FwdParams &p, hipStream_t s)
{
    if (SEG || p.out_dtype == kF32) return launch_typed<DT, FT, CB, SEG, kF32>(p, s);
    if (p.out_dtype == kF16) return launch_typed<DT, FT, CB, SEG, kF16>(p, s);
    if (p.out_dtype == kBF16) return launch_typed<DT, FT, CB, SEG, kBF16>(p, s);
    return hipErrorInvalidValue;
}

template <bool SEG>
hipError_t dispatch(const FwdParams &p, hipStream_t s)
{
    const int row_bytes = p.C * elem_bytes(p.feat_dtype);
    FwdParams q = p;
    if (p.depth_dtype == kF32 && p.feat_dtype == kF32) {
        q.chunks = row_bytes / 16;
        return launch_out<kF32, kF32, 16, SEG>(q, s);
    }
    if (p.depth_dtype == kF16 && p.feat_dtype == kF16) {
        q.chunks = row_bytes / 16;
        return launch_out<kF16, kF16, 16, SEG>(q, s);
    }
    if (p.depth_dtype == kF16 && p.feat_dtype == kE4M3) {
        // 8-byte chunks keep narrow e4m3 rows on the fp16 row geometry (ten
        // lanes a row at C=80); 16-byte chunks measured faster from 256-byte
        // rows (C=256: -10 %) and, for segments, from 128-byte rows (-8 %),
        // but slower below (C=80: +26 %, C=128: +19 %)
        const int wide = SEG ? 128 : 256;
        if (row_bytes <= 8 * kWave && (row_bytes < wide || row_bytes % 16 != 0)) {
            q.chunks = row_bytes / 8;
            return launch_out<kF16, kE4M3, 8, SEG>(q, s);
        }
        q.chunks = row_bytes / 16;
        return launch_out<kF16, kE4M3, 16, SEG>(q, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t run_forward(const FwdParams &p, hipStream_t s)
{
    if (p.n_intervals == 0) {
        const int n4 = p.n_cells * (p.C / 4);                 // groups of four elements
        const int blocks = (n4 + kBlock * kFillPer - 1) / (kBlock * kFillPer);
        if (p.out_dtype == kF32) zero_fill<<<blocks, kBlock, 0, s>>>(static_cast<f32x4 *>(p.out), n4);
        else zero_fill<<<blocks, kBlock, 0, s>>>(static_cast<u32x2 *>(p.out), n4);
        return hipGetLastError();
    }
    return dispatch<false>(p, s);
}

hipError_t run_segment_reduce(const FwdParams &p, hipStream_t s)
{
    return dispatch<true>(p, s);
}

}  // namespace bevpool
