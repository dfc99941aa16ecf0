/*
 * CPU oracle for BEV pooling: TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct C used to check the HIP path.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it;
 * the product library never calls, links or includes anything here, and
 * this file includes nothing from the product.
 *
 * Source: "Accelerating BEV Pooling on NVIDIA GPUs for Physical AI
 * Applications" (NVIDIA technical blog; Vietnamese and Chinese copies).
 *   - Section "Remove redundant scatter traffic": the operator is the
 *     scatter-reduce  out[ranks_bev[t], c] += depth[ranks_depth[t]] *
 *     feat[ranks_feat[t], c]  over scatter points t, and the scatter map is
 *     five INT32 arrays (ranks_depth, ranks_feat, ranks_bev,
 *     interval_starts, interval_lengths).
 *   - Section "Implement the interval-owned scatter-reduce": the map is
 *     prepared in advance; an interval is a run of points with the same
 *     ranks_bev and its cell is ranks_bev[start]; every output cell is
 *     written once.
 * The article leaves the map's construction open.  Readings used here:
 *   points are the frustum points whose cell is >= 0; they are ordered by
 *   the key (cell, frustum index p), a total order, so the map is unique;
 *   intervals are the maximal runs of equal cell in that order, listed in
 *   increasing cell; ranks_depth[t] = p (depth is [img, D, H, W] flat) and
 *   ranks_feat[t] = img * H * W + h * W + w (feat is [img, H, W, C]);
 *   cells that own no interval are zero.
 * Arithmetic: every value is decoded to double and summed in double in
 * increasing t.  fp16 x fp16 and (e4m3 * fp32 scale) x fp16 products are
 * exact in double, so only the double summation rounds.
 *
 * Pins (tests/test_oracle_pins.py): all 65536 fp16 and 256 e4m3 codes
 * against numpy / torch and the format's closed form; the map against
 * numpy.lexsort and a hand-worked example; the forward against a dense
 * one-hot matrix product, closed forms and invariants; the segmented reduce
 * against torch.nn.functional.embedding_bag and against the forward itself.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_E4M3 = 2 };

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double oracle_decode_f16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m/1024 * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);          /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("FN": finite, no infinities):
 * sign, 4-bit exponent (bias 7), 3-bit mantissa; S.1111.111 is NaN. */
double oracle_decode_e4m3(uint8_t q)
{
    int sign = q >> 7;
    int e = (q >> 3) & 0xf;
    int m = q & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);               /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(8.0 + m, e - 10);             /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double load_value(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[i];
    case ORACLE_F16: return oracle_decode_f16(((const uint16_t *)base)[i]);
    default:         return oracle_decode_e4m3(((const uint8_t *)base)[i]);
    }
}

typedef struct { int64_t cell; int64_t p; } oracle_key;

static int key_cmp(const void *a, const void *b)
{
    const oracle_key *x = (const oracle_key *)a, *y = (const oracle_key *)b;
    if (x->cell != y->cell) return x->cell < y->cell ? -1 : 1;
    if (x->p != y->p) return x->p < y->p ? -1 : 1;
    return 0;
}

/*
 * Scatter map from the per-point cell index.
 * point_cell[p], p < n_img*D*H*W, is a cell in [0, n_cells) or -1 (dropped).
 * Outputs need room for every kept point.  Returns 0, or -1 when a cell is
 * out of range (outputs then undefined), or -2 when memory runs out.
 */
int oracle_build_map(const int32_t *point_cell, int64_t n_img, int64_t D,
                     int64_t H, int64_t W, int64_t n_cells,
                     int32_t *ranks_depth, int32_t *ranks_feat, int32_t *ranks_bev,
                     int32_t *interval_starts, int32_t *interval_lengths,
                     int64_t *n_points, int64_t *n_intervals)
{
    int64_t P = n_img * D * H * W;
    int64_t N = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (point_cell[p] < -1 || point_cell[p] >= n_cells) return -1;
        if (point_cell[p] >= 0) ++N;
    }
    oracle_key *keys = (oracle_key *)malloc((size_t)(N > 0 ? N : 1) * sizeof(oracle_key));
    if (!keys) return -2;
    int64_t k = 0;
    for (int64_t p = 0; p < P; ++p)
        if (point_cell[p] >= 0) { keys[k].cell = point_cell[p]; keys[k].p = p; ++k; }

    /* order the kept points by (cell, p) */
    qsort(keys, (size_t)N, sizeof(oracle_key), key_cmp);

    int64_t dhw = D * H * W, hw = H * W;
    for (int64_t t = 0; t < N; ++t) {
        int64_t p = keys[t].p;
        ranks_bev[t] = (int32_t)keys[t].cell;
        ranks_depth[t] = (int32_t)p;
        ranks_feat[t] = (int32_t)((p / dhw) * hw + p % hw);   /* image, then (h, w) */
    }
    free(keys);

    /* an interval starts wherever the cell changes */
    int64_t I = 0;
    for (int64_t t = 0; t < N; ++t)
        if (t == 0 || ranks_bev[t] != ranks_bev[t - 1])
            interval_starts[I++] = (int32_t)t;
    for (int64_t i = 0; i < I; ++i)
        interval_lengths[i] = (int32_t)((i + 1 < I ? interval_starts[i + 1] : N) - interval_starts[i]);

    *n_points = N;
    *n_intervals = I;
    return 0;
}

/* The forward's operands, as passed to oracle_forward. */
typedef struct {
    const void *depth; int depth_dtype; int64_t n_depth;
    const void *feat; int feat_dtype; int64_t n_feat_rows; int64_t C; double feat_scale;
    const int32_t *ranks_depth, *ranks_feat, *ranks_bev;
    int64_t n_cells;
    double *out, *out_abs;
} oracle_fwd_args;

/* e4m3 values are dequantised with the per-tensor scale; other types not. */
static double feat_scale_of(int feat_dtype, double feat_scale)
{
    return feat_dtype == ORACLE_E4M3 ? feat_scale : 1.0;
}

/* Adds the terms of points [t_lo, t_hi), in increasing t, into out (and
 * out_abs).  Returns -1 on an index outside the stated sizes, else 0. */
static int sum_points(const oracle_fwd_args *a, int64_t t_lo, int64_t t_hi)
{
    int64_t C = a->C;
    double fscale = feat_scale_of(a->feat_dtype, a->feat_scale);
    for (int64_t t = t_lo; t < t_hi; ++t) {
        int64_t rd = a->ranks_depth[t], rf = a->ranks_feat[t], rb = a->ranks_bev[t];
        if (rd < 0 || rd >= a->n_depth || rf < 0 || rf >= a->n_feat_rows || rb < 0 ||
            rb >= a->n_cells)
            return -1;
        double d = load_value(a->depth, a->depth_dtype, rd);
        for (int64_t c = 0; c < C; ++c) {
            double term = d * (load_value(a->feat, a->feat_dtype, rf * C + c) * fscale);
            a->out[rb * C + c] += term;
            if (a->out_abs) a->out_abs[rb * C + c] += fabs(term);
        }
    }
    return 0;
}

static int check_dtypes(int depth_dtype, int feat_dtype)
{
    return depth_dtype >= ORACLE_F32 && depth_dtype <= ORACLE_F16 &&
           feat_dtype >= ORACLE_F32 && feat_dtype <= ORACLE_E4M3;
}

/*
 * The scatter-reduce itself, in double:
 *   out[ranks_bev[t], c] = sum over t (increasing) of
 *                          depth[ranks_depth[t]] * feat[ranks_feat[t], c]
 * with e4m3 features read as e4m3(q) * feat_scale.  Cells no point maps to
 * stay 0.  out_abs (optional) receives the same sum of |term|, the scale of
 * the rounding-error bound of any summation order.
 * out and out_abs are [n_cells, C].  Returns 0, or -1 on a bad dtype or an
 * index outside the stated sizes.
 */
int oracle_forward(const void *depth, int depth_dtype, int64_t n_depth,
                   const void *feat, int feat_dtype, int64_t n_feat_rows, int64_t C,
                   double feat_scale,
                   const int32_t *ranks_depth, const int32_t *ranks_feat,
                   const int32_t *ranks_bev, int64_t n_points, int64_t n_cells,
                   double *out, double *out_abs)
{
    if (!check_dtypes(depth_dtype, feat_dtype)) return -1;
    oracle_fwd_args a = {depth, depth_dtype, n_depth, feat, feat_dtype, n_feat_rows, C,
                         feat_scale, ranks_depth, ranks_feat, ranks_bev, n_cells, out, out_abs};
    memset(out, 0, (size_t)(n_cells * C) * sizeof(double));
    if (out_abs) memset(out_abs, 0, (size_t)(n_cells * C) * sizeof(double));
    return sum_points(&a, 0, n_points);
}

/*
 * The same sum spread over host threads, for timing the oracle on all host
 * cores.  It takes the map's intervals as well, and requires what a map from
 * oracle_build_map satisfies: the intervals tile [0, n_points) in order and
 * their cells strictly increase, so no cell is split between intervals.
 * Thread k takes a contiguous range of whole intervals: those that end at or
 * before point n_points * (k + 1) / n_threads and were not taken by thread
 * k - 1 (the last thread takes the rest), so every cell is summed by one
 * thread over its points in increasing t -- the same operations in the same
 * order as oracle_forward (the same sum_points), hence the same bits for any
 * thread count.  Returns 0, or -1 when the map breaks that structure (or as
 * oracle_forward), or -2 when a thread cannot be started.
 */
typedef struct {
    const oracle_fwd_args *a;
    int64_t t_lo, t_hi;
    int status;
} oracle_range;

static void *sum_range(void *arg)
{
    oracle_range *r = (oracle_range *)arg;
    r->status = sum_points(r->a, r->t_lo, r->t_hi);
    return NULL;
}

int oracle_forward_threads(const void *depth, int depth_dtype, int64_t n_depth,
                           const void *feat, int feat_dtype, int64_t n_feat_rows, int64_t C,
                           double feat_scale,
                           const int32_t *ranks_depth, const int32_t *ranks_feat,
                           const int32_t *ranks_bev, int64_t n_points,
                           const int32_t *interval_starts, const int32_t *interval_lengths,
                           int64_t n_intervals, int64_t n_cells, int n_threads,
                           double *out, double *out_abs)
{
    if (!check_dtypes(depth_dtype, feat_dtype) || n_threads < 1) return -1;
    /* the intervals must tile the points in order, one per cell */
    int64_t next = 0;
    for (int64_t i = 0; i < n_intervals; ++i) {
        int64_t st = interval_starts[i], len = interval_lengths[i];
        if (st != next || len < 1 || st + len > n_points) return -1;
        for (int64_t t = st + 1; t < st + len; ++t)
            if (ranks_bev[t] != ranks_bev[st]) return -1;
        if (i > 0 && ranks_bev[st] <= ranks_bev[st - 1]) return -1;
        next = st + len;
    }
    if (next != n_points) return -1;

    oracle_fwd_args a = {depth, depth_dtype, n_depth, feat, feat_dtype, n_feat_rows, C,
                         feat_scale, ranks_depth, ranks_feat, ranks_bev, n_cells, out, out_abs};
    memset(out, 0, (size_t)(n_cells * C) * sizeof(double));
    if (out_abs) memset(out_abs, 0, (size_t)(n_cells * C) * sizeof(double));
    if (n_threads > n_intervals) n_threads = n_intervals > 0 ? (int)n_intervals : 1;

    oracle_range *rs = (oracle_range *)calloc((size_t)n_threads, sizeof(oracle_range));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!rs || !th) { free(rs); free(th); return -2; }
    int64_t iv = 0;
    for (int k = 0; k < n_threads; ++k) {
        int64_t end = n_points * (k + 1) / n_threads;
        rs[k].a = &a;
        rs[k].t_lo = iv < n_intervals ? interval_starts[iv] : n_points;
        while (iv < n_intervals && interval_starts[iv] + interval_lengths[iv] <= end) ++iv;
        if (k == n_threads - 1) iv = n_intervals;
        rs[k].t_hi = iv < n_intervals ? interval_starts[iv] : n_points;
    }
    int started = 0, status = 0;
    for (; started < n_threads; ++started)
        if (pthread_create(&th[started], NULL, sum_range, &rs[started]) != 0) {
            status = -2;
            break;
        }
    for (int k = 0; k < started; ++k) {
        pthread_join(th[k], NULL);
        if (rs[k].status) status = rs[k].status;
    }
    free(rs);
    free(th);
    return status;
}

/*
 * Weighted segmented gather-reduce, the same owner pattern applied to a
 * generic table ("Accelerating BEV Pooling on NVIDIA GPUs for Physical AI
 * Applications", section "Map the algorithm to hardware" and "Getting
 * started", name sparse embeddings and segmented reductions as the same
 * workload shape):
 *   out[s, c] = sum over t in [offsets[s], offsets[s+1]) (increasing) of
 *               w[t] * table[indices[t], c]
 * with w[t] = 1 when weights is NULL and e4m3 table values read as
 * e4m3(q) * table_scale.  Empty segments are 0.  out (and out_abs, the sum
 * of |term|, optional) are [n_segments, C].  Returns 0, or -1 on a bad dtype,
 * decreasing offsets or an index outside the table.
 */
int oracle_segment_reduce(const void *weights, int w_dtype, const void *table, int t_dtype,
                          int64_t n_rows, int64_t C, double table_scale,
                          const int32_t *indices, const int32_t *offsets, int64_t n_segments,
                          double *out, double *out_abs)
{
    if (weights && (w_dtype < ORACLE_F32 || w_dtype > ORACLE_F16)) return -1;
    if (t_dtype < ORACLE_F32 || t_dtype > ORACLE_E4M3) return -1;
    double tscale = t_dtype == ORACLE_E4M3 ? table_scale : 1.0;
    memset(out, 0, (size_t)(n_segments * C) * sizeof(double));
    if (out_abs) memset(out_abs, 0, (size_t)(n_segments * C) * sizeof(double));
    for (int64_t s = 0; s < n_segments; ++s) {
        if (offsets[s + 1] < offsets[s]) return -1;
        for (int64_t t = offsets[s]; t < offsets[s + 1]; ++t) {
            int64_t r = indices[t];
            if (r < 0 || r >= n_rows) return -1;
            double w = weights ? load_value(weights, w_dtype, t) : 1.0;
            for (int64_t c = 0; c < C; ++c) {
                double term = w * (load_value(table, t_dtype, r * C + c) * tscale);
                out[s * C + c] += term;
                if (out_abs) out_abs[s * C + c] += fabs(term);
            }
        }
    }
    return 0;
}
