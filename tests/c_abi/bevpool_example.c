/*
 * A plain C consumer of the BEV-pooling C ABI (include/bevpool.h): no Python,
 * no C++.  It reads one problem from a directory, builds the scatter map and
 * pools on the GPU, and writes the map and the pooled grid back, so a test
 * can compare them with the CPU oracle.
 *
 *   bevpool_example <dir>
 *
 * <dir>/meta.txt     "n_img D H W n_cells C feat_dtype depth_dtype out_dtype"
 * <dir>/point_cell   int32 [n_img*D*H*W]
 * <dir>/depth        [n_img*D*H*W] of depth_dtype
 * <dir>/feat         [n_img*H*W, C] of feat_dtype (e4m3 as bytes)
 * writes <dir>/map (n_points, n_intervals, then the five arrays) and
 *        <dir>/out ([n_cells, C] of out_dtype).
 * Exit status 0 on success; otherwise the failing call and its status text
 * are printed.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bevpool.h"

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

#define CHECK_BP(x)                                                                    \
    do {                                                                               \
        int s_ = (x);                                                                  \
        if (s_ != BEVPOOL_OK) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #x, bevpool_status_string(s_));         \
            return 3;                                                                  \
        }                                                                              \
    } while (0)

static size_t dtype_bytes(int dt)
{
    return dt == BEVPOOL_F32 ? 4 : dt == BEVPOOL_FP8_E4M3 ? 1 : 2;
}

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *buf = malloc(bytes ? bytes : 1);
    size_t got = buf ? fread(buf, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(buf);
        return NULL;
    }
    return buf;
}

static int write_file(const char *dir, const char *name, const void *a, size_t na, const void *b,
                      size_t nb)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 1;
    int ok = fwrite(a, 1, na, f) == na && (nb == 0 || fwrite(b, 1, nb, f) == nb);
    fclose(f);
    return ok ? 0 : 1;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s <dir>\n", argv[0]);
        return 1;
    }
    const char *dir = argv[1];
    int n_img, D, H, W, C, fdt, ddt, odt;
    long long n_cells_ll;
    char meta_path[4096];
    snprintf(meta_path, sizeof meta_path, "%s/meta.txt", dir);
    FILE *mf = fopen(meta_path, "r");
    if (!mf || fscanf(mf, "%d %d %d %d %lld %d %d %d %d", &n_img, &D, &H, &W, &n_cells_ll, &C, &fdt,
                      &ddt, &odt) != 9) {
        fprintf(stderr, "cannot read %s\n", meta_path);
        return 1;
    }
    fclose(mf);
    const int64_t n_cells = n_cells_ll;
    const int64_t P = (int64_t)n_img * D * H * W, rows = (int64_t)n_img * H * W;

    /* the library reports bad arguments without touching the GPU */
    if (bevpool_forward(NULL, BEVPOOL_F16, 0, NULL, BEVPOOL_F16, 0, C, 1.0f, NULL, NULL, NULL,
                        NULL, NULL, 0, 0, NULL, n_cells, NULL) != BEVPOOL_ERR_INVALID_ARG) {
        fprintf(stderr, "expected BEVPOOL_ERR_INVALID_ARG for a NULL output\n");
        return 4;
    }

    int32_t *h_pc = read_file(dir, "point_cell", (size_t)P * 4);
    void *h_depth = read_file(dir, "depth", (size_t)P * dtype_bytes(ddt));
    void *h_feat = read_file(dir, "feat", (size_t)(rows * C) * dtype_bytes(fdt));
    if (!h_pc || !h_depth || !h_feat) {
        fprintf(stderr, "cannot read the inputs in %s\n", dir);
        return 1;
    }

    int32_t *d_pc, *d_map[5];
    void *d_depth, *d_feat, *d_out, *d_ws;
    const size_t ws_bytes = bevpool_build_map_workspace_size(n_img, D, H, W, n_cells);
    if (ws_bytes == 0) {
        fprintf(stderr, "bad geometry\n");
        return 1;
    }
    CHECK_HIP(hipMalloc((void **)&d_pc, (size_t)P * 4));
    for (int i = 0; i < 5; ++i) CHECK_HIP(hipMalloc((void **)&d_map[i], (size_t)P * 4));
    CHECK_HIP(hipMalloc(&d_depth, (size_t)P * dtype_bytes(ddt)));
    CHECK_HIP(hipMalloc(&d_feat, (size_t)(rows * C) * dtype_bytes(fdt)));
    CHECK_HIP(hipMalloc(&d_out, (size_t)(n_cells * C) * dtype_bytes(odt)));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMemcpy(d_pc, h_pc, (size_t)P * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_depth, h_depth, (size_t)P * dtype_bytes(ddt), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_feat, h_feat, (size_t)(rows * C) * dtype_bytes(fdt), hipMemcpyHostToDevice));

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    int32_t n_points = 0, n_intervals = 0;
    CHECK_BP(bevpool_build_map(d_pc, n_img, D, H, W, n_cells, d_map[0], d_map[1], d_map[2], d_map[3],
                               d_map[4], P, &n_points, &n_intervals, d_ws, ws_bytes, stream));
    CHECK_BP(bevpool_forward_ex(d_depth, ddt, P, d_feat, fdt, rows, C, 1.0f, d_map[0], d_map[1],
                                d_map[2], d_map[3], d_map[4], n_points, n_intervals, d_out, odt,
                                n_cells, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    const size_t out_bytes = (size_t)(n_cells * C) * dtype_bytes(odt);
    size_t map_bytes = 2 * 4 + (size_t)(3 * n_points + 2 * n_intervals) * 4;
    char *h_map = malloc(map_bytes);
    void *h_out = malloc(out_bytes);
    int32_t counts[2] = {n_points, n_intervals};
    memcpy(h_map, counts, 8);
    size_t off = 8;
    for (int i = 0; i < 5; ++i) {
        const size_t n = (size_t)(i < 3 ? n_points : n_intervals) * 4;
        CHECK_HIP(hipMemcpy(h_map + off, d_map[i], n, hipMemcpyDeviceToHost));
        off += n;
    }
    CHECK_HIP(hipMemcpy(h_out, d_out, out_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "map", h_map, map_bytes, NULL, 0) || write_file(dir, "out", h_out, out_bytes, NULL, 0)) {
        fprintf(stderr, "cannot write the results\n");
        return 1;
    }
    CHECK_HIP(hipStreamDestroy(stream));
    hipFree(d_pc);
    for (int i = 0; i < 5; ++i) hipFree(d_map[i]);
    hipFree(d_depth);
    hipFree(d_feat);
    hipFree(d_out);
    hipFree(d_ws);
    free(h_pc);
    free(h_depth);
    free(h_feat);
    free(h_map);
    free(h_out);
    printf("ok: %d points, %d intervals\n", n_points, n_intervals);
    return 0;
}
