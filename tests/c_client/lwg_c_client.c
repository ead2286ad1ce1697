/*
 * A plain C99 client of liblwg: only lwg.h and the HIP runtime's C API, no C++,
 * no Python, no PyTorch. It shows the boundary works on its own: the caller
 * owns every device buffer and the stream, and the library only enqueues work.
 *
 * Usage: lwg_c_client DIR
 *   DIR/meta.txt      "Z H W C wz wh ww sz sh sw" (grid, width, window, shift)
 *   DIR/x.bin         binary16 [Z*H*W, C], the LayerNorm input and add branch
 *   DIR/residual.bin  binary16 [Z*H*W, C]
 * Writes DIR/{ln,add_r,add_y,table,gather,norm_gather}.bin with the results of
 * lwg_ln_fixed, lwg_add_ln, lwg_window_index_build, lwg_window_gather and
 * lwg_norm_gather, and DIR/status.txt with the statuses of calls that must be
 * refused. Exit status 0 when every call returned what it should.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lwg.h"

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            return 2;                                                                    \
        }                                                                                \
    } while (0)

#define LWG_OK_(call)                                                                    \
    do {                                                                                 \
        int32_t s_ = (call);                                                             \
        if (s_ != LWG_OK) {                                                              \
            fprintf(stderr, "%s: %s (%s)\n", #call, lwg_status_string(s_), lwg_last_error()); \
            return 3;                                                                    \
        }                                                                                \
    } while (0)

static char path_buf[4096];

static const char* path(const char* dir, const char* name) {
    snprintf(path_buf, sizeof path_buf, "%s/%s", dir, name);
    return path_buf;
}

static int read_all(const char* dir, const char* name, void* buf, size_t bytes) {
    FILE* f = fopen(path(dir, name), "rb");
    if (!f) return -1;
    size_t got = fread(buf, 1, bytes, f);
    int extra = fgetc(f);
    fclose(f);
    return (got == bytes && extra == EOF) ? 0 : -1;
}

static int write_all(const char* dir, const char* name, const void* buf, size_t bytes) {
    FILE* f = fopen(path(dir, name), "wb");
    if (!f) return -1;
    size_t put = fwrite(buf, 1, bytes, f);
    return (fclose(f) == 0 && put == bytes) ? 0 : -1;
}

/* One refused call: its status must equal `want` and leave a message. */
static int expect_status(FILE* log, const char* what, int32_t got, int32_t want) {
    const char* msg = lwg_last_error();
    fprintf(log, "%s %s %s\n", what, lwg_status_string(got), got == LWG_OK ? "-" : msg);
    if (got != want) {
        fprintf(stderr, "%s: got %s, want %s\n", what, lwg_status_string(got), lwg_status_string(want));
        return 1;
    }
    if (want != LWG_OK && msg[0] == '\0') {
        fprintf(stderr, "%s: no message from lwg_last_error\n", what);
        return 1;
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    if (lwg_abi_version() != LWG_ABI_VERSION) {
        fprintf(stderr, "ABI version %d, header %d\n", lwg_abi_version(), LWG_ABI_VERSION);
        return 1;
    }

    int Z, H, W, C, wz, wh, ww, sz, sh, sw;
    FILE* meta = fopen(path(dir, "meta.txt"), "r");
    if (!meta || fscanf(meta, "%d %d %d %d %d %d %d %d %d %d", &Z, &H, &W, &C, &wz, &wh, &ww, &sz, &sh,
                        &sw) != 10) {
        fprintf(stderr, "cannot read %s\n", path(dir, "meta.txt"));
        return 1;
    }
    fclose(meta);
    const int64_t n = (int64_t)Z * H * W;
    const int64_t m = lwg_window_token_count(Z, H, W, wz, wh, ww);
    if (n <= 0 || m < n) {
        fprintf(stderr, "bad grid: n=%lld m=%lld\n", (long long)n, (long long)m);
        return 1;
    }
    const size_t row_bytes = (size_t)C * 2;
    const size_t nb = (size_t)n * row_bytes, mb = (size_t)m * row_bytes, tb = (size_t)m * 4;

    uint16_t* hx = malloc(nb);
    uint16_t* hres = malloc(nb);
    void* hout = malloc(mb > nb ? mb : nb);
    if (!hx || !hres || !hout) return 1;
    if (read_all(dir, "x.bin", hx, nb) || read_all(dir, "residual.bin", hres, nb)) {
        fprintf(stderr, "cannot read the inputs\n");
        return 1;
    }

    void *dx, *dres, *dln, *dr, *dy, *dg, *dng;
    int32_t* dtable;
    HIP_OK(hipMalloc(&dx, nb));
    HIP_OK(hipMalloc(&dres, nb));
    HIP_OK(hipMalloc(&dln, nb));
    HIP_OK(hipMalloc(&dr, nb));
    HIP_OK(hipMalloc(&dy, nb));
    HIP_OK(hipMalloc(&dg, mb));
    HIP_OK(hipMalloc(&dng, mb));
    HIP_OK(hipMalloc((void**)&dtable, tb));
    HIP_OK(hipMemcpy(dx, hx, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dres, hres, nb, hipMemcpyHostToDevice));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* the table on the default stream (NULL), the rest on the caller's stream */
    LWG_OK_(lwg_window_index_build(Z, H, W, wz, wh, ww, sz, sh, sw, dtable, m, NULL));
    HIP_OK(hipStreamSynchronize(NULL));
    LWG_OK_(lwg_ln_fixed(dx, dln, n, C, 1e-5, stream));
    LWG_OK_(lwg_add_ln(dx, dres, dr, dy, n, C, 1e-5, stream));
    LWG_OK_(lwg_window_gather(dx, n, C, dtable, m, dg, stream));
    LWG_OK_(lwg_norm_gather(dx, n, C, dtable, m, 1e-5, dng, stream));
    HIP_OK(hipStreamSynchronize(stream));

    struct { const char* name; const void* src; size_t bytes; } outs[] = {
        {"ln.bin", dln, nb}, {"add_r.bin", dr, nb}, {"add_y.bin", dy, nb},
        {"table.bin", dtable, tb}, {"gather.bin", dg, mb}, {"norm_gather.bin", dng, mb},
    };
    for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
        HIP_OK(hipMemcpy(hout, outs[i].src, outs[i].bytes, hipMemcpyDeviceToHost));
        if (write_all(dir, outs[i].name, hout, outs[i].bytes)) {
            fprintf(stderr, "cannot write %s\n", outs[i].name);
            return 1;
        }
    }

    /* calls that must be refused before anything is enqueued, and an empty call */
    FILE* log = fopen(path(dir, "status.txt"), "w");
    if (!log) return 1;
    int bad = 0;
    bad += expect_status(log, "width_100", lwg_ln_fixed(dx, dln, n, 100, 1e-5, stream), LWG_ERR_UNSUPPORTED_WIDTH);
    bad += expect_status(log, "misaligned",
                         lwg_ln_fixed((const char*)dx + 2, dln, n - 1, C, 1e-5, stream), LWG_ERR_MISALIGNED);
    bad += expect_status(log, "eps_negative", lwg_norm_gather(dx, n, C, dtable, m, -1.0, dng, stream),
                         LWG_ERR_INVALID_ARGUMENT);
    bad += expect_status(log, "table_len",
                         lwg_window_index_build(Z, H, W, wz, wh, ww, sz, sh, sw, dtable, m - 1, stream),
                         LWG_ERR_SIZE_MISMATCH);
    bad += expect_status(log, "partial_overlap",
                         lwg_ln_fixed(dx, (char*)dx + row_bytes, n - 1, C, 1e-5, stream), LWG_ERR_ALIASING);
    bad += expect_status(log, "null_x", lwg_ln_fixed(NULL, dln, n, C, 1e-5, stream), LWG_ERR_INVALID_ARGUMENT);
    bad += expect_status(log, "empty", lwg_ln_fixed(NULL, NULL, 0, C, 1e-5, stream), LWG_OK);
    fclose(log);
    HIP_OK(hipStreamSynchronize(stream));

    HIP_OK(hipStreamDestroy(stream));
    void* bufs[] = {dx, dres, dln, dr, dy, dg, dng, dtable};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(hx);
    free(hres);
    free(hout);
    printf("lwg_c_client: n=%lld m=%lld C=%d, %d refused-call check(s) failed\n", (long long)n, (long long)m, C,
           bad);
    return bad ? 4 : 0;
}
