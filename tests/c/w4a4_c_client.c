/*
 * A plain C99 client of the library's C ABI (include/w4a4.h): no C++ and no Python.
 *
 *   w4a4_c_client host
 *       host-side queries only (status names, blob and workspace sizes); prints them.
 *   w4a4_c_client run IN OUT
 *       reads T, d_in, d_out, k, layout, T_cal (int64), alpha (float), X [T][d_in],
 *       X_cal [T_cal][d_in], W [d_out][d_in] (fp32) from IN; runs calibration, packing
 *       and the per-call linear on the current HIP device with hipMalloc'd buffers;
 *       writes s [d_in] (fp32), O [k] (int32) and Y [T][d_out] (fp32) to OUT.
 * Exit status 0 on success; any failing call prints its status name and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "w4a4.h"

#define W4A4_CHECK(call)                                                                  \
    do {                                                                                  \
        const int st_ = (call);                                                           \
        if (st_ != W4A4_OK) {                                                             \
            fprintf(stderr, "%s failed: %s\n", #call, w4a4_status_string(st_));           \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)
#define HIP_CHECK(call)                                                                   \
    do {                                                                                  \
        const hipError_t e_ = (call);                                                     \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static void read_exact(FILE* f, void* p, size_t n) {
    if (fread(p, 1, n, f) != n) {
        fprintf(stderr, "short read\n");
        exit(1);
    }
}

static void* dev_copy(const void* h, size_t n) {
    void* d = NULL;
    HIP_CHECK(hipMalloc(&d, n > 0 ? n : 1));
    if (n > 0) HIP_CHECK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static int host_mode(void) {
    size_t n = 0;
    int s;
    for (s = W4A4_OK; s <= W4A4_ERR_NONFINITE; ++s) printf("status %d %s\n", s, w4a4_status_string(s));
    W4A4_CHECK(w4a4_packed_size(512, 1024, 16, W4A4_WS_1X32, &n));
    printf("packed_size %zu\n", n);
    printf("packed_size_bad_k %d\n", w4a4_packed_size(512, 1024, 513, W4A4_WS_1X32, &n));
    W4A4_CHECK(w4a4_packed_dyn_size(512, 1024, 16, W4A4_WS_1X32, &n));
    printf("packed_dyn_size %zu\n", n);
    return 0;
}

static int run_mode(const char* in_path, const char* out_path) {
    FILE* f = fopen(in_path, "rb");
    int64_t hdr[6];
    float alpha;
    if (!f) {
        fprintf(stderr, "cannot open %s\n", in_path);
        return 1;
    }
    read_exact(f, hdr, sizeof hdr);
    read_exact(f, &alpha, sizeof alpha);
    {
        const int64_t T = hdr[0], d_in = hdr[1], d_out = hdr[2], k = hdr[3], layout = hdr[4], T_cal = hdr[5];
        float* X = (float*)malloc((size_t)(T * d_in) * sizeof(float));
        float* Xc = (float*)malloc((size_t)(T_cal * d_in) * sizeof(float));
        float* W = (float*)malloc((size_t)(d_out * d_in) * sizeof(float));
        float* s = (float*)malloc((size_t)d_in * sizeof(float));
        int32_t* O = (int32_t*)malloc((size_t)(k > 0 ? k : 1) * sizeof(int32_t));
        float* Y = (float*)malloc((size_t)(T * d_out) * sizeof(float));
        void *dX, *dXc, *dW, *blob = NULL, *ws = NULL;
        float* dY = NULL;
        size_t blob_bytes = 0, ws_bytes = 0;
        w4a4_packed desc;
        hipStream_t stream;
        FILE* g;
        read_exact(f, X, (size_t)(T * d_in) * sizeof(float));
        read_exact(f, Xc, (size_t)(T_cal * d_in) * sizeof(float));
        read_exact(f, W, (size_t)(d_out * d_in) * sizeof(float));
        fclose(f);

        HIP_CHECK(hipStreamCreate(&stream));
        dX = dev_copy(X, (size_t)(T * d_in) * sizeof(float));
        dXc = dev_copy(Xc, (size_t)(T_cal * d_in) * sizeof(float));
        dW = dev_copy(W, (size_t)(d_out * d_in) * sizeof(float));

        W4A4_CHECK(w4a4_calibrate_scales(dXc, W4A4_X_F32, T_cal, d_in, (const float*)dW, d_out, alpha,
                                         (int32_t)k, s, O, NULL, NULL, stream));
        W4A4_CHECK(w4a4_packed_size(d_in, d_out, (int32_t)k, (int)layout, &blob_bytes));
        HIP_CHECK(hipMalloc(&blob, blob_bytes));
        W4A4_CHECK(w4a4_pack_weights((const float*)dW, d_in, d_out, s, O, (int32_t)k, (int)layout, blob,
                                     blob_bytes, &desc, stream));
        W4A4_CHECK(w4a4_workspace_size(T, &desc, &ws_bytes));
        HIP_CHECK(hipMalloc(&ws, ws_bytes));
        HIP_CHECK(hipMalloc((void**)&dY, (size_t)(T * d_out) * sizeof(float)));
        W4A4_CHECK(w4a4_linear(dX, W4A4_X_F32, T, &desc, dY, ws, ws_bytes, stream));
        HIP_CHECK(hipStreamSynchronize(stream));
        HIP_CHECK(hipMemcpy(Y, dY, (size_t)(T * d_out) * sizeof(float), hipMemcpyDeviceToHost));

        g = fopen(out_path, "wb");
        if (!g) {
            fprintf(stderr, "cannot open %s\n", out_path);
            return 1;
        }
        fwrite(s, sizeof(float), (size_t)d_in, g);
        fwrite(O, sizeof(int32_t), (size_t)k, g);
        fwrite(Y, sizeof(float), (size_t)(T * d_out), g);
        fclose(g);

        HIP_CHECK(hipFree(dY));
        HIP_CHECK(hipFree(ws));
        HIP_CHECK(hipFree(blob));
        HIP_CHECK(hipFree(dW));
        HIP_CHECK(hipFree(dXc));
        HIP_CHECK(hipFree(dX));
        HIP_CHECK(hipStreamDestroy(stream));
        free(X);
        free(Xc);
        free(W);
        free(s);
        free(O);
        free(Y);
    }
    printf("ok\n");
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode();
    if (argc >= 4 && strcmp(argv[1], "run") == 0) return run_mode(argv[2], argv[3]);
    fprintf(stderr, "usage: %s host | run IN OUT\n", argv[0]);
    return 2;
}
