// C-ABI front end of the W4A4 library: argument validation, size queries, blob and
// workspace layout, the host half of offline calibration, and kernel dispatch.
// The operations and their page citations are documented in include/w4a4.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

#include "w4a4_internal.h"

using namespace w4a4;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

int dev_status(hipError_t e) { return e == hipSuccess ? W4A4_OK : W4A4_ERR_DEVICE; }

int64_t weight_scale_bytes(int64_t d_out, int64_t k_pad, int layout) {
    if (layout == W4A4_WS_1X32) return d_out * (k_pad / 32);
    if (layout == W4A4_WS_128X1_STRIPE) return d_out * (k_pad / 128);
    return (k_pad / 32) * ((d_out + 31) / 32);
}

struct BlobLayout {
    size_t colmap, s, O, J, B_q, B_s, B_s_rows, W_O, B_q_tiles, total;
};

BlobLayout blob_layout(int64_t d_in, int64_t d_out, int32_t k, int layout) {
    const int64_t k_j = d_in - k;
    const int64_t k_pad = round_up(k_j, 128);
    const int64_t k_ld = round_up(k, 32);
    BlobLayout b;
    size_t off = 0;
    b.colmap = off; off = align_up(off + (size_t)d_in * 4);
    b.s = off;      off = align_up(off + (size_t)d_in * 4);
    b.O = off;      off = align_up(off + (size_t)k * 4);
    b.J = off;      off = align_up(off + (size_t)k_j * 4);
    b.B_q = off;    off = align_up(off + (size_t)(d_out * (k_pad / 2)));
    b.B_s = off;    off = align_up(off + (size_t)weight_scale_bytes(d_out, k_pad, layout));
    b.B_s_rows = off;     off = align_up(off + (size_t)(d_out * (k_pad / 32)));
    b.W_O = off;    off = align_up(off + (size_t)(d_out * k_ld) * 2);
    b.B_q_tiles = off; off = align_up(off + (size_t)(round_up(d_out, 16) * (k_pad / 2)));
    b.total = off;
    return b;
}

bool valid_layout(int layout) {
    return layout == W4A4_WS_1X32 || layout == W4A4_WS_32X32_TILE || layout == W4A4_WS_128X1_STRIPE;
}

int check_dims(int64_t d_in, int64_t d_out, int32_t k, int layout) {
    if (!valid_layout(layout)) return W4A4_ERR_INVALID;
    if (d_in <= 0 || d_out <= 0 || k < 0 || k > d_in) return W4A4_ERR_INVALID;
    if (d_in > W4A4_MAX_D_IN) return W4A4_ERR_SHAPE;
    if (d_out > ((int64_t)1 << 30)) return W4A4_ERR_SHAPE;
    return W4A4_OK;
}

int check_desc(const w4a4_packed* d) {
    if (!d) return W4A4_ERR_INVALID;
    int st = check_dims(d->d_in, d->d_out, d->k, d->layout);
    if (st) return st;
    if (d->k_j != d->d_in - d->k || d->k_pad != round_up(d->k_j, 128) || d->k_ld != round_up(d->k, 32))
        return W4A4_ERR_INVALID;
    if (!d->colmap || !d->s) return W4A4_ERR_INVALID;
    if (d->k_pad > 0 && (!d->B_q || !d->B_s || !d->B_s_rows || !d->B_q_tiles || !d->J))
        return W4A4_ERR_INVALID;
    if (d->k > 0 && (!d->W_O || !d->O)) return W4A4_ERR_INVALID;
    if (misaligned(d->colmap) || misaligned(d->s) || misaligned(d->B_q) || misaligned(d->W_O) ||
        misaligned(d->B_q_tiles))
        return W4A4_ERR_ALIGN;
    return W4A4_OK;
}

w4a4_ws_layout ws_layout_of(int64_t T, int64_t d_out, int64_t k_pad, int64_t k_ld) {
    w4a4_ws_layout w;
    size_t off = 0;
    w.a_q = off;     off = align_up(off + (size_t)(round_up(T, 16) * (k_pad / 2)));
    w.a_s = off;     off = align_up(off + (size_t)(T * (k_pad / 32)));
    w.x_o = off;     off = align_up(off + (size_t)(T * k_ld) * 2);
    w.partial = off; off = align_up(off + gemm_split_plan(T, d_out, k_pad, k_ld).part_bytes);
    w.total = off;
    return w;
}
w4a4_ws_layout ws_layout(int64_t T, const w4a4_packed* d) { return ws_layout_of(T, d->d_out, d->k_pad, d->k_ld); }

// Host half of calibration from the column maxima (bit patterns of max |x| over the
// calibration tokens and of max |w| over the outputs, per input column):
// s_j = a^alpha / w^(1-alpha) (sec. 3.2), maxima floored at 1e-5, in double with one
// rounding; the static top-k of score_j = a_j / s_j (sec. 3.3, scored after the fold
// per sec. 3.5), larger score first, ties to the smaller column, O ascending.
int smooth_and_select(const uint32_t* act_bits, const uint32_t* w_bits, int64_t d_in, float alpha, int32_t k,
                      float* s_out, int32_t* O_out, float* act_scale_out, float* weight_scale_out) {
    std::vector<float> act((size_t)d_in), wsc((size_t)d_in);
    for (int64_t j = 0; j < d_in; ++j) {
        if (act_bits[j] >= 0x7F800000u || w_bits[j] >= 0x7F800000u) return W4A4_ERR_NONFINITE;
        std::memcpy(&act[j], &act_bits[j], 4);
        std::memcpy(&wsc[j], &w_bits[j], 4);
    }
    const float floor_v = 1e-5f;
    std::vector<float> score((size_t)d_in);
    for (int64_t j = 0; j < d_in; ++j) {
        const float a = act[j] > floor_v ? act[j] : floor_v;
        const float w = wsc[j] > floor_v ? wsc[j] : floor_v;
        const double num = std::pow((double)a, (double)alpha);
        const double den = std::pow((double)w, 1.0 - (double)alpha);
        s_out[j] = (float)(num / den);
        score[j] = act[j] / s_out[j];   // = max_t |x_tj / s_j| (binary32 division is monotone)
    }
    if (act_scale_out) std::memcpy(act_scale_out, act.data(), (size_t)d_in * 4);
    if (weight_scale_out) std::memcpy(weight_scale_out, wsc.data(), (size_t)d_in * 4);
    std::vector<int32_t> idx((size_t)d_in);
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return score[x] > score[y]; });
    std::sort(idx.begin(), idx.begin() + k);
    for (int32_t i = 0; i < k; ++i) O_out[i] = idx[i];
    return W4A4_OK;
}

// Caller scratch of the alpha / k search: column maxima | packed blob | workspace |
// reference Y | quantized Y | per-block error sums (sizes for the largest candidate).
constexpr int kErrBlocks = 512;
struct SearchLayout {
    size_t cols, blob, ws, y_ref, y_q, partials, total, blob_bytes, ws_bytes;
};
SearchLayout search_layout(int64_t T, int64_t d_in, int64_t d_out, const int32_t* ks, int n_k, int layout) {
    SearchLayout L;
    L.blob_bytes = 0;
    L.ws_bytes = 0;
    for (int b = 0; b < n_k; ++b) {
        L.blob_bytes = std::max(L.blob_bytes, blob_layout(d_in, d_out, ks[b], layout).total);
        const int64_t k_pad = round_up(d_in - ks[b], 128), k_ld = round_up(ks[b], 32);
        L.ws_bytes = std::max(L.ws_bytes, ws_layout_of(T, d_out, k_pad, k_ld).total);
    }
    size_t off = 0;
    L.cols = off;     off = align_up(off + (size_t)d_in * 2 * sizeof(uint32_t));
    L.blob = off;     off = align_up(off + L.blob_bytes);
    L.ws = off;       off = align_up(off + L.ws_bytes);
    L.y_ref = off;    off = align_up(off + (size_t)(T * d_out) * sizeof(float));
    L.y_q = off;      off = align_up(off + (size_t)(T * d_out) * sizeof(float));
    L.partials = off; off = align_up(off + (size_t)kErrBlocks * 2 * sizeof(double));
    L.total = off;
    return L;
}

// Per-call outlier path: the blob is the k = 0 layer's blob followed by W_t; the
// workspace is the k-column layer's (over K_pad = roundup(d_in, 128)) followed by the
// per-call column maxima, O, column map and W_O.
int check_dyn_dims(int64_t d_in, int64_t d_out, int32_t k, int layout) {
    const int st = check_dims(d_in, d_out, k, layout);
    if (st) return st;
    if (d_in % 2 != 0 || d_in > W4A4_DYN_MAX_D_IN) return W4A4_ERR_SHAPE;
    return W4A4_OK;
}
size_t dyn_blob_base(int64_t d_in, int64_t d_out, int layout) { return blob_layout(d_in, d_out, 0, layout).total; }
size_t dyn_blob_total(int64_t d_in, int64_t d_out, int layout) {
    return dyn_blob_base(d_in, d_out, layout) + align_up((size_t)(d_out * d_in) * 2);
}
w4a4_ws_dyn_layout ws_dyn_layout(int64_t T, const w4a4_packed_dyn* d) {
    w4a4_ws_dyn_layout w;
    w.base = ws_layout_of(T, d->base.d_out, d->base.k_pad, round_up(d->k, 32));
    size_t off = w.base.total;
    w.colmax = off; off = align_up(off + (size_t)d->base.d_in * 4);
    w.O = off;      off = align_up(off + (size_t)(d->k > 0 ? d->k : 1) * 4);
    w.colmap = off; off = align_up(off + (size_t)d->base.d_in * 4);
    w.W_O = off;    off = align_up(off + (size_t)(d->base.d_out * round_up(d->k, 32)) * 2);
    w.total = off;
    return w;
}
int check_desc_dyn(const w4a4_packed_dyn* d) {
    if (!d) return W4A4_ERR_INVALID;
    int st = check_desc(&d->base);
    if (st) return st;
    if (d->base.k != 0) return W4A4_ERR_INVALID;
    st = check_dyn_dims(d->base.d_in, d->base.d_out, d->k, d->base.layout);
    if (st) return st;
    if (!d->W_t) return W4A4_ERR_INVALID;
    if (misaligned(d->W_t)) return W4A4_ERR_ALIGN;
    return W4A4_OK;
}

int check_search_args(int64_t T_cal, int64_t d_in, int64_t d_out, const int32_t* ks, int n_k, int layout) {
    if (!ks || n_k <= 0 || T_cal <= 0) return W4A4_ERR_INVALID;
    for (int b = 0; b < n_k; ++b) {
        const int st = check_dims(d_in, d_out, ks[b], layout);
        if (st) return st;
    }
    // the reference kernel's grid has at most 65535 row blocks of 64 tokens
    if (T_cal > (int64_t)65535 * 64 || T_cal * d_out > ((int64_t)1 << 40)) return W4A4_ERR_SHAPE;
    return W4A4_OK;
}

}  // namespace

extern "C" {

const char* w4a4_status_string(int status) {
    switch (status) {
        case W4A4_OK: return "ok";
        case W4A4_ERR_INVALID: return "invalid argument";
        case W4A4_ERR_SHAPE: return "unsupported shape or buffer too small";
        case W4A4_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case W4A4_ERR_DEVICE: return "HIP runtime error";
        case W4A4_ERR_NONFINITE: return "non-finite calibration data";
        case W4A4_ERR_SCRATCH: return "workspace needed exceeds the fixed scratch of w4a4_linear_noalloc";
        default: return "unknown status";
    }
}

int w4a4_column_absmax(const void* X, int x_dtype, int64_t rows, int64_t cols, uint32_t* out_bits,
                       void* stream) {
    if (!X || !out_bits || rows < 0 || cols < 0) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    return dev_status(launch_column_absmax(X, x_dtype, rows, cols, out_bits, (hipStream_t)stream));
}

int w4a4_calibrate_scales(const void* X_cal, int x_dtype, int64_t T_cal, int64_t d_in, const float* W,
                          int64_t d_out, float alpha, int32_t k, float* s_out, int32_t* O_out,
                          float* act_scale_out, float* weight_scale_out, void* stream) {
    if (!X_cal || !W || !s_out || (k > 0 && !O_out)) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    if (T_cal <= 0 || d_in <= 0 || d_out <= 0 || k < 0 || k > d_in) return W4A4_ERR_INVALID;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return W4A4_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    uint32_t* dev = nullptr;
    if (hipMalloc(&dev, (size_t)d_in * 2 * sizeof(uint32_t)) != hipSuccess) return W4A4_ERR_DEVICE;
    std::vector<uint32_t> bits((size_t)d_in * 2);
    hipError_t e = launch_column_absmax(X_cal, x_dtype, T_cal, d_in, dev, st);
    if (e == hipSuccess) e = launch_column_absmax(W, W4A4_X_F32, d_out, d_in, dev + d_in, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(bits.data(), dev, bits.size() * sizeof(uint32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipFree(dev);
    if (e != hipSuccess) return W4A4_ERR_DEVICE;

    return smooth_and_select(bits.data(), bits.data() + d_in, d_in, alpha, k, s_out, O_out, act_scale_out,
                             weight_scale_out);
}

int w4a4_packed_size(int64_t d_in, int64_t d_out, int32_t k, int layout, size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    const int st = check_dims(d_in, d_out, k, layout);
    if (st) return st;
    *bytes = blob_layout(d_in, d_out, k, layout).total;
    return W4A4_OK;
}

int w4a4_pack_weights(const float* W, int64_t d_in, int64_t d_out, const float* s, const int32_t* O,
                      int32_t k, int layout, void* blob, size_t blob_bytes, w4a4_packed* desc,
                      void* stream) {
    if (!W || !s || !blob || !desc || (k > 0 && !O)) return W4A4_ERR_INVALID;
    int st = check_dims(d_in, d_out, k, layout);
    if (st) return st;
    if (((uintptr_t)W & 3u) != 0 || misaligned(blob)) return W4A4_ERR_ALIGN;
    const BlobLayout b = blob_layout(d_in, d_out, k, layout);
    if (blob_bytes < b.total) return W4A4_ERR_SHAPE;
    for (int64_t j = 0; j < d_in; ++j)
        if (!(s[j] > 0.0f) || !std::isfinite(s[j])) return W4A4_ERR_INVALID;
    for (int32_t i = 0; i < k; ++i) {
        if (O[i] < 0 || O[i] >= d_in) return W4A4_ERR_INVALID;
        if (i > 0 && O[i] <= O[i - 1]) return W4A4_ERR_INVALID;
    }
    const int64_t k_j = d_in - k;
    std::vector<int32_t> colmap((size_t)d_in), J((size_t)k_j);
    {
        int32_t io = 0, p = 0;
        for (int64_t j = 0; j < d_in; ++j) {
            if (io < k && O[io] == j) { colmap[j] = -(io + 1); ++io; }
            else { colmap[j] = p; J[p] = (int32_t)j; ++p; }
        }
    }
    uint8_t* base = (uint8_t*)blob;
    w4a4_packed d;
    d.d_in = d_in;
    d.d_out = d_out;
    d.k = k;
    d.layout = layout;
    d.k_j = k_j;
    d.k_pad = round_up(k_j, 128);
    d.k_ld = round_up(k, 32);
    d.colmap = (const int32_t*)(base + b.colmap);
    d.s = (const float*)(base + b.s);
    d.O = (const int32_t*)(base + b.O);
    d.J = (const int32_t*)(base + b.J);
    d.B_q = base + b.B_q;
    d.B_s = base + b.B_s;
    d.B_s_rows = base + b.B_s_rows;
    d.B_q_tiles = base + b.B_q_tiles;
    d.W_O = (const uint16_t*)(base + b.W_O);

    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync((void*)d.colmap, colmap.data(), (size_t)d_in * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync((void*)d.s, s, (size_t)d_in * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess && k > 0) e = hipMemcpyAsync((void*)d.O, O, (size_t)k * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess && k_j > 0)
        e = hipMemcpyAsync((void*)d.J, J.data(), (size_t)k_j * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = launch_pack(W, d, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return W4A4_ERR_DEVICE;
    *desc = d;
    return W4A4_OK;
}

int w4a4_workspace_layout(int64_t T, const w4a4_packed* desc, w4a4_ws_layout* out) {
    if (!out || T < 0) return W4A4_ERR_INVALID;
    const int st = check_desc(desc);
    if (st) return st;
    *out = ws_layout(T, desc);
    return W4A4_OK;
}

int w4a4_workspace_size(int64_t T, const w4a4_packed* desc, size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    w4a4_ws_layout w;
    const int st = w4a4_workspace_layout(T, desc, &w);
    if (st) return st;
    *bytes = w.total;
    return W4A4_OK;
}

int w4a4_quantize_activations(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, void* ws,
                              size_t ws_bytes, void* stream) {
    if (T < 0) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    int st = check_desc(desc);
    if (st) return st;
    if (T == 0) return W4A4_OK;
    if (!X || !ws) return W4A4_ERR_INVALID;
    if (misaligned(X) || misaligned(ws)) return W4A4_ERR_ALIGN;
    const w4a4_ws_layout w = ws_layout(T, desc);
    if (ws_bytes < w.total) return W4A4_ERR_SHAPE;
    uint8_t* b = (uint8_t*)ws;
    return dev_status(launch_actprep(X, x_dtype, T, *desc, b + w.a_q, b + w.a_s, (uint16_t*)(b + w.x_o),
                                     (hipStream_t)stream));
}

}  // extern "C"

namespace {

int gemm_into(void* ws, size_t ws_bytes, int64_t T, const w4a4_packed* desc, void* out, bool gelu,
              void* stream) {
    if (T < 0) return W4A4_ERR_INVALID;
    int st = check_desc(desc);
    if (st) return st;
    if (T == 0) return W4A4_OK;
    if (!ws || !out) return W4A4_ERR_INVALID;
    if (misaligned(ws) || misaligned(out)) return W4A4_ERR_ALIGN;
    const w4a4_ws_layout w = ws_layout(T, desc);
    if (ws_bytes < w.total) return W4A4_ERR_SHAPE;
    uint8_t* b = (uint8_t*)ws;
    return dev_status(launch_gemm(b + w.a_q, b + w.a_s, (const uint16_t*)(b + w.x_o), T, *desc, out, gelu,
                                  (float*)(b + w.partial),
                                  (hipStream_t)stream));
}

int linear_into(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, void* out, bool gelu,
                void* ws, size_t ws_bytes, void* stream) {
    if (T < 0) return W4A4_ERR_INVALID;
    int st = check_desc(desc);
    if (st) return st;
    if (T == 0) return W4A4_OK;
    if (!out) return W4A4_ERR_INVALID;
    if (misaligned(out)) return W4A4_ERR_ALIGN;
    st = w4a4_quantize_activations(X, x_dtype, T, desc, ws, ws_bytes, stream);
    if (st) return st;
    return gemm_into(ws, ws_bytes, T, desc, out, gelu, stream);
}

w4a4_ffn_ws_layout ffn_layout(int64_t T, const w4a4_packed* up, const w4a4_packed* down) {
    w4a4_ffn_ws_layout w;
    w.up = ws_layout(T, up);
    w.up_base = 0;
    w.down = ws_layout(T, down);
    w.down_base = align_up(w.up.total);
    w.rinv = align_up(w.down_base + w.down.total);
    w.total = align_up(w.rinv + (size_t)down->k_j * sizeof(double));
    return w;
}
int check_ffn(int64_t T, const w4a4_packed* up, const w4a4_packed* down) {
    if (T < 0) return W4A4_ERR_INVALID;
    int st = check_desc(up);
    if (st) return st;
    st = check_desc(down);
    if (st) return st;
    if (up->d_out != down->d_in) return W4A4_ERR_SHAPE;
    return W4A4_OK;
}

}  // namespace

extern "C" {

int w4a4_ffn_workspace_layout(int64_t T, const w4a4_packed* up, const w4a4_packed* down, w4a4_ffn_ws_layout* out) {
    if (!out) return W4A4_ERR_INVALID;
    const int st = check_ffn(T, up, down);
    if (st) return st;
    *out = ffn_layout(T, up, down);
    return W4A4_OK;
}

int w4a4_ffn_workspace_size(int64_t T, const w4a4_packed* up, const w4a4_packed* down, size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    w4a4_ffn_ws_layout w;
    const int st = w4a4_ffn_workspace_layout(T, up, down, &w);
    if (st) return st;
    *bytes = w.total;
    return W4A4_OK;
}

int w4a4_ffn_up_quantize(const void* X, int x_dtype, int64_t T, const w4a4_packed* up, const w4a4_packed* down,
                         void* ws, size_t ws_bytes, void* stream) {
    int st = check_ffn(T, up, down);
    if (st) return st;
    if (!X || !ws) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    if (misaligned(X) || misaligned(ws)) return W4A4_ERR_ALIGN;
    const w4a4_ffn_ws_layout w = ffn_layout(T, up, down);
    if (ws_bytes < w.total) return W4A4_ERR_SHAPE;
    if (T == 0) return W4A4_OK;
    uint8_t* b = (uint8_t*)ws;
    st = w4a4_quantize_activations(X, x_dtype, T, up, b + w.up_base, w.up.total, stream);
    if (st) return st;
    uint8_t* d = b + w.down_base;
    QuantDst q;
    q.aq = d + w.down.a_q;
    q.as = d + w.down.a_s;
    q.xo = (uint16_t*)(d + w.down.x_o);
    q.rinv = (const double*)(b + w.rinv);
    q.k_j = down->k_j;
    q.k_pad = down->k_pad;
    q.k_ld = down->k_ld;
    q.k = down->k;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = launch_ffn_prologue(*down, T, q, hs);
    if (e == hipSuccess) {
        uint8_t* u = b + w.up_base;
        e = launch_gemm_quant(u + w.up.a_q, u + w.up.a_s, (const uint16_t*)(u + w.up.x_o), T, *up, q,
                              (float*)(b + w.up_base + w.up.partial), hs);
    }
    return dev_status(e);
}

int w4a4_ffn_forward(const void* X, int x_dtype, int64_t T, const w4a4_packed* up, const w4a4_packed* down,
                     float* Y, void* ws, size_t ws_bytes, void* stream) {
    int st = check_ffn(T, up, down);
    if (st) return st;
    if (!Y) return W4A4_ERR_INVALID;
    if (misaligned(Y)) return W4A4_ERR_ALIGN;
    st = w4a4_ffn_up_quantize(X, x_dtype, T, up, down, ws, ws_bytes, stream);
    if (st || T == 0) return st;
    const w4a4_ffn_ws_layout w = ffn_layout(T, up, down);
    return gemm_into((uint8_t*)ws + w.down_base, w.down.total, T, down, Y, false, stream);
}

int w4a4_gemm_prequantized(void* ws, size_t ws_bytes, int64_t T, const w4a4_packed* desc, float* Y,
                           void* stream) {
    return gemm_into(ws, ws_bytes, T, desc, Y, false, stream);
}

int w4a4_gemm_prequantized_gelu_bf16(void* ws, size_t ws_bytes, int64_t T, const w4a4_packed* desc,
                                     uint16_t* H, void* stream) {
    return gemm_into(ws, ws_bytes, T, desc, H, true, stream);
}

int w4a4_linear(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, float* Y, void* ws,
                size_t ws_bytes, void* stream) {
    return linear_into(X, x_dtype, T, desc, Y, false, ws, ws_bytes, stream);
}

int w4a4_linear_gelu_bf16(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, uint16_t* H,
                          void* ws, size_t ws_bytes, void* stream) {
    return linear_into(X, x_dtype, T, desc, H, true, ws, ws_bytes, stream);
}

int w4a4_packed_dyn_size(int64_t d_in, int64_t d_out, int32_t k, int layout, size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    const int st = check_dyn_dims(d_in, d_out, k, layout);
    if (st) return st;
    *bytes = dyn_blob_total(d_in, d_out, layout);
    return W4A4_OK;
}

int w4a4_pack_weights_dyn(const float* W, int64_t d_in, int64_t d_out, const float* s, int32_t k, int layout,
                          void* blob, size_t blob_bytes, w4a4_packed_dyn* desc, void* stream) {
    if (!W || !s || !blob || !desc) return W4A4_ERR_INVALID;
    int st = check_dyn_dims(d_in, d_out, k, layout);
    if (st) return st;
    if (blob_bytes < dyn_blob_total(d_in, d_out, layout)) return W4A4_ERR_SHAPE;
    const int32_t no_outliers = 0;
    st = w4a4_pack_weights(W, d_in, d_out, s, &no_outliers, 0, layout, blob, dyn_blob_base(d_in, d_out, layout),
                           &desc->base, stream);
    if (st) return st;
    uint16_t* wbf = (uint16_t*)((uint8_t*)blob + dyn_blob_base(d_in, d_out, layout));
    const hipError_t e = launch_dyn_transpose(W, d_in, d_out, wbf, (hipStream_t)stream);
    if (e != hipSuccess) return W4A4_ERR_DEVICE;
    desc->k = k;
    desc->reserved = 0;
    desc->W_t = wbf;
    return W4A4_OK;
}

int w4a4_workspace_dyn_layout(int64_t T, const w4a4_packed_dyn* desc, w4a4_ws_dyn_layout* out) {
    if (!out || T < 0) return W4A4_ERR_INVALID;
    const int st = check_desc_dyn(desc);
    if (st) return st;
    *out = ws_dyn_layout(T, desc);
    return W4A4_OK;
}

int w4a4_workspace_dyn_size(int64_t T, const w4a4_packed_dyn* desc, size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    w4a4_ws_dyn_layout w;
    const int st = w4a4_workspace_dyn_layout(T, desc, &w);
    if (st) return st;
    *bytes = w.total;
    return W4A4_OK;
}

int w4a4_linear_dyn(const void* X, int x_dtype, int64_t T, const w4a4_packed_dyn* desc, float* Y, void* ws,
                    size_t ws_bytes, void* stream) {
    if (!X || !Y || !ws || T < 0) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    int st = check_desc_dyn(desc);
    if (st) return st;
    if (misaligned(X) || misaligned(Y) || misaligned(ws)) return W4A4_ERR_ALIGN;
    const w4a4_ws_dyn_layout w = ws_dyn_layout(T, desc);
    if (ws_bytes < w.total) return W4A4_ERR_SHAPE;
    if (T == 0) return W4A4_OK;
    hipStream_t hs = (hipStream_t)stream;
    uint8_t* b = (uint8_t*)ws;
    const w4a4_packed& base = desc->base;
    const int64_t k_ld = round_up(desc->k, 32);
    uint32_t* colmax = (uint32_t*)(b + w.colmax);
    int32_t* O = (int32_t*)(b + w.O);
    int32_t* colmap = (int32_t*)(b + w.colmap);
    uint16_t* W_O = (uint16_t*)(b + w.W_O);
    hipError_t e = launch_column_absmax(X, x_dtype, T, base.d_in, colmax, hs);
    if (e == hipSuccess) e = launch_dyn_select(colmax, base.s, base.d_in, desc->k, O, colmap, hs);
    if (e == hipSuccess) e = launch_dyn_gather(desc->W_t, O, base.d_in, base.d_out, desc->k, k_ld, W_O, hs);
    if (e != hipSuccess) return W4A4_ERR_DEVICE;
    // The call's layer: every column keeps its K position; act-prep zeroes the J
    // positions [k_j, k_pad) of its LDS row once per workgroup and never writes the J
    // position of an outlier column, so k_j = 0 leaves the chosen columns at zero.
    w4a4_packed d = base;
    d.k = desc->k;
    d.k_ld = k_ld;
    d.k_j = 0;
    d.colmap = colmap;
    d.O = O;
    d.W_O = W_O;
    e = launch_actprep(X, x_dtype, T, d, b + w.base.a_q, b + w.base.a_s, (uint16_t*)(b + w.base.x_o), hs);
    if (e == hipSuccess)
        e = launch_gemm(b + w.base.a_q, b + w.base.a_s, (const uint16_t*)(b + w.base.x_o), T, d, Y, false,
                        (float*)(b + w.base.partial), hs);
    return dev_status(e);
}

int w4a4_search_scratch_size(int64_t T_cal, int64_t d_in, int64_t d_out, const int32_t* ks, int n_k, int layout,
                             size_t* bytes) {
    if (!bytes) return W4A4_ERR_INVALID;
    const int st = check_search_args(T_cal, d_in, d_out, ks, n_k, layout);
    if (st) return st;
    *bytes = search_layout(T_cal, d_in, d_out, ks, n_k, layout).total;
    return W4A4_OK;
}

int w4a4_search_alpha_k(const void* X_cal, int x_dtype, int64_t T_cal, int64_t d_in, const float* W,
                        int64_t d_out, const float* alphas, int n_alpha, const int32_t* ks, int n_k, int layout,
                        void* scratch, size_t scratch_bytes, double* err_out, int32_t* best_out, void* stream) {
    if (!X_cal || !W || !alphas || n_alpha <= 0 || !scratch || !err_out || !best_out) return W4A4_ERR_INVALID;
    if (x_dtype != W4A4_X_F32 && x_dtype != W4A4_X_BF16) return W4A4_ERR_INVALID;
    for (int a = 0; a < n_alpha; ++a)
        if (!(alphas[a] >= 0.0f && alphas[a] <= 1.0f)) return W4A4_ERR_INVALID;
    int st = check_search_args(T_cal, d_in, d_out, ks, n_k, layout);
    if (st) return st;
    if (misaligned(X_cal) || misaligned(W) || misaligned(scratch)) return W4A4_ERR_ALIGN;
    const SearchLayout L = search_layout(T_cal, d_in, d_out, ks, n_k, layout);
    if (scratch_bytes < L.total) return W4A4_ERR_SHAPE;
    hipStream_t hs = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)scratch;
    uint32_t* cols = (uint32_t*)(base + L.cols);
    float* y_ref = (float*)(base + L.y_ref);
    float* y_q = (float*)(base + L.y_q);
    double* partials = (double*)(base + L.partials);
    const int64_t n = T_cal * d_out;

    // column maxima once for the whole grid, and the unquantized reference product
    std::vector<uint32_t> bits((size_t)d_in * 2);
    hipError_t e = launch_column_absmax(X_cal, x_dtype, T_cal, d_in, cols, hs);
    if (e == hipSuccess) e = launch_column_absmax(W, W4A4_X_F32, d_out, d_in, cols + d_in, hs);
    if (e == hipSuccess)
        e = hipMemcpyAsync(bits.data(), cols, bits.size() * sizeof(uint32_t), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = launch_ref_linear(X_cal, x_dtype, T_cal, d_in, W, d_out, y_ref, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return W4A4_ERR_DEVICE;

    std::vector<float> s((size_t)d_in);
    std::vector<double> part((size_t)kErrBlocks * 2);
    best_out[0] = best_out[1] = -1;
    double best = 0.0;
    for (int a = 0; a < n_alpha; ++a) {
        for (int b = 0; b < n_k; ++b) {
            std::vector<int32_t> O((size_t)ks[b] + 1);
            st = smooth_and_select(bits.data(), bits.data() + d_in, d_in, alphas[a], ks[b], s.data(), O.data(),
                                   nullptr, nullptr);
            if (st) return st;
            w4a4_packed desc;
            st = w4a4_pack_weights(W, d_in, d_out, s.data(), O.data(), ks[b], layout, base + L.blob,
                                   L.blob_bytes, &desc, stream);
            if (st) return st;
            st = w4a4_linear(X_cal, x_dtype, T_cal, &desc, y_q, base + L.ws, L.ws_bytes, stream);
            if (st) return st;
            e = launch_sq_err(y_q, y_ref, n, partials, kErrBlocks, hs);
            if (e == hipSuccess)
                e = hipMemcpyAsync(part.data(), partials, part.size() * sizeof(double), hipMemcpyDeviceToHost, hs);
            if (e == hipSuccess) e = hipStreamSynchronize(hs);
            if (e != hipSuccess) return W4A4_ERR_DEVICE;
            double num = 0.0, den = 0.0;
            for (int i = 0; i < kErrBlocks; ++i) {
                num += part[2 * i];
                den += part[2 * i + 1];
            }
            const double err = std::sqrt(num / den);
            err_out[a * n_k + b] = err;
            if (std::isfinite(err) && (best_out[0] < 0 || err < best)) {
                best = err;
                best_out[0] = a;
                best_out[1] = b;
            }
        }
    }
    return W4A4_OK;
}

int w4a4_gelu_tanh_bf16(const float* Y, int64_t n, uint16_t* H, void* stream) {
    if (n < 0) return W4A4_ERR_INVALID;
    if (n == 0) return W4A4_OK;
    if (!Y || !H) return W4A4_ERR_INVALID;
    if (misaligned(Y) || misaligned(H)) return W4A4_ERR_ALIGN;
    return dev_status(launch_gelu(Y, n, H, (hipStream_t)stream));
}

}  // extern "C"

// The fixed workspace of w4a4_linear_noalloc.  Each device holds its own copy of this
// array; in host code its name is only a stand-in, so every host use goes through the
// device address looked up below.
static __device__ __align__(256) uint8_t scratch[W4A4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device with
// that device current.
int scratch_on_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A4_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A4_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A4_OK;
}

}  // namespace

extern "C" int w4a4_linear_noalloc(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, float* Y,
                                   void* stream) {
    if (T < 0) return W4A4_ERR_INVALID;
    int st = check_desc(desc);
    if (st) return st;
    if (T == 0) return W4A4_OK;
    if (ws_layout(T, desc).total > W4A4_NOALLOC_SCRATCH_BYTES) return W4A4_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st) return st;
    return linear_into(X, x_dtype, T, desc, Y, false, ws, W4A4_NOALLOC_SCRATCH_BYTES, stream);
}
