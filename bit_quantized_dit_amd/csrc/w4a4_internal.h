// Internal launchers shared between the C-ABI front end and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a4.h"

namespace w4a4 {

hipError_t launch_column_absmax(const void* X, int x_dtype, int64_t rows, int64_t cols,
                                uint32_t* out_bits, hipStream_t st);

hipError_t launch_pack(const float* W, const w4a4_packed& d, hipStream_t st);

hipError_t launch_actprep(const void* X, int x_dtype, int64_t T, const w4a4_packed& d,
                          uint8_t* Aq, uint8_t* As, uint16_t* XO, hipStream_t st);

// out: fp32 Y [T][d_out], or bf16 H = bf16(gelu_tanh(bf16(Y))) when gelu_bf16
// Destination of the FFN up projection's epilogue that quantizes for the down layer:
// the down layer's A_q / A_s / X_O (workspace order) and RN64(1 / s_j) of its J columns
// in compacted order.
struct QuantDst {
    uint8_t* aq;
    uint8_t* as;
    uint16_t* xo;
    const double* rinv;
    int64_t k_j, k_pad, k_ld;
    int32_t k;
};
// Down-layer preparation that the fused epilogue leaves to a separate pass: rinv from
// the down layer's s and J, zero codes and scales for the 32-blocks past the J columns
// (up to k_pad), zero X_O columns k .. k_ld-1.
hipError_t launch_ffn_prologue(const w4a4_packed& down, int64_t T, const QuantDst& q, hipStream_t st);
// The up projection with GELU and the down layer's activation quantization fused into
// the epilogue: the up layer's output feature f is the down layer's compacted J
// position f for f < k_j and its outlier slot f - k_j above.
hipError_t launch_gemm_quant(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T,
                             const w4a4_packed& up, const QuantDst& q, float* part, hipStream_t st);
hipError_t launch_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T,
                       const w4a4_packed& d, void* out, bool gelu_bf16, float* part, hipStream_t st);
// Split-K plan of the GEMM for T tokens and N outputs (host logic): tiles [0, full)
// run whole, each later tile as `split` K ranges whose fp32 partial sums take
// part_bytes of workspace (`part`, 256-byte aligned; unused and may be null when
// split == 1), or, with half set, as two 256 x 128 half tiles in a launch of their own.
struct GemmSplit {
    int64_t full;
    int32_t split;
    int32_t half;
    size_t part_bytes;
};
GemmSplit gemm_split_plan(int64_t T, int64_t N, int64_t k_pad, int64_t k_ld);

hipError_t launch_gelu(const float* Y, int64_t n, uint16_t* H, hipStream_t st);

// alpha / k search: the unquantized fp32 product Y = X W^T, and per-block sums of
// (Yq - Yr)^2 and Yr^2 (partials[2b], partials[2b + 1])
hipError_t launch_ref_linear(const void* X, int x_dtype, int64_t T, int64_t d_in, const float* W, int64_t d_out,
                             float* Y, hipStream_t st);
hipError_t launch_sq_err(const float* yq, const float* yr, int64_t n, double* partials, int blocks,
                         hipStream_t st);

// per-call outliers: top-k of the scores into O (ascending) and the column map, and
// the W_O gather from the bf16 copy of W
hipError_t launch_dyn_select(const uint32_t* colmax_bits, const float* s, int64_t d_in, int32_t k, int32_t* O,
                             int32_t* colmap, hipStream_t st);
// W_O[n][i] = W_t[O[i]][n] for i < k, zero for k <= i < k_ld (k_ld a multiple of 32)
hipError_t launch_dyn_gather(const uint16_t* W_t, const int32_t* O, int64_t d_in, int64_t d_out, int32_t k,
                             int64_t k_ld, uint16_t* WO, hipStream_t st);
// W_t[j][n] = bf16_rne(W[n][j]), W fp32 [d_out][d_in]
hipError_t launch_dyn_transpose(const float* W, int64_t d_in, int64_t d_out, uint16_t* W_t, hipStream_t st);

}  // namespace w4a4
