// Offline weight fold + split + block pack ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.2: s folded into the master
// weights; sec. 3.3: outlier rows O kept in high precision; sec. 3.4: block-wise
// scales after the fold and the column extraction, 32x32 tiles or 128x1 K-major
// stripes, exponent stored beside the 4-bit payload).
//
// W arrives in nn.Linear orientation [d_out][d_in] (K contiguous).  For the row-local
// layouts (1x32, 128x1 stripes) one workgroup packs one row: the folded J weights
// w'[p] = fl32(s[J[p]] * W[n][J[p]]) are staged in LDS at their compacted positions
// (a coalesced pass over the row), then each lane quantizes 8 consecutive positions.
// For 32x32 tiles, whose groups span 32 rows, pass 1 computes one E8M0 code per group
// and pass 2 recomputes w' per 32-element chunk and writes 16 bytes of nibbles; both
// are gathers through J that favour plainness over bandwidth.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

__device__ __forceinline__ float folded(const float* __restrict__ W, const float* __restrict__ s,
                                        const int32_t* __restrict__ J, int64_t d_in, int64_t k_j,
                                        int64_t n, int64_t p) {
    if (p >= k_j) return 0.0f;
    const int32_t j = J[p];
    return s[j] * W[n * d_in + j];   // one binary32 multiply (no contraction possible)
}

// Pass 1: one thread per scale group.
__global__ __launch_bounds__(256) void pack_scales_kernel(const float* __restrict__ W,
                                                          const float* __restrict__ s,
                                                          const int32_t* __restrict__ J, int64_t d_in,
                                                          int64_t d_out, int64_t k_j, int64_t k_pad,
                                                          int layout, uint8_t* __restrict__ Bs) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t m = 0;
    if (layout == W4A4_WS_1X32 || layout == W4A4_WS_128X1_STRIPE) {
        const int64_t gk = layout == W4A4_WS_1X32 ? 32 : 128;
        const int64_t per_row = k_pad / gk;
        if (g >= d_out * per_row) return;
        const int64_t n = g / per_row, q = g % per_row;
        for (int64_t i = 0; i < gk; ++i) {
            const uint32_t a = abs_bits(folded(W, s, J, d_in, k_j, n, q * gk + i));
            m = a > m ? a : m;
        }
    } else {
        const int64_t ntile = (d_out + 31) / 32;
        if (g >= (k_pad / 32) * ntile) return;
        const int64_t kb = g / ntile, nt = g % ntile;
        for (int64_t n = nt * 32; n < nt * 32 + 32 && n < d_out; ++n)
            for (int64_t i = 0; i < 32; ++i) {
                const uint32_t a = abs_bits(folded(W, s, J, d_in, k_j, n, kb * 32 + i));
                m = a > m ? a : m;
            }
    }
    Bs[g] = (uint8_t)e8m0_from_absbits(m);
}

// Byte offset of the 16-byte chunk c (0..3) of row n, 128-code step kb, in the tiled
// copy: 1 KiB per (16-row block, step), row n % 16 at 64-byte stride, chunk c at
// chunk position c ^ ((n % 16) / 4) (the order the GEMM's LDS ring uses).
__device__ __forceinline__ int64_t tiled_chunk(int64_t n, int64_t kb, int64_t nkb, int c) {
    const int r = (int)(n & 15);
    return (((n >> 4) * nkb + kb) << 10) + (r << 6) + ((c ^ (r >> 2)) << 4);
}

// Pass 2: one thread per (row n, 32-block kb): 32 codes -> 16 bytes, written to the
// canonical B_q and to the tiled copy (rows d_out .. roundup(d_out, 16) are zero there).
__global__ __launch_bounds__(256) void pack_codes_kernel(const float* __restrict__ W,
                                                         const float* __restrict__ s,
                                                         const int32_t* __restrict__ J, int64_t d_in,
                                                         int64_t d_out, int64_t k_j, int64_t k_pad,
                                                         int layout, const uint8_t* __restrict__ Bs,
                                                         uint8_t* __restrict__ Bq, uint8_t* __restrict__ Bqt) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nkb = k_pad / 32;
    const int64_t rows = (d_out + 15) / 16 * 16;
    if (g >= rows * nkb) return;
    const int64_t n = g / nkb, kb = g % nkb;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    if (n < d_out) {
        uint32_t code;
        if (layout == W4A4_WS_1X32) code = Bs[n * nkb + kb];
        else if (layout == W4A4_WS_128X1_STRIPE) code = Bs[n * (k_pad / 128) + kb / 4];
        else code = Bs[kb * ((d_out + 31) / 32) + n / 32];
        if (code != 0xFFu) {
            const float inv = e8m0_inverse(code);
            for (int i = 0; i < 32; ++i) {
                const float w = folded(W, s, J, d_in, k_j, n, kb * 32 + i);
                words[i >> 3] |= e2m1_nibble(w, inv) << (4 * (i & 7));
            }
        }
        *reinterpret_cast<uint4*>(Bq + n * (k_pad / 2) + kb * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    }
    *reinterpret_cast<uint4*>(Bqt + tiled_chunk(n, kb / 4, k_pad / 128, (int)(kb % 4))) =
        make_uint4(words[0], words[1], words[2], words[3]);
}

// Step-major per-row copy of the weight scales: for each 128-code step kb, row n's
// four 32-block codes at Bs_rows[(kb*d_out + n)*4 + q], derived from the canonical
// codes of any layout.  One GEMM workgroup then reads a step's scales for its 256
// rows as one contiguous 1 KiB run instead of 256 scattered words.
__global__ __launch_bounds__(256) void pack_row_scales_kernel(const uint8_t* __restrict__ Bs, int64_t d_out,
                                                              int64_t k_pad, int layout,
                                                              uint8_t* __restrict__ Bs_rows) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nkb = k_pad / 32;
    if (g >= d_out * nkb) return;
    const int64_t n = g / nkb, kb = g % nkb;
    uint8_t c;
    if (layout == W4A4_WS_1X32) c = Bs[n * nkb + kb];
    else if (layout == W4A4_WS_128X1_STRIPE) c = Bs[n * (k_pad / 128) + kb / 4];
    else c = Bs[kb * ((d_out + 31) / 32) + n / 32];
    Bs_rows[((kb / 4) * d_out + n) * 4 + (kb % 4)] = c;
}

// LDS word of compacted position p: 16 bytes of padding after every 32 positions, so
// that the 16-byte reads of consecutive lanes (32 bytes apart) spread over the banks.
__device__ __forceinline__ int32_t pack_lds_pos(int64_t p) { return (int32_t)(p + ((p >> 5) << 2)); }

// Row-local layouts: one 256-lane workgroup per row n of roundup(d_out, 16) (rows past
// d_out only zero their part of the tiled copy).  Lane i takes positions 8i + 2048m:
// the block maximum over |w'| (IEEE maximum, so a NaN propagates; a 32-block is a quad
// of lanes, a 128-stripe 16 lanes), the E8M0 code from its exponent field, and the
// nibbles from four scaled FP4 conversions (nearest even, saturating at 6, divisor
// 2^E; a NaN/Inf group gets zero nibbles).  Writes B_q, its tiled copy, B_s and the
// step-major B_s_rows directly.
__global__ __launch_bounds__(256) void pack_rows_kernel(const float* __restrict__ W, const float* __restrict__ s,
                                                        const int32_t* __restrict__ colmap, int64_t d_in,
                                                        int64_t d_out, int64_t k_j, int64_t k_pad, int layout,
                                                        uint8_t* __restrict__ Bq, uint8_t* __restrict__ Bqt,
                                                        uint8_t* __restrict__ Bs, uint8_t* __restrict__ Bs_rows) {
    extern __shared__ float wrow[];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nkb128 = k_pad / 128;
    if (n >= d_out) {
        for (int64_t p0 = (int64_t)tid * 8; p0 < k_pad; p0 += 256 * 8)
            *reinterpret_cast<uint32_t*>(Bqt + tiled_chunk(n, p0 >> 7, nkb128, (int)((p0 >> 5) & 3)) +
                                         ((p0 & 31) >> 1)) = 0u;
        return;
    }
    const float* wr = W + n * d_in;
    for (int64_t j = tid; j < d_in; j += 256) {
        const int32_t m = colmap[j];
        if (m >= 0) wrow[pack_lds_pos(m)] = s[j] * wr[j];   // one binary32 multiply
    }
    for (int64_t p = k_j + tid; p < k_pad; p += 256) wrow[pack_lds_pos(p)] = 0.0f;
    __syncthreads();
    const bool stripe = layout == W4A4_WS_128X1_STRIPE;
    for (int64_t p0 = (int64_t)tid * 8; p0 < k_pad; p0 += 256 * 8) {
        const float* src = wrow + pack_lds_pos(p0);
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const float m01 = __builtin_elementwise_maximum(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
        const float m23 = __builtin_elementwise_maximum(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]));
        const float m45 = __builtin_elementwise_maximum(__builtin_fabsf(v[4]), __builtin_fabsf(v[5]));
        const float m67 = __builtin_elementwise_maximum(__builtin_fabsf(v[6]), __builtin_fabsf(v[7]));
        uint32_t mb = __float_as_uint(__builtin_elementwise_maximum(__builtin_elementwise_maximum(m01, m23),
                                                                    __builtin_elementwise_maximum(m45, m67)));
        // the 32-block: lanes 4q .. 4q+3
        uint32_t o = (uint32_t)__shfl_xor((int)mb, 1);
        mb = o > mb ? o : mb;
        o = (uint32_t)__shfl_xor((int)mb, 2);
        mb = o > mb ? o : mb;
        if (stripe) {   // the 128-stripe: lanes 16r .. 16r+15
            o = (uint32_t)__shfl_xor((int)mb, 4);
            mb = o > mb ? o : mb;
            o = (uint32_t)__shfl_xor((int)mb, 8);
            mb = o > mb ? o : mb;
        }
        const uint32_t code = e8m0_from_absbits(mb);
        const float scale = __uint_as_float(__builtin_elementwise_max(code << 23, 0x00400000u));
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
        w = code == 0xFFu ? 0u : w;
        *reinterpret_cast<uint32_t*>(Bq + n * (k_pad / 2) + (p0 >> 1)) = w;
        *reinterpret_cast<uint32_t*>(Bqt + tiled_chunk(n, p0 >> 7, nkb128, (int)((p0 >> 5) & 3)) + ((p0 & 31) >> 1)) = w;
        if ((p0 & 31) == 0) {
            Bs_rows[((p0 >> 7) * d_out + n) * 4 + ((p0 >> 5) & 3)] = (uint8_t)code;
            if (!stripe) Bs[n * (k_pad / 32) + (p0 >> 5)] = (uint8_t)code;
            else if ((p0 & 127) == 0) Bs[n * nkb128 + (p0 >> 7)] = (uint8_t)code;
        }
    }
}

// Outlier rows in bf16, raw (unsmoothed), zero padded to k_ld.
__global__ __launch_bounds__(256) void pack_outliers_kernel(const float* __restrict__ W,
                                                            const int32_t* __restrict__ O, int64_t d_in,
                                                            int64_t d_out, int32_t k, int64_t k_ld,
                                                            uint16_t* __restrict__ WO) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= d_out * k_ld) return;
    const int64_t n = g / k_ld, i = g % k_ld;
    WO[g] = i < k ? bf16_rne(W[n * d_in + O[i]]) : (uint16_t)0;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_pack(const float* W, const w4a4_packed& d, hipStream_t st) {
    if (d.k_pad > 0 && (d.layout == W4A4_WS_1X32 || d.layout == W4A4_WS_128X1_STRIPE)) {
        const size_t lds = (size_t)(d.k_pad + d.k_pad / 8) * sizeof(float);
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute((const void*)pack_rows_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        const int64_t rows = (d.d_out + 15) / 16 * 16;
        if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
        pack_rows_kernel<<<(unsigned)rows, 256, lds, st>>>(W, d.s, d.colmap, d.d_in, d.d_out, d.k_j, d.k_pad,
                                                           d.layout, (uint8_t*)d.B_q, (uint8_t*)d.B_q_tiles,
                                                           (uint8_t*)d.B_s, (uint8_t*)d.B_s_rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (d.k_pad > 0) {
        int64_t groups;
        if (d.layout == W4A4_WS_1X32) groups = d.d_out * (d.k_pad / 32);
        else if (d.layout == W4A4_WS_128X1_STRIPE) groups = d.d_out * (d.k_pad / 128);
        else groups = (d.k_pad / 32) * ((d.d_out + 31) / 32);
        pack_scales_kernel<<<blocks_for(groups), 256, 0, st>>>(W, d.s, d.J, d.d_in, d.d_out, d.k_j,
                                                               d.k_pad, d.layout, (uint8_t*)d.B_s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        pack_codes_kernel<<<blocks_for((d.d_out + 15) / 16 * 16 * (d.k_pad / 32)), 256, 0, st>>>(
            W, d.s, d.J, d.d_in, d.d_out, d.k_j, d.k_pad, d.layout, d.B_s, (uint8_t*)d.B_q,
            (uint8_t*)d.B_q_tiles);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        pack_row_scales_kernel<<<blocks_for(d.d_out * (d.k_pad / 32)), 256, 0, st>>>(
            d.B_s, d.d_out, d.k_pad, d.layout, (uint8_t*)d.B_s_rows);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (d.k_ld > 0) {
        pack_outliers_kernel<<<blocks_for(d.d_out * d.k_ld), 256, 0, st>>>(W, d.O, d.d_in, d.d_out, d.k,
                                                                           d.k_ld, (uint16_t*)d.W_O);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace w4a4
