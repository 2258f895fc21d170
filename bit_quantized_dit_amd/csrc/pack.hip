// Offline weight fold + split + block pack ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.2: s folded into the master
// weights; sec. 3.3: outlier rows O kept in high precision; sec. 3.4: block-wise
// scales after the fold and the column extraction, 32x32 tiles or 128x1 K-major
// stripes, exponent stored beside the 4-bit payload).
//
// W arrives in nn.Linear orientation [d_out][d_in] (K contiguous).  The folded J
// weights w'[p] = fl32(s[J[p]] * W[n][J[p]]) of one row at a time are staged in LDS at
// their compacted positions (a coalesced pass over the row), then each lane quantizes
// 8 consecutive positions.  Row-local layouts (1x32, 128x1 stripes) take one workgroup
// per row; 32x32 tiles, whose groups span 32 rows, one workgroup per 32-row strip with
// a pass for the tile maxima and a pass for the codes.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

// Byte offset of the 16-byte chunk c (0..3) of row n, 128-code step kb, in the tiled
// copy: 1 KiB per (16-row block, step), row n % 16 at 64-byte stride, chunk c at
// chunk position c ^ ((n % 16) / 4) (the order the GEMM's LDS ring uses).
__device__ __forceinline__ int64_t tiled_chunk(int64_t n, int64_t kb, int64_t nkb, int c) {
    const int r = (int)(n & 15);
    return (((n >> 4) * nkb + kb) << 10) + (r << 6) + ((c ^ (r >> 2)) << 4);
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

// 32x32 tiles: one 256-lane workgroup per strip of 32 rows (rows 32t .. 32t+31).
// Pass A stages each row's folded weights in LDS, as pack_rows_kernel does, and folds
// its 32-block maxima into a running maximum per block (LDS, one quad per block, a
// barrier between rows), which after the strip's rows is the tile maximum; pass B
// stages each row again and quantizes it with its tile's code.  Rows past d_out take
// no part in the maxima and get zero codes in the tiled copy up to roundup(d_out, 16).
__global__ __launch_bounds__(256) void pack_tiles_kernel(const float* __restrict__ W, const float* __restrict__ s,
                                                         const int32_t* __restrict__ colmap, int64_t d_in,
                                                         int64_t d_out, int64_t k_j, int64_t k_pad,
                                                         uint8_t* __restrict__ Bq, uint8_t* __restrict__ Bqt,
                                                         uint8_t* __restrict__ Bs, uint8_t* __restrict__ Bs_rows) {
    extern __shared__ float wrow[];
    uint32_t* const gmax = reinterpret_cast<uint32_t*>(wrow + (k_pad + k_pad / 8));   // [k_pad / 32]
    const int64_t strip = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nkb128 = k_pad / 128, ntile = (d_out + 31) / 32;
    const int64_t r_end = (strip * 32 + 32 < d_out ? strip * 32 + 32 : d_out);
    for (int64_t kb = tid; kb < k_pad / 32; kb += 256) gmax[kb] = 0u;
    auto stage = [&](int64_t n) {
        const float* wr = W + n * d_in;
        for (int64_t j = tid; j < d_in; j += 256) {
            const int32_t m = colmap[j];
            if (m >= 0) wrow[pack_lds_pos(m)] = s[j] * wr[j];   // one binary32 multiply
        }
        for (int64_t p = k_j + tid; p < k_pad; p += 256) wrow[pack_lds_pos(p)] = 0.0f;
    };
    auto read8 = [&](int64_t p0, float* v) {
        const float* src = wrow + pack_lds_pos(p0);
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
    // pass A: tile maxima
    for (int64_t n = strip * 32; n < r_end; ++n) {
        __syncthreads();   // the previous row's reads of wrow (and the gmax clear) are done
        stage(n);
        __syncthreads();
        for (int64_t p0 = (int64_t)tid * 8; p0 < k_pad; p0 += 256 * 8) {
            float v[8];
            read8(p0, v);
            const float m01 = __builtin_elementwise_maximum(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
            const float m23 = __builtin_elementwise_maximum(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]));
            const float m45 = __builtin_elementwise_maximum(__builtin_fabsf(v[4]), __builtin_fabsf(v[5]));
            const float m67 = __builtin_elementwise_maximum(__builtin_fabsf(v[6]), __builtin_fabsf(v[7]));
            uint32_t mb = __float_as_uint(__builtin_elementwise_maximum(__builtin_elementwise_maximum(m01, m23),
                                                                        __builtin_elementwise_maximum(m45, m67)));
            uint32_t o = (uint32_t)__shfl_xor((int)mb, 1);
            mb = o > mb ? o : mb;
            o = (uint32_t)__shfl_xor((int)mb, 2);
            mb = o > mb ? o : mb;
            if ((p0 & 31) == 0 && mb > gmax[p0 >> 5]) gmax[p0 >> 5] = mb;
        }
    }
    __syncthreads();
    for (int64_t kb = tid; kb < k_pad / 32; kb += 256) {
        const uint32_t code = e8m0_from_absbits(gmax[kb]);
        gmax[kb] = code;
        Bs[kb * ntile + strip] = (uint8_t)code;
    }
    // pass B: codes, rows past d_out (up to the tiled copy's 16-row granule) as zeros
    const int64_t r_tiles = strip * 32 + 32 < (d_out + 15) / 16 * 16 ? strip * 32 + 32 : (d_out + 15) / 16 * 16;
    for (int64_t n = strip * 32; n < r_tiles; ++n) {
        __syncthreads();   // codes written (first row) / the previous row's reads done
        if (n < d_out) stage(n);
        __syncthreads();
        for (int64_t p0 = (int64_t)tid * 8; p0 < k_pad; p0 += 256 * 8) {
            uint32_t w = 0;
            const uint32_t code = gmax[p0 >> 5];
            if (n < d_out) {
                float v[8];
                read8(p0, v);
                const float scale = __uint_as_float(__builtin_elementwise_max(code << 23, 0x00400000u));
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
                w = code == 0xFFu ? 0u : w;
                *reinterpret_cast<uint32_t*>(Bq + n * (k_pad / 2) + (p0 >> 1)) = w;
                if ((p0 & 31) == 0) Bs_rows[((p0 >> 7) * d_out + n) * 4 + ((p0 >> 5) & 3)] = (uint8_t)code;
            }
            *reinterpret_cast<uint32_t*>(Bqt + tiled_chunk(n, p0 >> 7, nkb128, (int)((p0 >> 5) & 3)) +
                                         ((p0 & 31) >> 1)) = w;
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
        // 32x32 tiles
        const size_t lds = (size_t)(d.k_pad + d.k_pad / 8) * sizeof(float) + (size_t)(d.k_pad / 32) * 4;
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute((const void*)pack_tiles_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        const int64_t strips = (d.d_out + 31) / 32;
        if (strips > 0x7FFFFFFF) return hipErrorInvalidValue;
        pack_tiles_kernel<<<(unsigned)strips, 256, lds, st>>>(W, d.s, d.colmap, d.d_in, d.d_out, d.k_j, d.k_pad,
                                                             (uint8_t*)d.B_q, (uint8_t*)d.B_q_tiles,
                                                             (uint8_t*)d.B_s, (uint8_t*)d.B_s_rows);
        const hipError_t e = hipGetLastError();
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
