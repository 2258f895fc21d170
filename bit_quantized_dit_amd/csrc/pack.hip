// Offline weight fold + split + block pack ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.2: s folded into the master
// weights; sec. 3.3: outlier rows O kept in high precision; sec. 3.4: block-wise
// scales after the fold and the column extraction, 32x32 tiles or 128x1 K-major
// stripes, exponent stored beside the 4-bit payload).
//
// W arrives in nn.Linear orientation [d_out][d_in] (K contiguous).  The folded J
// weights w'[n][p] = fl32(s[J[p]] * W[n][J[p]]) are never materialised: pass 1
// computes one E8M0 code per scale group, pass 2 recomputes w' per 32-element
// chunk and writes 16 bytes of nibbles.  Both passes are gathers through J and run
// once per layer, so they favour plainness over bandwidth.
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
    if (d.k_pad > 0) {
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
