// Dual-branch W4A4 GEMM on gfx950 ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.3):
//
//   Y[t][n] = sum_p Q(X_J / s_J)[t][p] Q(s_J * W_J)[n][p]      (MXFP4 x MXFP4)
//           + sum_i X_O[t][i] W_O[n][i]                         (BF16 x BF16)
//
// Both branches accumulate into the same fp32 registers:
//   - the J branch with v_mfma_scale_f32_16x16x128_f8f6f4 in FP4 (E2M1) mode, whose
//     per-lane E8M0 scale operand applies 2^(c-127) per 32-element K block to each
//     operand, i.e. exactly the MXFP4 block scaling;
//   - the O branch with v_mfma_f32_16x16x32_bf16.
// Operand roles: src0 = weight rows (16 features), src1 = activation rows (16
// tokens), so each lane ends up holding 4 consecutive features of one token and
// stores them as one float4.
//
// Tiling: a 256-thread workgroup (4 wavefronts, 2 x 2) owns a 128-token x
// 128-feature output tile; each wavefront a 64 x 64 sub-tile (4 x 4 MFMA tiles).
// Per 128-K step the workgroup stages 128 rows x 64 bytes of A and of B in LDS
// (16-byte chunks XOR-swizzled by row so that fragment reads are bank-conflict
// free) plus one 32-bit word of four E8M0 codes per row; weight scales of the
// tile and stripe layouts are expanded to that per-row word while staging.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int G_THREADS = 256;
constexpr int BT = 128;          // tokens per workgroup tile
constexpr int BF = 128;          // features per workgroup tile
constexpr int FT = 4;            // 16-token MFMA tiles per wavefront
constexpr int FF = 4;            // 16-feature MFMA tiles per wavefront
constexpr int ROW_BYTES = 64;    // 128 FP4 codes per row per K step

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROW_BYTES + ((chunk ^ ((row >> 2) & 3)) << 4); }

__device__ __forceinline__ uint32_t weight_scale_word(const uint8_t* __restrict__ Bs, int64_t n, int64_t kb,
                                                      int64_t k_pad, int64_t N, int layout) {
    if (layout == W4A4_WS_1X32) return *reinterpret_cast<const uint32_t*>(Bs + n * (k_pad / 32) + kb * 4);
    if (layout == W4A4_WS_128X1_STRIPE) return 0x01010101u * (uint32_t)Bs[n * (k_pad / 128) + kb];
    const int64_t ntile = (N + 31) / 32;
    const int64_t base = (kb * 4) * ntile + n / 32;
    return (uint32_t)Bs[base] | ((uint32_t)Bs[base + ntile] << 8) | ((uint32_t)Bs[base + 2 * ntile] << 16) |
           ((uint32_t)Bs[base + 3 * ntile] << 24);
}

__global__ __launch_bounds__(G_THREADS) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ As, const uint16_t* __restrict__ XO,
    int64_t T, const uint8_t* __restrict__ Bq, const uint8_t* __restrict__ Bs,
    const uint16_t* __restrict__ WO, int64_t N, int64_t k_pad, int64_t k_ld, int layout,
    float* __restrict__ Y, int vec_store) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[BT * ROW_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BF * ROW_BYTES];
    __shared__ uint32_t sAs[BT];
    __shared__ uint32_t sBs[BF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wt = wave & 1;     // token half of the tile
    const int wf = wave >> 1;    // feature half of the tile
    const int64_t t0 = (int64_t)blockIdx.x * BT;
    const int64_t f0 = (int64_t)blockIdx.y * BF;
    const int l16 = lane & 15;
    const int lc = lane >> 4;    // K chunk (32 codes) this lane feeds

    v4f acc[FF][FT];
#pragma unroll
    for (int i = 0; i < FF; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int64_t a_ld = k_pad / 2;
    const int64_t nkb = k_pad / 128;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        // ---- stage A and B codes: thread -> (row, 16-byte chunk)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = (tid >> 2) + 64 * h;
            const int c = tid & 3;
            const int64_t t = t0 + r;
            uint4 va = make_uint4(0, 0, 0, 0);
            if (t < T) va = *reinterpret_cast<const uint4*>(Aq + t * a_ld + kb * 64 + c * 16);
            *reinterpret_cast<uint4*>(sA + swz(r, c)) = va;
            const int64_t n = f0 + r;
            uint4 vb = make_uint4(0, 0, 0, 0);
            if (n < N) vb = *reinterpret_cast<const uint4*>(Bq + n * a_ld + kb * 64 + c * 16);
            *reinterpret_cast<uint4*>(sB + swz(r, c)) = vb;
        }
        if (tid < BT) {
            const int64_t t = t0 + tid;
            sAs[tid] = t < T ? *reinterpret_cast<const uint32_t*>(As + t * (k_pad / 32) + kb * 4) : 0u;
        } else {
            const int r = tid - BT;
            const int64_t n = f0 + r;
            sBs[r] = n < N ? weight_scale_word(Bs, n, kb, k_pad, N, layout) : 0u;
        }
        __syncthreads();

        // ---- fragments and MFMAs
        v8i af[FT], bfr[FF];
        int as_[FT], bs_[FF];
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int r = wt * 64 + j * 16 + l16;
            const uint4 q = *reinterpret_cast<const uint4*>(sA + swz(r, lc));
            af[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            as_[j] = (int)(sAs[r] >> (8 * lc));
        }
#pragma unroll
        for (int i = 0; i < FF; ++i) {
            const int r = wf * 64 + i * 16 + l16;
            const uint4 q = *reinterpret_cast<const uint4*>(sB + swz(r, lc));
            bfr[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            bs_[i] = (int)(sBs[r] >> (8 * lc));
        }
#pragma unroll
        for (int i = 0; i < FF; ++i)
#pragma unroll
            for (int j = 0; j < FT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bfr[i], af[j], acc[i][j], 4, 4, 0, bs_[i], 0, as_[j]);
        __syncthreads();
    }

    // ---- outlier branch: bf16 x bf16 into the same accumulators
    for (int64_t kk = 0; kk < k_ld; kk += 32) {
        v8bf xa[FT], wb[FF];
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int64_t t = t0 + wt * 64 + j * 16 + l16;
            uint4 q = make_uint4(0, 0, 0, 0);
            if (t < T) q = *reinterpret_cast<const uint4*>(XO + t * k_ld + kk + 8 * lc);
            xa[j] = __builtin_bit_cast(v8bf, q);
        }
#pragma unroll
        for (int i = 0; i < FF; ++i) {
            const int64_t n = f0 + wf * 64 + i * 16 + l16;
            uint4 q = make_uint4(0, 0, 0, 0);
            if (n < N) q = *reinterpret_cast<const uint4*>(WO + n * k_ld + kk + 8 * lc);
            wb[i] = __builtin_bit_cast(v8bf, q);
        }
#pragma unroll
        for (int i = 0; i < FF; ++i)
#pragma unroll
            for (int j = 0; j < FT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], xa[j], acc[i][j], 0, 0, 0);
    }

    // ---- epilogue: lane holds features 4*lc..4*lc+3 of token l16 in each tile
#pragma unroll
    for (int j = 0; j < FT; ++j) {
        const int64_t t = t0 + wt * 64 + j * 16 + l16;
        if (t >= T) continue;
#pragma unroll
        for (int i = 0; i < FF; ++i) {
            const int64_t n = f0 + wf * 64 + i * 16 + 4 * lc;
            float* dst = Y + t * N + n;
            if (vec_store && n + 3 < N) {
                *reinterpret_cast<v4f*>(dst) = acc[i][j];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) dst[r] = acc[i][j][r];
            }
        }
    }
}

hipError_t launch_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T,
                       const w4a4_packed& d, float* Y, hipStream_t st) {
    if (T <= 0 || d.d_out <= 0) return hipSuccess;
    const int64_t gx = (T + BT - 1) / BT;
    const int64_t gy = (d.d_out + BF - 1) / BF;
    if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidValue;
    const int vec_store = (d.d_out % 4 == 0) && (((uintptr_t)Y & 15u) == 0);
    gemm_w4a4_kernel<<<dim3((unsigned)gx, (unsigned)gy), G_THREADS, 0, st>>>(
        Aq, As, XO, T, d.B_q, d.B_s, d.W_O, d.d_out, d.k_pad, d.k_ld, d.layout, Y, vec_store);
    return hipGetLastError();
}

}  // namespace w4a4
