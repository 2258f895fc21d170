// Fused activation prep ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME
// 2026 Challenge)", sec. 3.2: activations are divided by s and then quantized;
// sec. 3.3: the static outlier columns O bypass quantization).
//
// One workgroup streams whole token rows (persistent over rows).  Per row:
//   phase 1  each thread reads 8 consecutive input columns (one 16-byte load for
//            bf16, two for fp32) and, through the column map, either writes
//            x / s_j (IEEE binary32 division) into the LDS copy of the
//            J-compacted row, or writes bf16(x) into X_O.  The column map and s
//            for the thread's columns stay in registers across rows.
//   phase 2  each thread takes 8 consecutive compacted positions (two 16-byte LDS
//            reads); four lanes form one 32-block, their |x| maxima meet through
//            two xor-shuffles, and every lane emits 8 nibbles as one 32-bit store
//            (lane 0 of the four also stores the E8M0 byte, into the step-major
//            scale array [k_pad/128][T][4] that the GEMM streams contiguously).
// HBM traffic is the algorithmic minimum: X read once, A_q/A_s/X_O written once.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

constexpr int AP_THREADS = 512;
constexpr int AP_COLS_PER_PASS = AP_THREADS * 8;

template <typename XT>
struct Vec8;
template <>
struct Vec8<uint16_t> {
    __device__ static void load(const uint16_t* p, float* v) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
};
template <>
struct Vec8<float> {
    __device__ static void load(const float* p, float* v) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ static float load1(const float* p) { return *p; }
};

__device__ __forceinline__ void route(float x, int32_t m, float s, float* row, uint16_t* xo_row) {
    if (m >= 0) row[m] = x / s;
    else xo_row[-m - 1] = bf16_rne(x);
}

// Phase 2 for one token row held in LDS.
// as_t points at this token's scale slot of step 0 in the step-major A_s
// ([k_pad/128][T][4]); step kb's slot is as_t + kb * as_step.
__device__ __forceinline__ void quantize_row(const float* row, int64_t k_pad, uint8_t* aq_row,
                                             uint8_t* as_t, int64_t as_step) {
    for (int64_t p0 = (int64_t)threadIdx.x * 8; p0 < k_pad; p0 += AP_COLS_PER_PASS) {
        const float4 a = *reinterpret_cast<const float4*>(row + p0);
        const float4 b = *reinterpret_cast<const float4*>(row + p0 + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = abs_bits(v[i]);
            m = q > m ? q : m;
        }
        uint32_t o = (uint32_t)__shfl_xor((int)m, 1);
        m = o > m ? o : m;
        o = (uint32_t)__shfl_xor((int)m, 2);
        m = o > m ? o : m;
        const uint32_t code = e8m0_from_absbits(m);
        uint32_t word = 0;
        if (code != 0xFFu) {
            const float inv = e8m0_inverse(code);
#pragma unroll
            for (int i = 0; i < 8; ++i) word |= e2m1_nibble(v[i], inv) << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(aq_row + p0 / 2) = word;
        if ((threadIdx.x & 3) == 0) as_t[(p0 / 128) * as_step + (p0 / 32) % 4] = (uint8_t)code;
    }
}

// NCH > 0: d_in % 8 == 0, X 16-byte aligned, d_in <= NCH * AP_COLS_PER_PASS; the
// column map and s of the thread's columns are cached in registers.
template <typename XT, int NCH>
__global__ __launch_bounds__(AP_THREADS) void actprep_kernel(
    const XT* __restrict__ X, int64_t T, int64_t d_in, const int32_t* __restrict__ colmap,
    const float* __restrict__ s, int64_t k_j, int64_t k_pad, int32_t k, int64_t k_ld,
    uint8_t* __restrict__ Aq, uint8_t* __restrict__ As, uint16_t* __restrict__ XO) {
    extern __shared__ float row[];
    for (int64_t p = k_j + threadIdx.x; p < k_pad; p += AP_THREADS) row[p] = 0.0f;

    int32_t cm[NCH > 0 ? NCH : 1][8];
    float sv[NCH > 0 ? NCH : 1][8];
    if constexpr (NCH > 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t j0 = (int64_t)c * AP_COLS_PER_PASS + threadIdx.x * 8;
            if (j0 < d_in) {
                const int4 m0 = reinterpret_cast<const int4*>(colmap + j0)[0];
                const int4 m1 = reinterpret_cast<const int4*>(colmap + j0)[1];
                const float4 s0 = reinterpret_cast<const float4*>(s + j0)[0];
                const float4 s1 = reinterpret_cast<const float4*>(s + j0)[1];
                cm[c][0] = m0.x; cm[c][1] = m0.y; cm[c][2] = m0.z; cm[c][3] = m0.w;
                cm[c][4] = m1.x; cm[c][5] = m1.y; cm[c][6] = m1.z; cm[c][7] = m1.w;
                sv[c][0] = s0.x; sv[c][1] = s0.y; sv[c][2] = s0.z; sv[c][3] = s0.w;
                sv[c][4] = s1.x; sv[c][5] = s1.y; sv[c][6] = s1.z; sv[c][7] = s1.w;
            }
        }
    }

    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const XT* xr = X + t * d_in;
        uint16_t* xo_row = XO + t * k_ld;
        if constexpr (NCH > 0) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int64_t j0 = (int64_t)c * AP_COLS_PER_PASS + threadIdx.x * 8;
                if (j0 < d_in) {
                    float v[8];
                    Vec8<XT>::load(xr + j0, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) route(v[e], cm[c][e], sv[c][e], row, xo_row);
                }
            }
        } else {
            for (int64_t j = threadIdx.x; j < d_in; j += AP_THREADS)
                route(Vec8<XT>::load1(xr + j), colmap[j], s[j], row, xo_row);
        }
        for (int64_t i = k + threadIdx.x; i < k_ld; i += AP_THREADS) xo_row[i] = 0;
        __syncthreads();
        quantize_row(row, k_pad, Aq + t * (k_pad / 2), As + t * 4, T * 4);
        __syncthreads();
    }
}

template <typename XT>
static hipError_t launch_typed(const XT* X, int64_t T, const w4a4_packed& d, uint8_t* Aq, uint8_t* As,
                               uint16_t* XO, hipStream_t st) {
    const size_t lds = (size_t)(d.k_pad > 0 ? d.k_pad : 1) * sizeof(float);
    const int64_t grid64 = T < 2048 ? T : 2048;
    const unsigned grid = (unsigned)grid64;
    const bool vec = (d.d_in % 8 == 0) && (((uintptr_t)X & 15u) == 0);
    const int nch = (int)((d.d_in + AP_COLS_PER_PASS - 1) / AP_COLS_PER_PASS);
#define W4A4_AP_CALL(N)                                                                              \
    if (lds > 65536) {                                                                               \
        hipError_t e = hipFuncSetAttribute((const void*)actprep_kernel<XT, N>,                       \
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);    \
        if (e != hipSuccess) return e;                                                               \
    }                                                                                                \
    actprep_kernel<XT, N><<<grid, AP_THREADS, lds, st>>>(X, T, d.d_in, d.colmap, d.s, d.k_j, d.k_pad, \
                                                         d.k, d.k_ld, Aq, As, XO)
    if (vec && nch <= 1) { W4A4_AP_CALL(1); }
    else if (vec && nch == 2) { W4A4_AP_CALL(2); }
    else if (vec && nch <= 4) { W4A4_AP_CALL(4); }
    else { W4A4_AP_CALL(0); }
#undef W4A4_AP_CALL
    return hipGetLastError();
}

hipError_t launch_actprep(const void* X, int x_dtype, int64_t T, const w4a4_packed& d, uint8_t* Aq,
                          uint8_t* As, uint16_t* XO, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (x_dtype == W4A4_X_BF16) return launch_typed<uint16_t>((const uint16_t*)X, T, d, Aq, As, XO, st);
    return launch_typed<float>((const float*)X, T, d, Aq, As, XO, st);
}

}  // namespace w4a4
