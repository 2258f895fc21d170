// Kernels of the layer-wise alpha / k search ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)": sec. 3.2 gives alpha in [0.5, 0.7] for the
// FFN up projection; sec. 4 lists per-layer alpha and k, and sec. 6 names tuning them
// per layer as the next step).  Each candidate (alpha, k) is scored by the relative
// Frobenius error of the quantized layer's output against the unquantized product on
// the calibration tokens; these two kernels give that reference product and the two
// sums of squares.  The candidates themselves run through the library's own
// calibration, pack and per-call kernels.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

namespace {

template <typename XT>
__device__ __forceinline__ float x_value(const XT* p);
template <>
__device__ __forceinline__ float x_value<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float x_value<float>(const float* p) { return *p; }

constexpr int RT = 64;   // output tile: 64 tokens x 64 features per 256-lane workgroup
constexpr int RK = 16;   // K slice staged in LDS per iteration

// Y[t][n] = sum_j X[t][j] W[n][j] in fp32 (sequential fused multiply-adds over j in
// slices of 16), X fp32 or bf16 [T][d_in], W fp32 [d_out][d_in].  Each lane owns a
// 4 x 4 block of outputs.  A plain LDS-tiled kernel: the reference is computed once
// per search, so it favours plainness over speed.
template <typename XT>
__global__ __launch_bounds__(256) void ref_linear_kernel(const XT* __restrict__ X, const float* __restrict__ W,
                                                         int64_t T, int64_t d_in, int64_t d_out,
                                                         float* __restrict__ Y) {
    __shared__ float xs[RK][RT + 1];
    __shared__ float ws[RK][RT + 1];
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int64_t t0 = (int64_t)blockIdx.y * RT, n0 = (int64_t)blockIdx.x * RT;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int64_t k0 = 0; k0 < d_in; k0 += RK) {
        for (int e = threadIdx.x; e < RT * RK; e += 256) {
            const int r = e / RK, c = e % RK;
            const int64_t t = t0 + r, n = n0 + r, kk = k0 + c;
            xs[c][r] = (t < T && kk < d_in) ? x_value<XT>(X + t * d_in + kk) : 0.0f;
            ws[c][r] = (n < d_out && kk < d_in) ? W[n * d_in + kk] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < RK; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = xs[c][ty * 4 + i];
                b[i] = ws[c][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < d_out) Y[t * d_out + n] = acc[i][j];
        }
    }
}

// partials[2b] = sum (Yq - Yr)^2, partials[2b + 1] = sum Yr^2 over the elements that
// block b visits (a fixed grid-stride pattern), in fp64; the host adds the blocks in
// order, so the result is deterministic.
__global__ __launch_bounds__(256) void sq_err_kernel(const float* __restrict__ yq, const float* __restrict__ yr,
                                                     int64_t n, double* __restrict__ partials) {
    __shared__ double sn[256], sd[256];
    double num = 0.0, den = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const double d = (double)yq[i] - (double)yr[i];
        num += d * d;
        den += (double)yr[i] * (double)yr[i];
    }
    sn[threadIdx.x] = num;
    sd[threadIdx.x] = den;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            sn[threadIdx.x] += sn[threadIdx.x + w];
            sd[threadIdx.x] += sd[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        partials[2 * blockIdx.x] = sn[0];
        partials[2 * blockIdx.x + 1] = sd[0];
    }
}

}  // namespace

hipError_t launch_ref_linear(const void* X, int x_dtype, int64_t T, int64_t d_in, const float* W, int64_t d_out,
                             float* Y, hipStream_t st) {
    if (T <= 0 || d_out <= 0) return hipSuccess;
    const int64_t gx = (d_out + RT - 1) / RT, gy = (T + RT - 1) / RT;
    if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (x_dtype == W4A4_X_BF16)
        ref_linear_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)X, W, T, d_in, d_out, Y);
    else
        ref_linear_kernel<float><<<grid, 256, 0, st>>>((const float*)X, W, T, d_in, d_out, Y);
    return hipGetLastError();
}

hipError_t launch_sq_err(const float* yq, const float* yr, int64_t n, double* partials, int blocks,
                         hipStream_t st) {
    sq_err_kernel<<<blocks, 256, 0, st>>>(yq, yr, n, partials);
    return hipGetLastError();
}

}  // namespace w4a4
