// Calibration statistics: column-wise max |x| ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.2: per-channel activation and
// weight magnitudes gathered on calibration batches).
//
// The maximum is taken on the integer bit patterns of |x|: for non-negative
// binary32 values integer order equals numeric order, and NaN/Inf patterns sort
// above every finite value, so the result both is exact and flags bad data.
// Partial maxima over slices of rows are merged with a device-wide atomicMax, which is
// exact and order-independent, so the result is deterministic.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

template <typename XT>
__device__ __forceinline__ float load_as_f32(const XT* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

__global__ void fill_u32(uint32_t* p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Scalar form: each thread owns one column (coalesced across the wavefront) and a
// slice of rows.  Used where X is not 16-byte aligned.
template <typename XT>
__global__ __launch_bounds__(256) void column_absmax_kernel(const XT* __restrict__ X, int64_t rows,
                                                            int64_t cols, int64_t rows_per_slice,
                                                            uint32_t* __restrict__ out) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_slice;
    const int64_t r1 = r0 + rows_per_slice < rows ? r0 + rows_per_slice : rows;
    uint32_t m = 0;
    for (int64_t r = r0; r < r1; ++r) {
        const uint32_t a = abs_bits(load_as_f32<XT>(X, r * cols + j));
        m = a > m ? a : m;
    }
    atomicMax(out + j, m);
}

// Vector form, 16-byte loads.  X is read as a flat array of rows * cols elements,
// E = 16 / sizeof(XT) per load.  A super-row of m = E / gcd(cols, E) rows holds
// L = m * cols elements, a multiple of E, so the c-th 16-byte chunk of every
// super-row covers the same columns, (E c + q) mod cols for q < E.  A workgroup
// takes 64 chunk positions (one per lane of a wavefront) and a slice of super-rows,
// which its four wavefronts split round-robin; the four partial maxima meet in LDS
// and one atomicMax per element leaves the workgroup.  The rows past the last whole
// super-row (fewer than m) are read element by element by the last slice.
template <typename XT>
__global__ __launch_bounds__(256) void column_absmax_vec_kernel(const XT* __restrict__ X, int64_t rows,
                                                                int64_t cols, int64_t m, int64_t sr_per_slice,
                                                                uint32_t* __restrict__ out) {
    constexpr int E = 16 / (int)sizeof(XT);
    __shared__ uint32_t part[3][64 * E];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t L = m * cols, nchunk = L / E;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    const bool live = c < nchunk;
    const int64_t nsr = rows / m;
    const int64_t s0 = (int64_t)blockIdx.y * sr_per_slice;
    const int64_t s1 = s0 + sr_per_slice < nsr ? s0 + sr_per_slice : nsr;
    uint32_t mx[E];
#pragma unroll
    for (int q = 0; q < E; ++q) mx[q] = 0;
    const uint4* p = reinterpret_cast<const uint4*>(X) + (live ? c : 0);
    auto take = [&](const uint4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(XT) == 2) {
                // bf16 pairs: |x| as the f32 bit pattern of the widened value
                const uint32_t lo = (w[i] << 16) & 0x7FFFFFFFu, hi = w[i] & 0x7FFF0000u;
                mx[2 * i] = lo > mx[2 * i] ? lo : mx[2 * i];
                mx[2 * i + 1] = hi > mx[2 * i + 1] ? hi : mx[2 * i + 1];
            } else {
                const uint32_t a = w[i] & 0x7FFFFFFFu;
                mx[i] = a > mx[i] ? a : mx[i];
            }
        }
    };
    if (live) {
        int64_t s = s0 + wave;
        constexpr int U = 8;
        for (; s + 4 * (U - 1) < s1; s += 4 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = p[(s + 4 * u) * nchunk];
#pragma unroll
            for (int u = 0; u < U; ++u) take(v[u]);
        }
        for (; s < s1; s += 4) take(p[s * nchunk]);
        if (wave == 0 && blockIdx.y == gridDim.y - 1) {
            const int64_t total = rows * cols;
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const int64_t e = nsr * L + c * E + q;
                if (e < total) {
                    const uint32_t a = abs_bits(load_as_f32<XT>(X, e));
                    mx[q] = a > mx[q] ? a : mx[q];
                }
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int q = 0; q < E; ++q) part[wave - 1][q * 64 + lane] = mx[q];
    }
    __syncthreads();
    if (wave == 0 && live) {
        int64_t j = (c * E) % cols;
#pragma unroll
        for (int q = 0; q < E; ++q) {
            uint32_t a = mx[q];
#pragma unroll
            for (int w = 0; w < 3; ++w) a = part[w][q * 64 + lane] > a ? part[w][q * 64 + lane] : a;
            atomicMax(out + j, a);
            if (++j == cols) j = 0;
        }
    }
}

hipError_t launch_column_absmax(const void* X, int x_dtype, int64_t rows, int64_t cols,
                                uint32_t* out_bits, hipStream_t st) {
    if (cols <= 0) return hipSuccess;
    const unsigned gx = (unsigned)((cols + 255) / 256);
    fill_u32<<<gx, 256, 0, st>>>(out_bits, cols, 0u);
    if (rows <= 0) return hipGetLastError();
    const int64_t E = x_dtype == W4A4_X_BF16 ? 8 : 4;
    if (((uintptr_t)X & 15u) == 0) {
        int64_t g = cols, e = E;   // gcd(cols, E)
        while (e) { const int64_t r = g % e; g = e; e = r; }
        const int64_t m = E / g;
        const int64_t nchunk = m * cols / E;
        const int64_t bx = (nchunk + 63) / 64;
        const int64_t nsr = rows / m;
        // slices of super-rows: at most 2048 workgroups (8 per CU, all resident at once),
        // at least 16 super-rows each
        int64_t slices = 2048 / bx;
        if (slices > (nsr + 15) / 16) slices = (nsr + 15) / 16;
        if (slices < 1) slices = 1;
        if (slices > 65535) slices = 65535;
        const int64_t per = nsr > 0 ? (nsr + slices - 1) / slices : 0;
        slices = per > 0 ? (nsr + per - 1) / per : 1;
        if (bx <= 0x7FFFFFFF) {
            const dim3 grid((unsigned)bx, (unsigned)slices);
            if (x_dtype == W4A4_X_BF16)
                column_absmax_vec_kernel<uint16_t>
                    <<<grid, 256, 0, st>>>((const uint16_t*)X, rows, cols, m, per, out_bits);
            else
                column_absmax_vec_kernel<float><<<grid, 256, 0, st>>>((const float*)X, rows, cols, m, per, out_bits);
            return hipGetLastError();
        }
    }
    // enough slices to put a few thousand wavefronts in flight
    int64_t slices = (2048 + gx - 1) / gx;
    if (slices > rows) slices = rows;
    if (slices < 1) slices = 1;
    if (slices > 65535) slices = 65535;
    const int64_t per = (rows + slices - 1) / slices;
    slices = (rows + per - 1) / per;
    dim3 grid(gx, (unsigned)slices);
    if (x_dtype == W4A4_X_BF16)
        column_absmax_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)X, rows, cols, per, out_bits);
    else
        column_absmax_kernel<float><<<grid, 256, 0, st>>>((const float*)X, rows, cols, per, out_bits);
    return hipGetLastError();
}

}  // namespace w4a4
