// Calibration statistics: column-wise max |x| ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.2: per-channel activation and
// weight magnitudes gathered on calibration batches).
//
// The maximum is taken on the integer bit patterns of |x|: for non-negative
// binary32 values integer order equals numeric order, and NaN/Inf patterns sort
// above every finite value, so the result both is exact and flags bad data.
// Each thread owns one column (coalesced across the wavefront) and a slice of
// rows; slices are merged with a device-wide atomicMax, which is exact and
// order-independent, so the result is deterministic.
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

hipError_t launch_column_absmax(const void* X, int x_dtype, int64_t rows, int64_t cols,
                                uint32_t* out_bits, hipStream_t st) {
    if (cols <= 0) return hipSuccess;
    const unsigned gx = (unsigned)((cols + 255) / 256);
    fill_u32<<<gx, 256, 0, st>>>(out_bits, cols, 0u);
    if (rows <= 0) return hipGetLastError();
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
