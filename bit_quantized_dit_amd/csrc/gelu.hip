// Standalone GELU-tanh pass between the FFN up projection (ffn.0) and down
// projection (ffn.2) named in "W4A4 Quantization for Inference on Wan2.2-I2V-A14B
// (ICME 2026 Challenge)", sec. 3.1 and 3.5:  H = bf16(gelu_tanh(bf16(Y))), element
// function gelu_tanh_bf16x2 (w4a4_device.h, shared with the fused GEMM epilogue).
// Elementwise and HBM-bound: 8 elements per thread, 32-byte loads, 16-byte stores.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

__global__ __launch_bounds__(256) void gelu_kernel(const float* __restrict__ Y, int64_t n,
                                                   uint16_t* __restrict__ H, int vec) {
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= n) return;
    if (vec && i0 + 8 <= n) {
        const float4 a = reinterpret_cast<const float4*>(Y + i0)[0];
        const float4 b = reinterpret_cast<const float4*>(Y + i0)[1];
        const uint32_t w0 = gelu_tanh_bf16x2(a.x, a.y), w1 = gelu_tanh_bf16x2(a.z, a.w);
        const uint32_t w2 = gelu_tanh_bf16x2(b.x, b.y), w3 = gelu_tanh_bf16x2(b.z, b.w);
        *reinterpret_cast<uint4*>(H + i0) = make_uint4(w0, w1, w2, w3);
    } else {
        for (int64_t i = i0; i < i0 + 8 && i < n; ++i) H[i] = gelu_tanh_bf16(Y[i]);
    }
}

hipError_t launch_gelu(const float* Y, int64_t n, uint16_t* H, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t threads = (n + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int vec = (((uintptr_t)Y & 15u) == 0) && (((uintptr_t)H & 15u) == 0);
    gelu_kernel<<<(unsigned)blocks, 256, 0, st>>>(Y, n, H, vec);
    return hipGetLastError();
}

}  // namespace w4a4
