// GELU-tanh between the FFN up projection (ffn.0) and down projection (ffn.2)
// named in "W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME 2026
// Challenge)", sec. 3.1 and 3.5:  H = bf16(gelu_tanh(bf16(Y))) with
// gelu_tanh(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in fp32.
// It is evaluated as x / (1 + exp(-2z)), z = sqrt(2/pi)(x + 0.044715 x^3): the same
// function (0.5(1 + tanh z) is the logistic of 2z), but free of the cancellation in
// 1 + tanh z that wipes out every digit of the negative tail in binary32.
// Elementwise and HBM-bound: 8 elements per thread, 32-byte loads, 16-byte stores.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

__device__ __forceinline__ uint16_t gelu_one(float y) {
    const float x = bf16_to_f32(bf16_rne(y));
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    const float z = c * (x + 0.044715f * x * x * x);
    return bf16_rne(x / (1.0f + expf(-2.0f * z)));
}

__global__ __launch_bounds__(256) void gelu_kernel(const float* __restrict__ Y, int64_t n,
                                                   uint16_t* __restrict__ H, int vec) {
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= n) return;
    if (vec && i0 + 8 <= n) {
        const float4 a = reinterpret_cast<const float4*>(Y + i0)[0];
        const float4 b = reinterpret_cast<const float4*>(Y + i0)[1];
        const uint32_t w0 = gelu_one(a.x) | ((uint32_t)gelu_one(a.y) << 16);
        const uint32_t w1 = gelu_one(a.z) | ((uint32_t)gelu_one(a.w) << 16);
        const uint32_t w2 = gelu_one(b.x) | ((uint32_t)gelu_one(b.y) << 16);
        const uint32_t w3 = gelu_one(b.z) | ((uint32_t)gelu_one(b.w) << 16);
        *reinterpret_cast<uint4*>(H + i0) = make_uint4(w0, w1, w2, w3);
    } else {
        for (int64_t i = i0; i < i0 + 8 && i < n; ++i) H[i] = gelu_one(Y[i]);
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
