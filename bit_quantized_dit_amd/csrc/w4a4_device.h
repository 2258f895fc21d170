// Device-side helpers shared by the gfx950 kernels of the W4A4 library.
//
// MXFP4 encoding used throughout (format named by "W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 1-2, OCP MX
// definition):
//   scale  E8M0 code c, value 2^(c-127); for a group with largest magnitude
//          amax: c = max(biased_exponent(amax) - 2, 0), i.e.
//          E = floor(log2 amax) - 2 clamped at -127 (subnormal and zero amax
//          give c = 0); NaN/Inf anywhere in the group gives c = 0xFF.
//   element E2M1 nibble: magnitude code = nearest of {0,.5,1,1.5,2,3,4,6} to
//          |x| * 2^-E, ties to the even code, saturating at 6; bit 3 = sign of x.
//
// Taking the group maximum on the integer bit patterns of |x| makes NaN/Inf
// detection free: any such element has abs bits >= 0x7F800000, which forces
// the exponent field of the maximum to 0xFF.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// E8M0 code from the bit pattern of the group's largest |x|.
__device__ __forceinline__ uint32_t e8m0_from_absbits(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 23;
    const uint32_t c = __builtin_elementwise_sub_sat(e, 2u);   // max(e - 2, 0)
    return e == 0xFFu ? 0xFFu : c;
}

// binary32 -> bf16, round to nearest even; a NaN becomes the canonical quiet NaN
// with its sign kept.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (gfx9 family): base, 16 high address bits, no stride,
// num_records = byte range, word 3 = 32-bit data format.  Out-of-range loads read 0;
// the range check covers the lane offset, not the scalar offset (soffset), so an
// offset that may cross the range goes into the lane offset.
__device__ __forceinline__ v4i make_srd(const void* p, uint32_t nbytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
    r[3] = 0x00020000;
    return r;
}

// Global -> LDS without VGPRs: lane i's 16 (4) bytes land at LDS m0 + 16*i (4*i).
// The compiler does not track these writes, so the kernel waits on vmcnt itself
// before the barrier that publishes a slot.  The instruction has no register
// results; its address operands are read at issue.  Descriptor, LDS base and
// soffset are wave-uniform by construction; readfirstlane only tells the compiler.
// One wait state separates the SALU write of m0 from the DMA that reads it.
__device__ __forceinline__ v4i uniform(v4i r) {
    return v4i{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
__device__ __forceinline__ void dma16(v4i srd, uint32_t lds, int voff, int soff) {
    srd = uniform(srd);
    lds = __builtin_amdgcn_readfirstlane(lds);
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(srd), "s"(soff));
}
__device__ __forceinline__ void dma4(v4i srd, uint32_t lds, int voff, int soff) {
    srd = uniform(srd);
    lds = __builtin_amdgcn_readfirstlane(lds);
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(srd), "s"(soff));
}


__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Two binary32 values rounded to bf16, nearest-even, packed (a in the low half):
// v_cvt_pk_bf16_f32.  On every non-NaN input it equals bf16_rne (all 2^32 patterns
// compared); a NaN stays a quiet NaN that keeps its top payload bits.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    typedef float v2f __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// GELU-tanh between the FFN projections ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.1 and 3.5) on a pair of fp32 outputs:
// bf16(gelu_tanh(bf16(y))), gelu_tanh(x) = 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3))),
// evaluated as x / (1 + exp(-2z)), z = sqrt(2/pi)(x + 0.044715 x^3): the same function
// (0.5(1 + tanh z) is the logistic of 2z) without the cancellation in 1 + tanh z that
// wipes out every digit of the negative tail in binary32.  exp(-2z) = 2^(x (K0 + K1 x^2))
// with K0 = -2 log2(e) sqrt(2/pi), K1 = 0.044715 K0; exp and the reciprocal are the
// hardware v_exp_f32 (2^t) and v_rcp_f32, each within about one binary32 ulp, so the
// fp32 value is within a few ulps of the exact function before the final rounding to
// bf16 (8 significant bits).  Tails: x -> -inf gives exp -> inf, rcp -> 0 and a signed
// zero; x -> +inf gives x.  A NaN result (a NaN y, or y = -inf) is written as the quiet
// NaN 0x7FC0 with the sign of y.  Shared by the standalone GELU kernel and the GEMM
// epilogue that fuses it, so both give the same bits.
__device__ __forceinline__ float gelu_tanh_f32_raw(float x) {
    constexpr float K0 = -2.302208198144325f, K1 = -0.1029432395800235f;
    const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(x * x, K1, K0));
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_tanh_f32(float x) {
    const float g = gelu_tanh_f32_raw(x);
    return g != g ? __uint_as_float((__float_as_uint(x) & 0x80000000u) | 0x7FC00000u) : g;
}

__device__ __forceinline__ uint32_t gelu_tanh_bf16x2(float y0, float y1) {
    const uint32_t yb = pk_bf16(y0, y1);
    return pk_bf16(gelu_tanh_f32(__uint_as_float(yb << 16)), gelu_tanh_f32(__uint_as_float(yb & 0xFFFF0000u)));
}
// The same pair without the NaN canonicalization (a NaN stays a NaN of some payload),
// for values that only go on to the MXFP4 encoding: there any NaN gives its block the
// scale code 0xFF and zero nibbles, whatever its payload, so the encoded bits are those
// of the canonical pair.
__device__ __forceinline__ uint32_t gelu_tanh_bf16x2_raw(float y0, float y1) {
    const uint32_t yb = pk_bf16(y0, y1);
    return pk_bf16(gelu_tanh_f32_raw(__uint_as_float(yb << 16)), gelu_tanh_f32_raw(__uint_as_float(yb & 0xFFFF0000u)));
}

__device__ __forceinline__ uint16_t gelu_tanh_bf16(float y) { return (uint16_t)gelu_tanh_bf16x2(y, 0.0f); }

}  // namespace w4a4
