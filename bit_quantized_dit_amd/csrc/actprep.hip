// Fused activation prep ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME
// 2026 Challenge)", sec. 3.2: activations are divided by s and then quantized;
// sec. 3.3: the static outlier columns O bypass quantization).
//
// One workgroup streams whole token rows (persistent over rows) through an LDS copy
// laid out as [k_pad] J-compacted smoothed values followed by [k_ld] outlier values.
//   phase 1  every column goes to its fixed LDS slot, no branches: J column j at its
//            compacted position as fl32(x / s_j) (the correctly rounded binary32
//            quotient, from a double product with RN64(1 / s_j), see div_by_s), outlier
//            column O[i] at k_pad + i as the raw x.  Lane i of the workgroup owns the
//            column pairs 2(i + 512m), 2(i+512m)+1 (one 4-byte load for bf16, 8 bytes
//            for fp32, so each wavefront load is one contiguous run) and keeps their
//            slots and 1 / s_j in registers for the whole launch.
//   phase 2  each thread takes 8 consecutive compacted positions (two 16-byte LDS
//            reads); four lanes form one 32-block and meet their |x| maxima through two
//            DPP quad permutes; the E8M0 code follows from the maximum's exponent field
//            and the eight E2M1 nibbles come from four scaled FP4 conversions
//            (v_cvt_scalef32_pk_fp4_f32 with the scale 2^E as divisor), one 32-bit store
//            per lane into A_q in the GEMM's tiled order.  Lane 0 of the four stores the E8M0 byte into the step-major
//            scale array [k_pad/128][T][4] that the GEMM streams contiguously.  X_O is
//            copied out of the outlier slots as bf16.
// Rows are loaded in batches of D rows per workgroup, the next batch issued while the
// current one is processed, so that a full batch of loads is in flight across each
// batch's work.  HBM traffic is the algorithmic minimum: X read once, A_q/A_s/X_O
// written once.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

// Workgroup size of the generic kernel, and of the fast path up to d_in = 8192; the
// fast path takes 1024 lanes up to d_in = 16384.
constexpr int AP_THREADS = 512;


// LDS word of compacted position p: 16 bytes of padding follow every 32 positions,
// so that the 16-byte phase-2 reads of consecutive lanes (32 bytes apart) spread
// over all banks.  The outlier slots follow the last padded block.
__device__ __forceinline__ int32_t lds_pos(int64_t p) { return (int32_t)(p + ((p >> 5) << 2)); }
__device__ __forceinline__ int32_t lds_outliers(int64_t k_pad) { return lds_pos(k_pad); }
__host__ __device__ inline int64_t lds_words(int64_t k_pad, int64_t k_ld) { return k_pad + k_pad / 8 + k_ld; }

// Maximum of v over the four lanes of this lane's quad (lanes 4q..4q+3).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
    return o > v ? o : v;
}

// Eight E2M1 nibbles (element 2i in the low nibble of byte i) for finite values whose
// group scale code is `code` (< 0xFF; for 0xFF the result is meaningless).  The conversion divides by the fp32 scale 2^E
// and rounds to nearest even, saturating at 6; E = -127 is the subnormal 2^-127.
__device__ __forceinline__ uint32_t e2m1_word8(const float* v, uint32_t code) {
    // 2^E, E = code - 127: the biased exponent field, or the subnormal 2^-127 for code 0
    // (code << 23 is at least 2^-126 otherwise, so a maximum selects)
    const float scale = __uint_as_float(__builtin_elementwise_max(code << 23, 0x00400000u));
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
    return w;
}

// Phase 2 for token t held in LDS (row[0, k_pad)).
// A_q is written in the GEMM's tiled order: 1 KiB per (16-token block, 128-code step),
// token t % 16 at 64-byte stride, 16-byte chunk c at chunk position c ^ ((t % 16) / 4).
// as_t points at this token's scale slot of step 0 in the step-major A_s
// ([k_pad/128][T][4]); step kb's slot is as_t + kb * as_step.  k_pad is a multiple of
// 128, so the four lanes of a quad are active together.
// A pass of the NT lanes spans NT / 16 whole 128-code steps, so a lane's byte
// position within a step is the same on every pass and only the step advances: the
// A_q offset (32-bit, from the token's uniform block base), the A_s pointer and the
// LDS position all move by constants.  k_pad < 2^31 (the host checks it).
template <int NT>
__device__ __forceinline__ void quantize_row(const float* row, int64_t k_pad, uint8_t* Aq, int64_t t,
                                             uint8_t* as_t, int64_t as_step) {
    static_assert(NT % 16 == 0, "whole steps per pass");
    const int r = (int)(t & 15);
    uint8_t* const aq_blk = Aq + (((t >> 4) * (k_pad / 128)) << 10) + (r << 6);
    const int kp = (int)k_pad;
    const int first = (int)threadIdx.x * 8;
    uint32_t aq_off = ((uint32_t)(first >> 7) << 10) |
                      (((((uint32_t)first >> 5) & 3u) ^ (uint32_t)(r >> 2)) << 4) | (((uint32_t)first & 31u) >> 1);
    uint8_t* as_p = as_t + (int64_t)(first >> 7) * as_step + ((first >> 5) & 3);
    int lp = (int)lds_pos(first);
    for (int p0 = first; p0 < kp; p0 += NT * 8, aq_off += (NT / 16) << 10, as_p += (NT / 16) * as_step, lp += 9 * NT) {
        const float* src = row + lp;
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        // max |v| as IEEE maximum (v_maximum3_f32 with |.| source modifiers): a NaN
        // propagates, so its bit pattern (positive after |.|) tops every other one
        const float m01 = __builtin_elementwise_maximum(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
        const float m23 = __builtin_elementwise_maximum(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]));
        const float m45 = __builtin_elementwise_maximum(__builtin_fabsf(v[4]), __builtin_fabsf(v[5]));
        const float m67 = __builtin_elementwise_maximum(__builtin_fabsf(v[6]), __builtin_fabsf(v[7]));
        const float m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m01, m23),
                                                      __builtin_elementwise_maximum(m45, m67));
        const uint32_t code = e8m0_from_absbits(quad_max_u32(__float_as_uint(m)));
        // converted unconditionally (a NaN/Inf block's scale 2^128 gives some nibbles)
        // and then replaced by zero nibbles, without a branch
        const uint32_t word = e2m1_word8(v, code);
        *reinterpret_cast<uint32_t*>(aq_blk + aq_off) = code == 0xFFu ? 0u : word;
        *as_p = (uint8_t)code;   // the four lanes of the block store the same byte
    }
}

// X_O row from the outlier slots (slots >= k hold zero).
template <int NT>
__device__ __forceinline__ void copy_outliers(const float* row, int64_t k_pad, int64_t k_ld, uint16_t* xo_row) {
    for (int64_t i = threadIdx.x; i < k_ld; i += NT) xo_row[i] = bf16_rne(row[lds_outliers(k_pad) + i]);
}

// fl32(x / s) from r = RN64(1 / s): the double product x * r lies within 2^-52
// (relative) of the exact quotient x / s (one rounding in r, one in the product),
// while a quotient of two binary32 numbers is never a binary32 rounding boundary
// (a midpoint between neighbours) and stays at least ~2^-49 (relative) away from
// every such boundary: with x = X 2^a, s = S 2^b (X, S < 2^24) and a midpoint
// M 2^c (M odd, 2^24 <= M < 2^25), x - M 2^c s is a nonzero multiple of the
// smaller of 2^a and 2^(b+c), which bounds |x/s - M 2^c| / (x/s) below by
// 1 / (S M) > 2^-49.  Rounding the double product to binary32 (nearest even, the
// default mode; subnormal results kept) therefore yields the correctly rounded
// binary32 quotient, signed zeros and infinities included (x = +-0 or +-Inf give
// +-0 or +-Inf; a NaN stays a NaN, which only ever sets its group's scale to NaN).
// Three VALU operations instead of the eleven of the IEEE binary32 divide.
__device__ __forceinline__ float div_by_s(float x, double r) {
    return (float)((double)x * r);
}

// Fixed LDS slot of input column j from its column-map entry.
__device__ __forceinline__ int32_t slot_of(int32_t m, int64_t k_pad) {
    return m >= 0 ? lds_pos(m) : lds_outliers(k_pad) + (-m - 1);
}

// Zero the parts of the LDS row that phase 1 never writes: the J tail [k_j, k_pad)
// and the unused outlier slots k .. k_ld-1.
template <int NT>
__device__ __forceinline__ void zero_pads(float* row, int64_t k_j, int64_t k_pad, int32_t k, int64_t k_ld) {
    for (int64_t p = k_j + threadIdx.x; p < k_pad; p += NT) row[lds_pos(p)] = 0.0f;
    for (int64_t i = k + threadIdx.x; i < k_ld; i += NT) row[lds_outliers(k_pad) + i] = 0.0f;
}

template <typename XT>
__device__ __forceinline__ float load1(const XT* p);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }

// Generic path: any d_in, any element alignment of X.  One column per lane per pass.
template <typename XT>
__global__ __launch_bounds__(AP_THREADS) void actprep_kernel(
    const XT* __restrict__ X, int64_t T, int64_t d_in, const int32_t* __restrict__ colmap,
    const float* __restrict__ s, int64_t k_j, int64_t k_pad, int32_t k, int64_t k_ld,
    uint8_t* __restrict__ Aq, uint8_t* __restrict__ As, uint16_t* __restrict__ XO) {
    extern __shared__ float row[];
    zero_pads<AP_THREADS>(row, k_j, k_pad, k, k_ld);
    // with k_j = 0 (per-call outliers) the zeroed range holds the J slots that other
    // wavefronts fill for the first row: every zero lands before any phase-1 write
    __syncthreads();
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const XT* xr = X + t * d_in;
        for (int64_t j = threadIdx.x; j < d_in; j += AP_THREADS) {
            const int32_t m = colmap[j];
            const float x = load1<XT>(xr + j);
            row[slot_of(m, k_pad)] = m >= 0 ? x / s[j] : x;
        }
        __syncthreads();
        quantize_row<AP_THREADS>(row, k_pad, Aq, t, As + t * 4, T * 4);
        copy_outliers<AP_THREADS>(row, k_pad, k_ld, XO + t * k_ld);
        __syncthreads();
    }
}

// Two neighbouring elements of X (a 4-byte bf16 pair, an 8-byte fp32 pair) from a
// buffer descriptor; out-of-range offsets read zero.
template <typename XT>
struct Pair;
template <>
struct Pair<uint16_t> {
    typedef uint32_t raw;
    __device__ static raw load(__amdgpu_buffer_rsrc_t r, int32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    __device__ static float lo(raw v) { return __uint_as_float(v << 16); }
    __device__ static float hi(raw v) { return __uint_as_float(v & 0xFFFF0000u); }
};
template <>
struct Pair<float> {
    typedef uint2 raw;
    __device__ static raw load(__amdgpu_buffer_rsrc_t r, int32_t off) {
        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
        const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_uint2(v.x, v.y);
    }
    __device__ static float lo(raw v) { return __uint_as_float(v.x); }
    __device__ static float hi(raw v) { return __uint_as_float(v.y); }
};

// Rows per batch: two batches are live at once; within ~10 registers of row data per
// lane and batch (one register per bf16 pair, two per fp32 pair), so that the kernel
// stays within 128 VGPRs (four waves per SIMD: two 512-lane workgroups or one
// 1024-lane workgroup per CU).
template <typename XT, int MAXM>
constexpr int ap_depth() {
    constexpr int regs = MAXM * (int)(sizeof(XT) / 2);
    return regs * 4 <= 10 ? 4 : regs * 3 <= 10 ? 3 : regs * 2 <= 10 ? 2 : 1;
}

// Fast path: d_in even, 2 * NT * (MAXM - 1) < d_in <= 2 * NT * MAXM (the launcher
// takes the smallest MAXM that fits), so every pass but the last covers all NT
// lanes.  Lane i owns the column pairs
// 2(i + NT*m), 2(i + NT*m) + 1: one 4-byte (bf16) or 8-byte (fp32) load per pair, so
// a wavefront's loads of one m are one contiguous run.  Rows are read through a
// buffer descriptor per row (range d_in elements; zero range past the workgroup's
// last row), so every load is unpredicated with a per-lane constant offset.
template <typename XT, int NT, int MAXM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void actprep_pairs_kernel(
    const XT* __restrict__ X, int64_t T, int64_t d_in, const int32_t* __restrict__ colmap,
    const float* __restrict__ s, int64_t k_j, int64_t k_pad, int32_t k, int64_t k_ld,
    uint8_t* __restrict__ Aq, uint8_t* __restrict__ As, uint16_t* __restrict__ XO) {
    // two LDS row buffers: row r is staged in buffer r % 2, so phase 1 of the next row
    // needs no barrier behind phase 2 of this one (a wavefront writes buffer r % 2 for
    // row r + 2 only after passing row r + 1's barrier, which every wavefront reaches
    // after finishing phase 2 of row r)
    extern __shared__ float lds_rows[];
    const int64_t row_words = lds_words(k_pad, k_ld);
    zero_pads<NT>(lds_rows, k_j, k_pad, k, k_ld);
    zero_pads<NT>(lds_rows + row_words, k_j, k_pad, k, k_ld);
    // with k_j = 0 (per-call outliers) the zeroed range holds the J slots that other
    // wavefronts fill for the first rows: every zero lands before any phase-1 write
    __syncthreads();

    const int64_t npairs = d_in / 2;
    int32_t slot[MAXM][2];
    double rv[MAXM][2];   // RN64(1 / s_j) of the lane's columns
    bool outl[MAXM][2];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int64_t pi = min((int64_t)threadIdx.x + (int64_t)NT * m, npairs - 1);
        const int2 cm = reinterpret_cast<const int2*>(colmap)[pi];
        const float2 s2 = reinterpret_cast<const float2*>(s)[pi];
        slot[m][0] = slot_of(cm.x, k_pad);
        slot[m][1] = slot_of(cm.y, k_pad);
        rv[m][0] = 1.0 / (double)s2.x;
        rv[m][1] = 1.0 / (double)s2.y;
        outl[m][0] = cm.x < 0;
        outl[m][1] = cm.y < 0;
    }

    constexpr int D = ap_depth<XT, MAXM>();
    typedef typename Pair<XT>::raw raw;
    // Tokens are dealt so that a line of the outputs fills within one round of rows in
    // one L2: workgroup b runs on XCD b % 8 (workgroups are dispatched round-robin over
    // the 8 XCDs), XCD x quantizes the 32-token groups g with g % 8 == x, and its
    // G / 8 workgroups take consecutive tokens of those groups in each round (row r of
    // workgroup b is position f = r G/8 + b/8 of the XCD's token sequence).  The 32
    // tokens that share a 128-byte line of A_s (one step's 4 scale bytes per token), and
    // the two tokens that share a line of the tiled A_q, are then written by workgroups
    // of one XCD within the same round, and the line reaches memory whole.  With a
    // contiguous token range per workgroup an A_s line stayed open across 32 rounds of
    // streaming traffic and was written back in pieces.  (A grid that is not a multiple
    // of 8 deals the tokens round-robin: row r of workgroup b is token r G + b.)
    const bool by_xcd = gridDim.x % 8 == 0;
    const int64_t gx = by_xcd ? gridDim.x / 8 : gridDim.x;
    const int64_t wx = by_xcd ? blockIdx.x / 8 : blockIdx.x;
    const int64_t xcd = by_xcd ? blockIdx.x % 8 : 0;
    auto tok = [&](int64_t r) __attribute__((always_inline)) {
        const int64_t f = r * gx + wx;
        return by_xcd ? ((((f >> 5) << 3) + xcd) << 5) + (f & 31) : f;
    };
    if (tok(0) >= T) return;
    const int row_bytes = (int)(d_in * (int64_t)sizeof(XT));
    auto fetch = [&](raw (*xv)[MAXM], int64_t r0) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t t = tok(r0 + d);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(X + (t < T ? t : 0) * d_in), 0, t < T ? row_bytes : 0, 0x00020000);
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                xv[d][m] = Pair<XT>::load(rs, (int32_t)((threadIdx.x + NT * m) * 2 * sizeof(XT)));
        }
    };
    // Rows r0 .. r0+D-1 of this workgroup from xv; the loads of the next batch into
    // xn are issued once the first row of this batch has left the registers.
    auto batch = [&](raw (*xv)[MAXM], raw (*xn)[MAXM], int64_t r0) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t t = tok(r0 + d);
            if (t >= T) break;
            float* const row = lds_rows + ((r0 + d) & 1) * row_words;
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                const float lo = Pair<XT>::lo(xv[d][m]), hi = Pair<XT>::hi(xv[d][m]);
                const float qlo = div_by_s(lo, rv[m][0]), qhi = div_by_s(hi, rv[m][1]);
                if (m + 1 < MAXM || (int64_t)threadIdx.x + (int64_t)NT * m < npairs) {
                    row[slot[m][0]] = outl[m][0] ? lo : qlo;
                    row[slot[m][1]] = outl[m][1] ? hi : qhi;
                }
            }
            if (d == 0) fetch(xn, r0 + D);
            __syncthreads();
            quantize_row<NT>(row, k_pad, Aq, t, As + t * 4, T * 4);
            copy_outliers<NT>(row, k_pad, k_ld, XO + t * k_ld);
        }
    };
    raw xa[D][MAXM], xb[D][MAXM];
    fetch(xa, 0);
    for (int64_t r = 0; tok(r) < T; r += 2 * D) {
        batch(xa, xb, r);
        if (tok(r + D) >= T) break;
        batch(xb, xa, r + D);
    }
}

template <typename XT>
static hipError_t launch_typed(const XT* X, int64_t T, const w4a4_packed& d, uint8_t* Aq, uint8_t* As,
                               uint16_t* XO, hipStream_t st) {
    const size_t lds = (size_t)(lds_words(d.k_pad, d.k_ld) > 0 ? lds_words(d.k_pad, d.k_ld) : 1) * sizeof(float);
    const int64_t n = d.d_in;
    // The fast paths run persistent workgroups, each over a contiguous token range:
    // as many as are resident at once (two 512-lane or one 1024-lane workgroup per CU),
    // so each pays its per-column setup (column map, 1/s) once for many rows.
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev] = c;
    }
    const int64_t resident = (n <= 2 * (int64_t)AP_THREADS * 8) ? 2 * (int64_t)cus[dev] : (int64_t)cus[dev];
    const unsigned grid = (unsigned)(T < resident ? T : resident);
#define W4A4_AP_LAUNCH(KERNEL, NT, LDS)                                                              \
    {                                                                                                \
        const size_t lds_b = (LDS);                                                                  \
        if (lds_b > 65536) {                                                                         \
            hipError_t e = hipFuncSetAttribute((const void*)KERNEL,                                  \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_b); \
            if (e != hipSuccess) return e;                                                           \
        }                                                                                            \
        KERNEL<<<grid, NT, lds_b, st>>>(X, T, d.d_in, d.colmap, d.s, d.k_j, d.k_pad, d.k, d.k_ld, Aq, \
                                        As, XO);                                                     \
        return hipGetLastError();                                                                    \
    }
#define W4A4_AP_PAIRS(NT, M) \
    if (n % 2 == 0 && n <= 2 * (int64_t)(NT) * (M)) W4A4_AP_LAUNCH((actprep_pairs_kernel<XT, NT, M>), NT, 2 * lds)
    W4A4_AP_PAIRS(512, 1)
    W4A4_AP_PAIRS(512, 2)
    W4A4_AP_PAIRS(512, 3)
    W4A4_AP_PAIRS(512, 4)
    W4A4_AP_PAIRS(512, 5)
    W4A4_AP_PAIRS(512, 6)
    W4A4_AP_PAIRS(512, 7)
    W4A4_AP_PAIRS(512, 8)
    W4A4_AP_PAIRS(1024, 5)
    W4A4_AP_PAIRS(1024, 6)
    W4A4_AP_PAIRS(1024, 7)
    W4A4_AP_PAIRS(1024, 8)
    W4A4_AP_LAUNCH((actprep_kernel<XT>), AP_THREADS, lds)
#undef W4A4_AP_PAIRS
#undef W4A4_AP_LAUNCH
}

hipError_t launch_actprep(const void* X, int x_dtype, int64_t T, const w4a4_packed& d, uint8_t* Aq,
                          uint8_t* As, uint16_t* XO, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (x_dtype == W4A4_X_BF16) return launch_typed<uint16_t>((const uint16_t*)X, T, d, Aq, As, XO, st);
    return launch_typed<float>((const float*)X, T, d, Aq, As, XO, st);
}

}  // namespace w4a4
