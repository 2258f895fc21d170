// Per-call outlier selection ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B
// (ICME 2026 Challenge)", sec. 3.3 and sec. 4: MixQ picks the high-precision columns
// online, per call, where the page's method fixes a static top-k offline).  Each call
// scores its own tokens, score_j = fl32(max_t |x_tj| / s_j), takes the top k, and
// runs the layer with those columns in the BF16 branch: the J branch keeps every
// column at its own K position (a per-call re-compaction would re-pack the weights),
// with the chosen columns' activations zero, and W_O is gathered from a transposed
// bf16 copy of W.  These kernels do the selection and the gather; act-prep and the GEMM are the
// static path's own kernels, driven by a per-call column map.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

namespace {

// One 1024-lane workgroup; lane t owns the c = ceil(d_in / 1024) <= 16 consecutive
// columns [t c, t c + c) and holds their score bit patterns u_j = bits(|score_j|) in
// registers.  The order taken is that of u (numeric for finite scores and +Inf; a NaN
// ranks above +Inf), ties to the smaller column.  A radix select over u, four passes
// of 8-bit digits from the top with a 256-bin LDS histogram each, finds the k-th
// largest value B and how many of the columns equal to B are taken (need >= 1, the
// first ones in column order).  One block-wide exclusive scan of the packed per-lane
// counts (#u > B) | (#u == B) << 16 then gives each chosen column its rank in O
// (ascending columns): the number of chosen columns before it is
// #(u > B before it) + min(#(u == B before it), need).
constexpr int SEL_PER = 16;   // columns per lane: d_in <= 1024 * 16

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__global__ __launch_bounds__(1024) void dyn_select_kernel(const uint32_t* __restrict__ colmax_bits,
                                                          const float* __restrict__ s, int d_in, int k,
                                                          int32_t* __restrict__ O, int32_t* __restrict__ colmap) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t wtot[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = (d_in + 1023) / 1024;
    const int j0 = tid * c;
    const int nv = max(0, min(c, d_in - j0));   // this lane's valid columns
    uint32_t u[SEL_PER];
#pragma unroll
    for (int q = 0; q < SEL_PER; ++q) {
        const bool v = q < nv;
        const float a = v ? __uint_as_float(colmax_bits[j0 + q]) : 0.0f;
        const float d = v ? s[j0 + q] : 1.0f;
        u[q] = __float_as_uint(a / d) & 0x7FFFFFFFu;
    }
    if (k == 0) {
        for (int q = 0; q < nv; ++q) colmap[j0 + q] = j0 + q;
        return;
    }
    // radix select of the k-th largest u
    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < SEL_PER; ++q)
            if (q < nv && (u[q] & mask) == prefix) atomicAdd(&hist[(u[q] >> shift) & 255u], 1u);
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255 - 4l .. 252 - 4l, the largest first
            uint32_t h[4], loc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = hist[255 - 4 * lane - e];
                loc += h[e];
            }
            const uint32_t incl = wave_incl_scan(loc), excl = incl - loc;
            if (excl < remaining && remaining <= incl) {   // exactly one lane
                uint32_t above = excl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (remaining <= above + h[e]) {
                        sel[0] = (uint32_t)(255 - 4 * lane - e);
                        sel[1] = remaining - above;
                        break;
                    }
                    above += h[e];
                }
            }
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        mask |= 255u << shift;
        remaining = sel[1];
    }
    const uint32_t B = prefix, need = remaining;
    // block-wide exclusive scan of (#u > B) | (#u == B) << 16
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < SEL_PER; ++q)
        if (q < nv) cnt += u[q] > B ? 1u : (u[q] == B ? 0x10000u : 0u);
    const uint32_t incl = wave_incl_scan(cnt);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = incl - cnt;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    uint32_t gt = before & 0xFFFFu, eq = before >> 16;
#pragma unroll
    for (int q = 0; q < SEL_PER; ++q) {
        if (q >= nv) continue;
        const int j = j0 + q;
        if (u[q] > B) {
            const uint32_t r = gt + (eq < need ? eq : need);
            O[r] = j;
            colmap[j] = -(int32_t)(r + 1);
            ++gt;
        } else if (u[q] == B && eq < need) {
            const uint32_t r = gt + eq;
            O[r] = j;
            colmap[j] = -(int32_t)(r + 1);
            ++eq;
        } else {
            if (u[q] == B) ++eq;
            colmap[j] = j;
        }
    }
}

// W_O[n][i] = W_t[O[i]][n] for i < k, 0 for k <= i < k_ld.  A workgroup takes 64
// output rows n (one per lane) and 32 consecutive i (8 per wavefront): each lane makes
// 8 independent 2-byte loads, coalesced across the wavefront along n, and one 16-byte
// store.
__global__ __launch_bounds__(256) void dyn_gather_kernel(const uint16_t* __restrict__ Wt, const int32_t* __restrict__ O,
                                                         int64_t d_out, int32_t k, int64_t k_ld,
                                                         uint16_t* __restrict__ WO) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n = (int64_t)blockIdx.x * 64 + lane;
    const int64_t i0 = (int64_t)blockIdx.y * 32 + wave * 8;
    if (n >= d_out) return;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t i = i0 + e;
        h[e] = i < k ? (uint32_t)Wt[(int64_t)O[i] * d_out + n] : 0u;
    }
    *reinterpret_cast<uint4*>(WO + n * k_ld + i0) =
        make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
}

// W_t[j][n] = bf16_rne(W[n][j]) through a 64 x 64 LDS tile: coalesced reads along j,
// coalesced writes along n.  Run once, when the layer is packed.
__global__ __launch_bounds__(256) void dyn_transpose_kernel(const float* __restrict__ W, int64_t d_in, int64_t d_out,
                                                            uint16_t* __restrict__ Wt) {
    __shared__ uint16_t tile[64][64 + 2];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t j0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64;
    for (int r = ty; r < 64; r += 4) {
        const int64_t n = n0 + r, j = j0 + tx;
        tile[r][tx] = (n < d_out && j < d_in) ? bf16_rne(W[n * d_in + j]) : (uint16_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t j = j0 + r, n = n0 + tx;
        if (j < d_in && n < d_out) Wt[j * d_out + n] = tile[tx][r];
    }
}

}  // namespace

hipError_t launch_dyn_select(const uint32_t* colmax_bits, const float* s, int64_t d_in, int32_t k, int32_t* O,
                             int32_t* colmap, hipStream_t st) {
    if (d_in <= 0 || d_in > 1024 * SEL_PER || k < 0 || k > d_in) return hipErrorInvalidValue;
    dyn_select_kernel<<<1, 1024, 0, st>>>(colmax_bits, s, (int)d_in, k, O, colmap);
    return hipGetLastError();
}

hipError_t launch_dyn_gather(const uint16_t* W_t, const int32_t* O, int64_t d_in, int64_t d_out, int32_t k,
                             int64_t k_ld, uint16_t* WO, hipStream_t st) {
    (void)d_in;
    if (d_out <= 0 || k_ld <= 0) return hipSuccess;
    if (k_ld % 32 != 0 || (d_out + 63) / 64 > 0x7FFFFFFF || k_ld / 32 > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((d_out + 63) / 64), (unsigned)(k_ld / 32));
    dyn_gather_kernel<<<grid, 256, 0, st>>>(W_t, O, d_out, k, k_ld, WO);
    return hipGetLastError();
}

hipError_t launch_dyn_transpose(const float* W, int64_t d_in, int64_t d_out, uint16_t* W_t, hipStream_t st) {
    if (d_in <= 0 || d_out <= 0) return hipSuccess;
    if ((d_out + 63) / 64 > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((d_in + 63) / 64), (unsigned)((d_out + 63) / 64));
    dyn_transpose_kernel<<<grid, 256, 0, st>>>(W, d_in, d_out, W_t);
    return hipGetLastError();
}

}  // namespace w4a4
