// Per-call outlier selection ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B
// (ICME 2026 Challenge)", sec. 3.3 and sec. 4: MixQ picks the high-precision columns
// online, per call, where the page's method fixes a static top-k offline).  Each call
// scores its own tokens, score_j = fl32(max_t |x_tj| / s_j), takes the top k, and
// runs the layer with those columns in the BF16 branch: the J branch keeps every
// column at its own K position (a per-call re-compaction would re-pack the weights),
// with the chosen columns' activations zero, and W_O is gathered from a bf16 copy of
// W.  These kernels do the selection and the gather; act-prep and the GEMM are the
// static path's own kernels, driven by a per-call column map.
#include "w4a4_device.h"
#include "w4a4_internal.h"

namespace w4a4 {

namespace {

// One 1024-lane workgroup.  key[j] = (bits(|score_j|) << 32) | (2^32 - 1 - j): the
// descending order of the keys is the order of the scores as binary32 bit patterns
// (numeric for finite values and +Inf; a NaN ranks above +Inf), ties to the smaller
// column.  A bitonic sort of the n = 2^ceil(log2 d_in) keys in LDS (padding keys are
// 0, below every real key), then the first k are marked, and one block-wide scan of
// the marks gives O in ascending order and the column map: colmap[j] = j for a J
// column, -(i + 1) for the i-th outlier.
__global__ __launch_bounds__(1024) void dyn_select_kernel(const uint32_t* __restrict__ colmax_bits,
                                                          const float* __restrict__ s, int d_in, int k, int n,
                                                          int32_t* __restrict__ O, int32_t* __restrict__ colmap) {
    extern __shared__ uint64_t key[];
    const int tid = threadIdx.x;
    for (int j = tid; j < n; j += 1024) {
        uint64_t kv = 0;
        if (j < d_in) {
            const float sc = __uint_as_float(colmax_bits[j]) / s[j];
            kv = ((uint64_t)(__float_as_uint(sc) & 0x7FFFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        }
        key[j] = kv;
    }
    __syncthreads();
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n / 2; i += 1024) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const uint64_t a = key[lo], b = key[hi];
                // descending where bit `size` of lo is clear: the final pass sorts all
                if ((a < b) == ((lo & size) == 0)) {
                    key[lo] = b;
                    key[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    // the chosen columns, held in registers while the LDS becomes the mark array
    constexpr int PER = 16;   // n <= 16384 = 1024 * PER
    int32_t pick[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int p = tid + 1024 * q;
        pick[q] = (p < k && p < n) ? (int32_t)(0xFFFFFFFFu - (uint32_t)key[p]) : -1;
    }
    __syncthreads();
    uint32_t* mark = reinterpret_cast<uint32_t*>(key);
    int32_t* scan = reinterpret_cast<int32_t*>(key) + n;   // 1024 counts after the marks
    for (int j = tid; j < d_in; j += 1024) mark[j] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (pick[q] >= 0) mark[pick[q]] = 1;
    __syncthreads();
    // lane tid owns the columns [tid * c, tid * c + c): count, scan, then place
    const int c = (d_in + 1023) / 1024;
    const int j0 = tid * c, j1 = min(d_in, j0 + c);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (int)mark[j];
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
        const int v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    int rank = scan[tid] - cnt;
    for (int j = j0; j < j1; ++j) {
        if (mark[j]) {
            O[rank] = j;
            colmap[j] = -(rank + 1);
            ++rank;
        } else {
            colmap[j] = j;
        }
    }
}

// W_O[n][i] = W_bf16[n][O[i]] for i < k, 0 for k <= i < k_ld.
__global__ __launch_bounds__(256) void dyn_gather_kernel(const uint16_t* __restrict__ Wbf, const int32_t* __restrict__ O,
                                                         int64_t d_in, int64_t d_out, int32_t k, int64_t k_ld,
                                                         uint16_t* __restrict__ WO) {
    const int64_t total = d_out * k_ld;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t n = e / k_ld, i = e % k_ld;
        WO[e] = i < k ? Wbf[n * d_in + O[i]] : (uint16_t)0;
    }
}

}  // namespace

int dyn_select_lds_keys(int64_t d_in) {
    int n = 1;
    while (n < d_in) n <<= 1;
    return n;
}

hipError_t launch_dyn_select(const uint32_t* colmax_bits, const float* s, int64_t d_in, int32_t k, int32_t* O,
                             int32_t* colmap, hipStream_t st) {
    const int n = dyn_select_lds_keys(d_in);
    if (n > W4A4_DYN_MAX_D_IN) return hipErrorInvalidValue;
    const size_t lds = (size_t)n * sizeof(uint64_t) > (size_t)(n + 1024) * sizeof(int32_t)
                           ? (size_t)n * sizeof(uint64_t)
                           : (size_t)(n + 1024) * sizeof(int32_t);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)dyn_select_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dyn_select_kernel<<<1, 1024, lds, st>>>(colmax_bits, s, (int)d_in, k, n, O, colmap);
    return hipGetLastError();
}

hipError_t launch_dyn_gather(const uint16_t* Wbf, const int32_t* O, int64_t d_in, int64_t d_out, int32_t k,
                             int64_t k_ld, uint16_t* WO, hipStream_t st) {
    const int64_t total = d_out * k_ld;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    dyn_gather_kernel<<<(unsigned)blocks, 256, 0, st>>>(Wbf, O, d_in, d_out, k, k_ld, WO);
    return hipGetLastError();
}

}  // namespace w4a4
