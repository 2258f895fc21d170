/*
 * w4a4.h -- C ABI of the MI355X (gfx950) W4A4 dual-branch linear library.
 *
 * The layer (page "W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME 2026
 * Challenge)", xllm-io paper review, sec. 3.2-3.4):
 *
 *     Y = Q(X_J / s_J) . Q(s_J * W_J)  +  X_O . W_O
 *
 *   - SmoothQuant smoothing s_j = act_scale_j^alpha / weight_scale_j^(1-alpha)
 *     (sec. 3.2), folded into the weights offline; activations are divided by s
 *     at inference time and then quantized.
 *   - A static set O of k outlier input columns, the top-k of
 *     score_j = max_t |x_tj / s_j| over calibration tokens (sec. 3.3, scored
 *     after the fold per sec. 3.5), runs as a narrow BF16 branch on the raw
 *     (unsmoothed) columns; the rest, J, runs as strict MXFP4.
 *   - MXFP4 (named in sec. 1-2; OCP MX definition): E2M1 codes
 *     {0,+-0.5,+-1,+-1.5,+-2,+-3,+-4,+-6}, two per byte with the even K index
 *     in the low nibble, one E8M0 scale 2^(code-127) per group;
 *     E = floor(log2 amax) - 2 clamped at -127, amax = 0 -> code 0, a NaN/Inf
 *     in the group -> code 0xFF with all its nibbles 0; elements round to
 *     nearest, ties to the even code, saturating at 6, sign kept.
 *   - Weight scale groups (sec. 3.4): 1x32 along K, 32x32 tiles, or 128x1
 *     K-major stripes.  Activation scales are always 1x32 per token.
 *   - The J columns are compacted in ascending order and zero padded to
 *     K_pad = roundup(K_J, 128), K_J = d_in - k.
 *
 * Conventions for every entry point:
 *   - Return value: a w4a4_status; no exception or abort crosses the ABI.
 *   - "device" pointers are HIP device memory on the current device; "host"
 *     pointers are ordinary host memory.  The caller owns every buffer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls marked async only enqueue work on it; kernel faults surface at the
 *     caller's next synchronisation as HIP errors.
 *   - Shapes are validated before anything is enqueued.  T = 0 is a no-op.
 *   - Device pointers handed to the per-call entry points must be 16-byte
 *     aligned; buffers sized by the size queries are 256-byte aligned inside.
 *   - Calls on different streams that share a workspace race; the library keeps
 *     no global state and is otherwise reentrant (the one exception is the fixed
 *     device scratch array of w4a4_linear_noalloc).
 *   - The async per-call entry points enqueue kernels only: no allocation, no
 *     memset or copy, no synchronisation (memory that must start at zero is
 *     cleared by a kernel).  They may be captured into a HIP graph once the same
 *     call has run eagerly on the device (the first call sets kernel attributes).
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4a4_status {
    W4A4_OK = 0,
    W4A4_ERR_INVALID = 1,   /* null pointer, bad dtype/layout, k not in [0,d_in], alpha not in [0,1], negative size */
    W4A4_ERR_SHAPE = 2,     /* size beyond the supported range, or a blob/workspace that is too small */
    W4A4_ERR_ALIGN = 3,     /* a device pointer that is not 16-byte aligned */
    W4A4_ERR_DEVICE = 4,    /* a HIP runtime error from a launch, copy or synchronisation */
    W4A4_ERR_NONFINITE = 5, /* calibration data holds NaN or Inf */
    W4A4_ERR_SCRATCH = 6    /* w4a4_linear_noalloc: the call needs more workspace than
                               W4A4_NOALLOC_SCRATCH_BYTES */
} w4a4_status;

enum { W4A4_X_F32 = 0, W4A4_X_BF16 = 1 };

/* Weight scale-group layouts (page above, sec. 3.4). */
enum {
    W4A4_WS_1X32 = 0,          /* B_s [d_out][K_pad/32]: one scale per row per 32 K          */
    W4A4_WS_32X32_TILE = 1,    /* B_s [K_pad/32][ceil(d_out/32)]: 32 K x 32 rows per scale   */
    W4A4_WS_128X1_STRIPE = 2   /* B_s [d_out][K_pad/128]: 128 K x 1 row, K-major stripes      */
};

/* Largest supported input width (act-prep stages smoothed rows, K_pad fp32 each,
 * in LDS). */
#define W4A4_MAX_D_IN 32768
/* Largest d_in of the per-call outlier path (its top-k holds every column's score
 * in the registers of one 1024-lane workgroup, 16 per lane). */
#define W4A4_DYN_MAX_D_IN 16384

/* Packed layer descriptor, filled by w4a4_pack_weights.  Plain data: copy it
 * freely; it points into the caller's blob and owns nothing. */
typedef struct w4a4_packed {
    int64_t d_in, d_out;
    int32_t k;              /* |O|, number of BF16 outlier columns                        */
    int32_t layout;         /* W4A4_WS_*                                                  */
    int64_t k_j;            /* d_in - k                                                   */
    int64_t k_pad;          /* roundup(k_j, 128)                                          */
    int64_t k_ld;           /* row stride in elements of W_O and X_O: roundup(k, 32)      */
    const int32_t* colmap;  /* device [d_in]: p >= 0 = J column at compacted position p;
                               -(i+1) = outlier column O[i]                               */
    const float* s;         /* device [d_in] smoothing factors                            */
    const int32_t* O;       /* device [k], ascending                                      */
    const int32_t* J;       /* device [k_j], ascending                                    */
    const uint8_t* B_q;     /* device [d_out][k_pad/2] E2M1 codes of fl32(s_j * W[n][j])  */
    const uint8_t* B_s;     /* device, E8M0 codes in the layout's shape (see enum)        */
    const uint8_t* B_s_rows;/* device [k_pad/128][d_out][4]: the same codes, one per row per
                               32-block, step-major (the four codes of a 128-code step of
                               one row are adjacent, and consecutive rows follow), a
                               derived copy that the GEMM streams                         */
    const uint16_t* W_O;    /* device bf16 [d_out][k_ld], raw W[n][O[i]], zero padded     */
    const uint8_t* B_q_tiles;/* device, the codes of B_q re-laid for the GEMM's DMA (a derived
                               copy): [ceil(d_out/16)][k_pad/128][16][64] -- for each block of
                               16 rows and each 128-code step one contiguous 1 KiB run, row r
                               of the block at r*64, its 16-byte chunk c at chunk position
                               c ^ ((r >> 2) & 3); rows past d_out are zero                 */
} w4a4_packed;

/* Offsets (bytes) of the quantized activations inside a workspace. */
/* Layer packed for per-call outlier selection (w4a4_pack_weights_dyn): `base` is the
 * layer packed over all d_in columns (k = 0: J = every column, s folded in, B_q, B_s,
 * B_s_rows, B_q_tiles over K_pad = roundup(d_in, 128)); W_t = bf16_rne(W) transposed
 * keeps every column of W, contiguous, for the per-call W_O gather; k columns are
 * chosen per call. */
typedef struct w4a4_packed_dyn {
    w4a4_packed base;
    int32_t k;              /* outlier columns chosen per call, 0 <= k <= d_in             */
    int32_t reserved;
    const uint16_t* W_t;    /* device bf16 [d_in][d_out]: W_t[j][n] = bf16_rne(W[n][j])   */
} w4a4_packed_dyn;

typedef struct w4a4_ws_layout {
    size_t a_q;       /* uint8 activation E2M1 codes in the GEMM's tiled order,
                         [ceil(T/16)][k_pad/128][16][64]: the byte holding codes
                         p, p+1 (p even) of token t sits at
                           ((t/16)*(k_pad/128) + p/128)*1024 + (t%16)*64
                           + (c ^ ((t%16)/4))*16 + ((p%128)/2)%16,
                         c = (p%128)/32 -- the order of B_q_tiles; rows past T
                         inside the last 16-row block are left unwritten     */
    size_t a_s;       /* uint8 [k_pad/128][T][4] activation E8M0 scales (1x32),
                         step-major: for each 128-code step the four codes of
                         token t sit at [(step*T + t)*4 .. +3]                 */
    size_t x_o;       /* bf16  [T][k_ld] outlier columns, zero padded         */
    size_t partial;   /* fp32 partial sums of the GEMM's split-K tail tiles
                         (scratch the GEMM writes and reads back within one
                         call; empty when the tiles fill whole rounds of 256
                         workgroups or too few would be split)              */
    size_t total;     /* bytes needed                                         */
} w4a4_ws_layout;

/* Human-readable name of a status code (static storage). */
const char* w4a4_status_string(int status);

/* Column-wise max |x| of a row-major [rows][cols] device matrix (fp32 or bf16),
 * the per-channel magnitudes of sec. 3.2.  out_bits (device, [cols]) receives the
 * binary32 bit pattern of each maximum; a pattern >= 0x7F800000 means the
 * column holds NaN or Inf.  Async; out_bits is overwritten. */
int w4a4_column_absmax(const void* X, int x_dtype, int64_t rows, int64_t cols,
                       uint32_t* out_bits, void* stream);

/* Offline calibration (sec. 3.2-3.3, order per sec. 2 / 3.5): per-channel maxima of
 * X_cal (device [T_cal][d_in], fp32 or bf16) and of W (device fp32 [d_out][d_in],
 * nn.Linear orientation, reduced over d_out), then on the host in double:
 *   s_j = max(a_j,1e-5)^alpha / max(w_j,1e-5)^(1-alpha), rounded once to fp32,
 *   score_j = fl32(a_j / s_j), O = top-k scores (ties -> smaller j), ascending.
 * s_out [d_in] and O_out [k] are HOST buffers; act_scale_out / weight_scale_out
 * (host [d_in]) may be NULL.  Blocking: synchronises `stream`.  Allocates a
 * small device scratch (8*d_in bytes) internally.  Returns W4A4_ERR_NONFINITE if
 * either input holds NaN/Inf. */
int w4a4_calibrate_scales(const void* X_cal, int x_dtype, int64_t T_cal, int64_t d_in,
                          const float* W, int64_t d_out, float alpha, int32_t k,
                          float* s_out, int32_t* O_out,
                          float* act_scale_out, float* weight_scale_out, void* stream);

/* Bytes of the device blob that w4a4_pack_weights fills. */
int w4a4_packed_size(int64_t d_in, int64_t d_out, int32_t k, int layout, size_t* bytes);

/* Offline fold + split + pack (sec. 3.2 fold, 3.3 split, 3.4 block packing):
 * W device fp32 [d_out][d_in]; s (host [d_in], s_j > 0 finite) and O (host [k],
 * strictly ascending, in [0,d_in)) as produced by calibration (s = 1, k = 0 gives
 * naive W4A4).  Writes B_q = E2M1(fl32(s_j * W[n][J[p]])) with E8M0 scales in
 * `layout`, W_O = bf16_rne(W[n][O[i]]), plus s, O, J and the column map, into
 * `blob` (device, blob_bytes >= w4a4_packed_size), and fills *desc.  Blocking:
 * synchronises `stream` (host inputs are staged before return). */
int w4a4_pack_weights(const float* W, int64_t d_in, int64_t d_out, const float* s,
                      const int32_t* O, int32_t k, int layout, void* blob,
                      size_t blob_bytes, w4a4_packed* desc, void* stream);

/* Workspace offsets and size for T tokens with this layer. */
int w4a4_workspace_layout(int64_t T, const w4a4_packed* desc, w4a4_ws_layout* out);
int w4a4_workspace_size(int64_t T, const w4a4_packed* desc, size_t* bytes);

/* Act-prep (sec. 3.2 "divide by s, then quantize", sec. 3.3 split): X device
 * [T][d_in] fp32 or bf16, row-major contiguous.  For each token: x~ = fl32(x / s_j)
 * (IEEE binary32 division, subnormals kept) over the J columns in ascending order,
 * 1x32 E8M0 + E2M1 codes into A_q/A_s (A_s step-major, see w4a4_ws_layout);
 * X_O = bf16_rne(x) over the O columns.
 * Async on `stream`; never allocates. */
int w4a4_quantize_activations(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc,
                              void* ws, size_t ws_bytes, void* stream);

/* Dual-branch GEMM (sec. 3.3) on quantized activations already in `ws`:
 * Y[t][n] = sum_b 2^(Ea+Eb) sum_{p in b} a.b  (block-scaled FP4 MFMA)
 *         + sum_i X_O[t][i] W_O[n][i]         (BF16 MFMA, same fp32 accumulator)
 * Y device fp32 [T][d_out].  Reads A_q, A_s and X_O of `ws`; writes its `partial`
 * region when the plan splits the last round of 256 x 256 output tiles along K
 * (results then sum the K ranges' fp32 partials in a fixed order, so a given shape
 * is bit-reproducible).  Async; never allocates. */
int w4a4_gemm_prequantized(void* ws, size_t ws_bytes, int64_t T, const w4a4_packed* desc,
                           float* Y, void* stream);

/* The per-call path: act-prep then the dual-branch GEMM.  Async; never allocates. */
int w4a4_linear(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, float* Y,
                void* ws, size_t ws_bytes, void* stream);

/* Per-call outlier selection, the online variant that sec. 3.3 / sec. 4 attribute to
 * MixQ and that the page's method replaces with a static top-k.  Each call scores its
 * own tokens, score_j = fl32(max_t |x_tj| / s_j), compared as binary32 bit patterns of
 * |score| (numeric order for finite values and +Inf, a NaN above +Inf), larger first,
 * ties to the smaller column; O = the top k, ascending.  The J branch keeps every
 * column at its own K position (K_pad = roundup(d_in, 128)) with the chosen columns'
 * activations set to zero, so its 32-blocks are the column blocks of X rather than
 * blocks of the compacted J; the O branch is bf16 X_O . bf16 W_O with W_O gathered per
 * call from W_t.  d_in <= W4A4_DYN_MAX_D_IN and even; s as for w4a4_pack_weights.
 *
 * w4a4_packed_dyn_size / w4a4_pack_weights_dyn: one device blob (blocking,
 * like w4a4_pack_weights).  w4a4_workspace_dyn_layout / _size: for T tokens, the static
 * workspace of the k-column layer over K_pad = roundup(d_in, 128) followed by the
 * per-call column maxima (uint32 bit patterns [d_in]), O (int32 [k]), the column map
 * (int32 [d_in]: j for a J column, -(i+1) for the i-th outlier) and W_O (bf16
 * [d_out][roundup(k, 32)]).  w4a4_linear_dyn: X device [T][d_in] fp32 or bf16, Y
 * device fp32 [T][d_out]; async, never allocates; a call reuses its workspace, so
 * concurrent calls need one each. */
typedef struct w4a4_ws_dyn_layout {
    w4a4_ws_layout base;    /* a_q, a_s, x_o as for the static path, k_pad over all columns */
    size_t colmax, O, colmap, W_O, total;
} w4a4_ws_dyn_layout;
int w4a4_packed_dyn_size(int64_t d_in, int64_t d_out, int32_t k, int layout, size_t* bytes);
int w4a4_pack_weights_dyn(const float* W, int64_t d_in, int64_t d_out, const float* s, int32_t k,
                          int layout, void* blob, size_t blob_bytes, w4a4_packed_dyn* desc,
                          void* stream);
int w4a4_workspace_dyn_layout(int64_t T, const w4a4_packed_dyn* desc, w4a4_ws_dyn_layout* out);
int w4a4_workspace_dyn_size(int64_t T, const w4a4_packed_dyn* desc, size_t* bytes);
int w4a4_linear_dyn(const void* X, int x_dtype, int64_t T, const w4a4_packed_dyn* desc, float* Y,
                    void* ws, size_t ws_bytes, void* stream);

/* FFN block with the down layer's activation prep fused into the up projection
 * (sec. 3.1 / 3.5: up projection, GELU-tanh, down projection; sec. 3.2-3.4 for the
 * down layer's smoothing, outlier split and MXFP4 codes).  H = bf16(gelu_tanh(bf16(
 * X W_up^T))) never goes to memory: the up GEMM's epilogue writes the down layer's
 * A_q, A_s and X_O directly, bit-identical to w4a4_quantize_activations(H, down).
 *
 * Precondition on the packing: output feature f of `up` must be the down layer's
 * input column P[f], with P = (the down layer's J columns, ascending, then its O
 * columns, ascending), i.e. `up` is packed from the rows W_up[P[f]].  Permuting the
 * rows of W_up does not change its calibration (the per-input-column maxima), and
 * GELU is elementwise.  With 1x32 or 128x1 weight scales (one row per scale group)
 * the permuted layer is the same layer with its outputs reordered; with 32x32 tiles
 * the permutation also regroups the rows that share a tile scale, so the permuted
 * layer is a different, equally valid quantization of W_up.  The up layer's output
 * feature f < k_j is the down layer's compacted J position f and f >= k_j its outlier
 * slot f - k_j.  The library cannot check the permutation.
 *
 * w4a4_ffn_workspace_layout / _size: for T tokens, the up layer's workspace (offsets
 * in `up` relative to up_base), the down layer's (relative to down_base) and
 * RN64(1 / s_j) of the down layer's J columns (double [down.k_j]).
 * w4a4_ffn_up_quantize: act-prep of X for `up`, then the up GEMM with GELU and the
 * down layer's act-prep in its epilogue; afterwards the down layer's A_q, A_s, X_O sit
 * in the workspace at down_base + down.{a_q, a_s, x_o}, in the layout
 * w4a4_ws_layout documents.  w4a4_ffn_forward: the same, then the down GEMM into Y
 * (fp32 [T][down.d_out]).  Errors: INVALID (null pointer, bad dtype, T < 0, a bad
 * descriptor), SHAPE (up.d_out != down.d_in, workspace too small), ALIGN (pointers
 * not 16-byte aligned), DEVICE.  Async; never allocates. */
typedef struct w4a4_ffn_ws_layout {
    w4a4_ws_layout up;     /* relative to up_base                                   */
    w4a4_ws_layout down;   /* relative to down_base                                 */
    size_t up_base, down_base;
    size_t rinv;           /* double [down.k_j]                                     */
    size_t total;
} w4a4_ffn_ws_layout;

int w4a4_ffn_workspace_layout(int64_t T, const w4a4_packed* up, const w4a4_packed* down,
                              w4a4_ffn_ws_layout* out);
int w4a4_ffn_workspace_size(int64_t T, const w4a4_packed* up, const w4a4_packed* down, size_t* bytes);
int w4a4_ffn_up_quantize(const void* X, int x_dtype, int64_t T, const w4a4_packed* up,
                         const w4a4_packed* down, void* ws, size_t ws_bytes, void* stream);
int w4a4_ffn_forward(const void* X, int x_dtype, int64_t T, const w4a4_packed* up,
                     const w4a4_packed* down, float* Y, void* ws, size_t ws_bytes, void* stream);

/* Layer-wise choice of alpha and k (sec. 3.2 gives alpha in [0.5, 0.7] for the FFN up
 * projection; sec. 4 lists per-layer alpha and k, and sec. 6 names tuning them per
 * layer as the next step; the pages give no selection rule, so the rule here is the
 * smallest output error on calibration tokens).  For every pair (alphas[a], ks[b]):
 * calibrate s and O on X_cal (as w4a4_calibrate_scales), pack W in `layout` (as
 * w4a4_pack_weights), run the layer on X_cal (as w4a4_linear), and score it by the
 * relative Frobenius error ||Y_q - Y_ref||_F / ||Y_ref||_F against the unquantized
 * product Y_ref = X_cal W^T (fp32 inputs and accumulation; the sums of squares in
 * fp64, added in a fixed order, so the result is deterministic).
 *   X_cal  device [T_cal][d_in] fp32 or bf16; W device fp32 [d_out][d_in];
 *   alphas host [n_alpha] in [0,1]; ks host [n_k] in [0,d_in];
 *   scratch device, scratch_bytes >= w4a4_search_scratch_size (16-byte aligned);
 *   err_out host [n_alpha * n_k]: err_out[a * n_k + b];
 *   best_out host [2]: (a, b) of the smallest finite error, first on ties, (-1, -1)
 *   if none is finite.
 * Blocking (synchronises `stream` once per candidate); never allocates.  Errors as
 * the calls it composes (W4A4_ERR_NONFINITE for non-finite calibration data). */
int w4a4_search_scratch_size(int64_t T_cal, int64_t d_in, int64_t d_out, const int32_t* ks, int n_k,
                             int layout, size_t* bytes);
int w4a4_search_alpha_k(const void* X_cal, int x_dtype, int64_t T_cal, int64_t d_in, const float* W,
                        int64_t d_out, const float* alphas, int n_alpha, const int32_t* ks, int n_k,
                        int layout, void* scratch, size_t scratch_bytes, double* err_out,
                        int32_t* best_out, void* stream);

/* The FFN up projection with its activation fused (sec. 3.1 / 3.5: ffn.0 is followed
 * by GELU-tanh, whose bf16 output feeds ffn.2): the dual-branch GEMM of
 * w4a4_gemm_prequantized / w4a4_linear, with every fp32 output y stored as
 * H = bf16_rne(gelu_tanh(bf16_rne(y))) -- bit-identical to w4a4_gelu_tanh_bf16 over
 * the fp32 Y of the unfused call, without writing or re-reading Y.
 * H device bf16 [T][d_out] (16-byte aligned).  Async; never allocate. */
int w4a4_gemm_prequantized_gelu_bf16(void* ws, size_t ws_bytes, int64_t T,
                                     const w4a4_packed* desc, uint16_t* H, void* stream);
int w4a4_linear_gelu_bf16(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc,
                          uint16_t* H, void* ws, size_t ws_bytes, void* stream);

/* GELU-tanh between the FFN up (ffn.0) and down (ffn.2) projections named in
 * sec. 3.1 / 3.5: H = bf16_rne(gelu_tanh(bf16_rne(Y))), gelu_tanh(x) =
 * 0.5x(1+tanh(sqrt(2/pi)(x+0.044715x^3))) in fp32.  Y device fp32 [n], H device
 * bf16 [n].  Async. */
int w4a4_gelu_tanh_bf16(const float* Y, int64_t n, uint16_t* H, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): w4a4_linear with its
 * workspace in a fixed device array that the library holds on every GPU it runs on,
 * W4A4_NOALLOC_SCRATCH_BYTES long, until the process ends.  The caller still passes X
 * and Y (as for w4a4_linear).  The call makes no allocation and frees nothing; its
 * first call on a device looks up that device's copy of the array.
 *   - T tokens need w4a4_workspace_size(T, desc) bytes of it; a larger need returns
 *     W4A4_ERR_SCRATCH before anything is enqueued.
 *   - The results are those of w4a4_linear, bit for bit (same kernels, same plan).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in time on
 *     one GPU (other streams, other host threads) race and give undefined results.
 *     Nothing in the array needs to start at zero; it keeps the last call's contents.
 * Async on `stream`. */
#define W4A4_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int w4a4_linear_noalloc(const void* X, int x_dtype, int64_t T, const w4a4_packed* desc, float* Y,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
