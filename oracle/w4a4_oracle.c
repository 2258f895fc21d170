/*
 * w4a4_oracle.c -- CPU oracle for the W4A4 dual-branch linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or helper with the HIP library under bit_quantized_dit_amd/.
 *
 * Source of the method (cited by page title and section):
 *   [R]  "W4A4 Quantization for Inference on Wan2.2-I2V-A14B (ICME 2026
 *        Challenge)" -- the xllm-io paper-review blog page.
 *          sec. 2   pipeline order: calibrate -> fold -> split -> pack -> GEMM
 *          sec. 3.1 FFN activations: column max > 6, weight column max < 0.6
 *          sec. 3.2 SmoothQuant: Y = (X / s)(s * W), s_j = a_j^alpha / w_j^(1-alpha),
 *                   s folded into the master weights offline, activations
 *                   divided by s at inference and then quantized
 *          sec. 3.3 score_j = max_t |x_tj|, static top-k set O, J = complement,
 *                   Y = X_J W^(q)_J + X_O W^(hp)_O (W4A4 main, FP16/BF16 narrow)
 *          sec. 3.4 block-wise weight scales after fold + column extraction:
 *                   32x32 tiles or 128x1 K-major stripes, exponent stored
 *                   beside the 4-bit payload
 *          sec. 3.5 smooth first, then split on the columns still heavy
 *   [MX] MXFP4, the format named in [R] sec. 1 and sec. 2, as the OCP
 *        Microscaling (MX) formats define it: E2M1 elements
 *        {0, 0.5, 1, 1.5, 2, 3, 4, 6} with one E8M0 power-of-two scale per
 *        32 elements.  The pages name the format but do not define it.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes):
 *   - shared exponent E = floor(log2(amax)) - 2 (2 = exponent of the largest
 *     E2M1 value, 6 = 1.5 * 2^2), clamped below at -127; amax = 0 -> code 0;
 *     any NaN/Inf in the group -> scale code 0xFF and all nibbles 0.
 *   - elements round to nearest E2M1 value, ties to the even code, values
 *     beyond 6 saturate to 6; the sign bit is kept (so -0 -> nibble 0x8).
 *   - two E2M1 codes per byte, the even K index in the low nibble.
 *   - division x / s and the fold s * w are single IEEE binary32 operations
 *     (round to nearest even, subnormals kept).
 *   - the score is taken on the smoothed activations (sec. 3.5 "after the
 *     fold"), which equals fl32(max_t |x_tj| / s_j) because a correctly
 *     rounded division is monotone in its numerator.
 *   - both maxima are floored at 1e-5 before the power law.
 *   - top-k ties go to the smaller column index; O and J are ascending.
 *   - the J columns are compacted in ascending order, then cut into 32-blocks
 *     and zero padded to a multiple of 128.
 *   - the outlier branch uses raw (unsmoothed) bf16 X_O and bf16 W_O.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no FMA contraction; SSE arithmetic, so float ops are IEEE binary32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_LAYOUT_1X32 0
#define ORC_LAYOUT_TILE32 1   /* 32 K x 32 N tiles          ([R] sec. 3.4) */
#define ORC_LAYOUT_STRIPE128 2 /* 128 K x 1 N, K-major stripe ([R] sec. 3.4) */

/* ---------------------------------------------------------------- scalars */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }


/* bf16 -> float is exact: the 16 bits are the top half of a binary32. */
double orc_bf16_value(uint16_t h) { return (double)f32_from_bits(((uint32_t)h) << 16); }

/* Round a real number (given as a double) to the nearest bf16, ties to even
 * mantissa, by comparing it with its two bf16 neighbours. */
uint16_t orc_bf16_round_double(double d)
{
    if (isnan(d)) return (uint16_t)(signbit(d) ? 0xFFC0u : 0x7FC0u);
    int neg = signbit(d) ? 1 : 0;
    double m = fabs(d);
    /* largest bf16 with |value| <= m, found by truncating the binary32 that is
     * nearest below m.  Work with exact doubles: bf16 values are doubles. */
    if (isinf(m)) return (uint16_t)((neg ? 0x8000u : 0) | 0x7F80u);
    /* candidate magnitudes as bf16 bit patterns (without sign) */
    uint32_t lo = 0, hi;
    /* binary search over the 0x0000..0x7F80 ordered bf16 magnitudes */
    uint32_t a = 0, b = 0x7F80; /* value(a) <= m always (a=0); find largest <= m */
    while (a < b) {
        uint32_t mid = (a + b + 1) / 2;
        double v = (mid == 0x7F80) ? ldexp(1.0, 128) : orc_bf16_value((uint16_t)mid);
        if (v <= m) a = mid; else b = mid - 1;
    }
    lo = a;
    if (lo >= 0x7F80) return (uint16_t)((neg ? 0x8000u : 0) | 0x7F80u);
    hi = lo + 1;
    double vlo = orc_bf16_value((uint16_t)lo);
    /* 0x7F80 stands for 2^128, the point where IEEE rounding overflows */
    double vhi = (hi == 0x7F80) ? ldexp(1.0, 128) : orc_bf16_value((uint16_t)hi);
    uint32_t pick;
    if (m - vlo < vhi - m) pick = lo;
    else if (m - vlo > vhi - m) pick = hi;
    else pick = (lo & 1u) ? hi : lo;
    return (uint16_t)((neg ? 0x8000u : 0) | pick);
}

uint16_t orc_bf16_round_f32(float f) { return orc_bf16_round_double((double)f); }

/* E8M0 shared-scale code for a group whose largest magnitude is amax [MX]. */
uint8_t orc_e8m0_code(float amax)
{
    if (!isfinite(amax)) return 0xFF;
    if (amax == 0.0f) return 0x00;
    int e;
    (void)frexp((double)amax, &e);      /* amax = f * 2^e, f in [0.5, 1) */
    int E = (e - 1) - 2;                /* floor(log2 amax) - emax(E2M1) */
    if (E < -127) E = -127;
    return (uint8_t)(E + 127);
}

/* E2M1 code of the exact real v: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
 * even code, saturating at 6; bit 3 carries the sign of v. */
uint8_t orc_e2m1_code(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double m = fabs(v);
    uint8_t c;
    if (m <= 0.25) c = 0;        /* 0.25 is the 0|0.5 midpoint: tie -> 0   */
    else if (m < 0.75) c = 1;    /* 0.75 is the 0.5|1 midpoint: tie -> 1.0 */
    else if (m <= 1.25) c = 2;   /* 1.25: 1|1.5 -> 1.0                     */
    else if (m < 1.75) c = 3;    /* 1.75: 1.5|2 -> 2.0                     */
    else if (m <= 2.5) c = 4;    /* 2.5 : 2|3   -> 2.0                     */
    else if (m < 3.5) c = 5;     /* 3.5 : 3|4   -> 4.0                     */
    else if (m <= 5.0) c = 6;    /* 5   : 4|6   -> 4.0                     */
    else c = 7;                  /* (5, inf): 6, saturating                */
    return (uint8_t)(sign | c);
}

double orc_e2m1_value(uint8_t code)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[code & 7];
    return (code & 8) ? -v : v;
}

/* Element-wise versions, for exhaustive comparisons. */
void orc_e8m0_codes(const float* amax, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_code(amax[i]);
}

void orc_e2m1_codes(const double* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_code(v[i]);
}

void orc_bf16_round_f32_many(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round_f32(x[i]);
}

/* Quantize a group of n values that share one scale.  codes[i] gets the
 * nibble of vals[i]; *scale the E8M0 code. */
void orc_quant_group(const float* vals, int64_t n, uint8_t* codes, uint8_t* scale)
{
    int nonfinite = 0;
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(vals[i])) nonfinite = 1;
        else if (fabsf(vals[i]) > amax) amax = fabsf(vals[i]);
    }
    if (nonfinite) {
        *scale = 0xFF;
        for (int64_t i = 0; i < n; ++i) codes[i] = 0;
        return;
    }
    uint8_t sc = orc_e8m0_code(amax);
    int E = (int)sc - 127;
    *scale = sc;
    for (int64_t i = 0; i < n; ++i)
        codes[i] = orc_e2m1_code((double)vals[i] * ldexp(1.0, -E)); /* exact in double */
}

/* ------------------------------------------------------------ calibration */

static float load_x(const void* X, int is_bf16, int64_t idx)
{
    if (is_bf16) return f32_from_bits(((uint32_t)((const uint16_t*)X)[idx]) << 16);
    return ((const float*)X)[idx];
}

/* out[j] = max_r |X[r, j]| over a row-major [rows x cols] matrix ([R] sec. 3.2:
 * per-channel activation / weight magnitudes).  Returns 1 if any entry is
 * NaN or Inf, else 0. */
int orc_col_absmax(const void* X, int is_bf16, int64_t rows, int64_t cols, float* out)
{
    int bad = 0;
    for (int64_t j = 0; j < cols; ++j) out[j] = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            float a = fabsf(load_x(X, is_bf16, r * cols + j));
            if (!isfinite(a)) bad = 1;
            else if (a > out[j]) out[j] = a;
        }
    return bad;
}

/* s_j = a_j^alpha / w_j^(1-alpha) ([R] sec. 3.2), maxima floored at 1e-5,
 * evaluated in double and rounded once to binary32. */
void orc_smoothing(const float* act_scale, const float* weight_scale, int64_t d_in,
                   float alpha, float* s)
{
    const float floor_v = 1e-5f;
    for (int64_t j = 0; j < d_in; ++j) {
        float a = act_scale[j] > floor_v ? act_scale[j] : floor_v;
        float w = weight_scale[j] > floor_v ? weight_scale[j] : floor_v;
        double num = pow((double)a, (double)alpha);
        double den = pow((double)w, 1.0 - (double)alpha);
        s[j] = (float)(num / den);
    }
}

/* score_j = max_t |x_tj / s_j| ([R] sec. 3.3 on the smoothed activations,
 * sec. 3.5), computed as fl32(act_scale_j / s_j). */
void orc_scores(const float* act_scale, const float* s, int64_t d_in, float* score)
{
    for (int64_t j = 0; j < d_in; ++j) score[j] = act_scale[j] / s[j];
}

/* Static top-k outlier set O ([R] sec. 3.3): the k largest scores, ties to the
 * smaller index; O and its complement J are written in ascending order.
 * Selection by repeated arg-max keeps it obviously correct. */
void orc_select_outliers(const float* score, int64_t d_in, int32_t k, int32_t* O, int32_t* J)
{
    char* taken = (char*)calloc((size_t)(d_in > 0 ? d_in : 1), 1);
    for (int32_t i = 0; i < k; ++i) {
        int64_t best = -1;
        for (int64_t j = 0; j < d_in; ++j) {
            if (taken[j]) continue;
            if (best < 0 || score[j] > score[best]) best = j; /* strict: keeps smaller j on ties */
        }
        taken[best] = 1;
    }
    int32_t no = 0, nj = 0;
    for (int64_t j = 0; j < d_in; ++j) {
        if (taken[j]) O[no++] = (int32_t)j;
        else J[nj++] = (int32_t)j;
    }
    free(taken);
}

/* ---------------------------------------------------------- weight packing */

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Number of B_s bytes for a layout. */
int64_t orc_weight_scale_bytes(int64_t d_out, int64_t K_pad, int layout)
{
    if (layout == ORC_LAYOUT_1X32) return d_out * (K_pad / 32);
    if (layout == ORC_LAYOUT_STRIPE128) return d_out * (K_pad / 128);
    return (K_pad / 32) * cdiv(d_out, 32);
}

/* Fold s into the J rows of the weights, quantize them to MXFP4 with the given
 * scale-group layout, and keep the O rows as bf16 ([R] sec. 3.2 fold, sec. 3.3
 * split, sec. 3.4 block packing).
 *   W  : fp32 [d_out][d_in]  (nn.Linear orientation: W[n][j] = W_paper[j][n])
 *   Bq : [d_out][K_pad/2], Bs : layout dependent, WO : bf16 [d_out][k]        */
void orc_pack_weights(const float* W, int64_t d_in, int64_t d_out, const float* s,
                      const int32_t* J, int64_t K_J, const int32_t* O, int32_t k,
                      int layout, int64_t K_pad, uint8_t* Bq, uint8_t* Bs, uint16_t* WO)
{
    /* folded weights w'[n][p] = fl32(s_J[p] * W[n][J[p]]), zero for p >= K_J */
    float* wf = (float*)malloc((size_t)(d_out * K_pad > 0 ? d_out * K_pad : 1) * sizeof(float));
    uint8_t* code = (uint8_t*)malloc((size_t)(d_out * K_pad > 0 ? d_out * K_pad : 1));
    for (int64_t n = 0; n < d_out; ++n)
        for (int64_t p = 0; p < K_pad; ++p) {
            float v = 0.0f;
            if (p < K_J) {
                float sj = s[J[p]];
                float w = W[n * d_in + J[p]];
                v = sj * w;
            }
            wf[n * K_pad + p] = v;
        }
    /* scale groups */
    float grp[1024];
    uint8_t gc[1024];
    if (layout == ORC_LAYOUT_1X32 || layout == ORC_LAYOUT_STRIPE128) {
        int64_t g = (layout == ORC_LAYOUT_1X32) ? 32 : 128;
        for (int64_t n = 0; n < d_out; ++n)
            for (int64_t q = 0; q < K_pad / g; ++q) {
                for (int64_t i = 0; i < g; ++i) grp[i] = wf[n * K_pad + q * g + i];
                orc_quant_group(grp, g, gc, &Bs[n * (K_pad / g) + q]);
                for (int64_t i = 0; i < g; ++i) code[n * K_pad + q * g + i] = gc[i];
            }
    } else {
        int64_t ntile = cdiv(d_out, 32);
        for (int64_t kb = 0; kb < K_pad / 32; ++kb)
            for (int64_t nt = 0; nt < ntile; ++nt) {
                int64_t cnt = 0;
                for (int64_t n = nt * 32; n < nt * 32 + 32 && n < d_out; ++n)
                    for (int64_t i = 0; i < 32; ++i) grp[cnt++] = wf[n * K_pad + kb * 32 + i];
                orc_quant_group(grp, cnt, gc, &Bs[kb * ntile + nt]);
                cnt = 0;
                for (int64_t n = nt * 32; n < nt * 32 + 32 && n < d_out; ++n)
                    for (int64_t i = 0; i < 32; ++i) code[n * K_pad + kb * 32 + i] = gc[cnt++];
            }
    }
    for (int64_t n = 0; n < d_out; ++n)
        for (int64_t p = 0; p < K_pad; p += 2)
            Bq[n * (K_pad / 2) + p / 2] =
                (uint8_t)((code[n * K_pad + p] & 0xF) | ((code[n * K_pad + p + 1] & 0xF) << 4));
    for (int64_t n = 0; n < d_out; ++n)
        for (int32_t i = 0; i < k; ++i) WO[n * k + i] = orc_bf16_round_f32(W[n * d_in + O[i]]);
    free(wf);
    free(code);
}

/* ------------------------------------------------------------ act-prep */

/* Per token: divide the J columns by s ([R] sec. 3.2, IEEE binary32 divide),
 * quantize each 32-block of the compacted J row to MXFP4, and pass the O
 * columns through as bf16 ([R] sec. 3.3).
 *   Aq : [T][K_pad/2], As : [T][K_pad/32], XO : bf16 [T][k]                 */
void orc_act_prep(const void* X, int is_bf16, int64_t T, int64_t d_in, const float* s,
                  const int32_t* J, int64_t K_J, const int32_t* O, int32_t k, int64_t K_pad,
                  uint8_t* Aq, uint8_t* As, uint16_t* XO)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
        float blk[32];
        uint8_t c[32];
        for (int64_t b = 0; b < K_pad / 32; ++b) {
            for (int64_t i = 0; i < 32; ++i) {
                int64_t p = b * 32 + i;
                float xt = 0.0f;
                if (p < K_J) {
                    float x = load_x(X, is_bf16, t * d_in + J[p]);
                    float sj = s[J[p]];
                    xt = x / sj;
                }
                blk[i] = xt;
            }
            orc_quant_group(blk, 32, c, &As[t * (K_pad / 32) + b]);
            for (int64_t i = 0; i < 32; i += 2)
                Aq[t * (K_pad / 2) + b * 16 + i / 2] = (uint8_t)((c[i] & 0xF) | ((c[i + 1] & 0xF) << 4));
        }
        for (int32_t i = 0; i < k; ++i)
            XO[t * k + i] = orc_bf16_round_f32(load_x(X, is_bf16, t * d_in + O[i]));
    }
}

/* ------------------------------------------------------------ output */

static double weight_scale_pow2(const uint8_t* Bs, int64_t n, int64_t p, int64_t d_out,
                                int64_t K_pad, int layout)
{
    uint8_t c;
    if (layout == ORC_LAYOUT_1X32) c = Bs[n * (K_pad / 32) + p / 32];
    else if (layout == ORC_LAYOUT_STRIPE128) c = Bs[n * (K_pad / 128) + p / 128];
    else c = Bs[(p / 32) * cdiv(d_out, 32) + n / 32];
    if (c == 0xFF) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* One output element ([R] sec. 3.3 dual-branch formula), in double:
 *   Y[t,n] = sum_b 2^(Ea+Eb) sum_{p in b} e2m1(A[t,p]) e2m1(B[n,p])
 *          + sum_i bf16(XO[t,i]) bf16(WO[n,i])                                */
double orc_output_element(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                          const uint8_t* Bq, const uint8_t* Bs, const uint16_t* WO,
                          int64_t d_out, int64_t K_pad, int32_t k, int layout,
                          int64_t t, int64_t n)
{
    double y = 0.0;
    for (int64_t b = 0; b < K_pad / 32; ++b) {
        uint8_t ea = As[t * (K_pad / 32) + b];
        double sa = (ea == 0xFF) ? NAN : ldexp(1.0, (int)ea - 127);
        double sb = weight_scale_pow2(Bs, n, b * 32, d_out, K_pad, layout);
        double part = 0.0;
        for (int64_t i = 0; i < 32; ++i) {
            int64_t p = b * 32 + i;
            uint8_t ab = Aq[t * (K_pad / 2) + p / 2];
            uint8_t bb = Bq[n * (K_pad / 2) + p / 2];
            uint8_t ac = (p & 1) ? (ab >> 4) : (ab & 0xF);
            uint8_t bc = (p & 1) ? (bb >> 4) : (bb & 0xF);
            part += orc_e2m1_value(ac) * orc_e2m1_value(bc);
        }
        y += sa * sb * part;
    }
    for (int32_t i = 0; i < k; ++i)
        y += orc_bf16_value(XO[t * k + i]) * orc_bf16_value(WO[n * k + i]);
    return y;
}

/* Y for a list of (t, n) pairs. */
void orc_output_pairs(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                      const uint8_t* Bq, const uint8_t* Bs, const uint16_t* WO,
                      int64_t d_out, int64_t K_pad, int32_t k, int layout,
                      const int64_t* ts, const int64_t* ns, int64_t npairs, double* Y)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npairs; ++i)
        Y[i] = orc_output_element(Aq, As, XO, Bq, Bs, WO, d_out, K_pad, k, layout, ts[i], ns[i]);
}

/* Full Y [T][d_out]. */
void orc_output_full(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                     const uint8_t* Bq, const uint8_t* Bs, const uint16_t* WO,
                     int64_t T, int64_t d_out, int64_t K_pad, int32_t k, int layout, double* Y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < d_out; ++n)
            Y[t * d_out + n] = orc_output_element(Aq, As, XO, Bq, Bs, WO, d_out, K_pad, k, layout, t, n);
}

/* ------------------------------------------------------------ GELU (FFN) */

/* H = bf16( gelu_tanh( bf16(Y) ) ), the activation between the FFN up
 * projection (ffn.0) and down projection (ffn.2) named in [R] sec. 3.1 and
 * sec. 3.5.  gelu_tanh(x) = 0.5 x (1 + tanh(z)), z = sqrt(2/pi) (x + 0.044715 x^3).
 * Since 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2z)), the same function is evaluated
 * as x / (1 + exp(-2z)) in double and rounded once: the sum 1 + tanh(z) would
 * cancel every digit for z below about -19 (x below about -6), where the true
 * value is still far above the bf16 range limit.  exp(-2z) = +inf for very
 * negative x gives a signed zero, which is the correctly rounded result there.
 * A NaN input, and x = -inf (where the formula is -inf / inf), give the quiet
 * NaN with the sign of x. */
void orc_gelu_bf16(const float* Y, int64_t n, uint16_t* H)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double x = orc_bf16_value(orc_bf16_round_f32(Y[i]));
        double z = c * (x + 0.044715 * x * x * x);
        double g = x / (1.0 + exp(-2.0 * z));
        H[i] = isnan(g) ? (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u) : orc_bf16_round_double(g);
    }
}
