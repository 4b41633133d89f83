/*
 * oracle.c -- plain, slow, single-threaded CPU reference for LUT-based
 * approximate FP32 multiplication and the GEMM / Conv2D passes built on it.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The product library
 * never links, includes or calls it, and it shares no code, header, table or
 * helper with the HIP path.
 *
 * What it follows (all from "ApproxTrain: Fast Simulation of Approximate
 * Multipliers for DNN Training and Inference", arXiv 2209.04161):
 *   - Section V-A, Algorithm 1: generation of the mantissa-product lookup
 *     table from a C model of the multiplier, with carry detection by
 *     comparing the product's exponent with the un-normalised exponent.
 *   - Section V, Algorithm 2 (AMSim): one approximate product from the sign
 *     XOR, the exponent sum plus the table's carry, and the table's mantissa,
 *     with the zero / underflow / overflow cases.
 *   - Section III (Fig. 3): forward product, weight gradient (errors x
 *     activations) and preceding-layer gradient (weights x errors).
 *   - Section VI-B (Algorithms 3 and 4, Fig. 8): Conv2D forward as
 *     IM2COL + GEMM, weight gradient as IM2COL_Weight + GEMM, and the
 *     preceding-layer gradient as GEMM over the padded, dilated errors with
 *     the transposed-and-reversed filter.
 * Convolution is cross-correlation (the deep-learning convention, as in
 * "Binarized Convolutional Neural Networks for Efficient Inference on GPUs",
 * arXiv 1808.00209, eq. (3)).
 *
 * Readings taken where the pages are silent or loose (numbered as in the
 * design notes of the repository, where each is restated):
 *   R1  Table entry: 16 bits. Bit 15 is the carry, bits 14..0 are the top 15
 *       bits of the product's 23-bit fraction (truncated).
 *   R2  Operand mantissa = the top M bits of the 23-bit fraction (truncated).
 *   R3  Index = (mantissa of the first operand << M) | mantissa of the second.
 *   R4  The underflow / overflow tests use the exponent after the carry is
 *       added: e = EA + EB - 127 + carry; e <= 0 gives a signed zero and
 *       e >= 255 a signed infinity.
 *   R5  Subnormal inputs count as zero (the table assumes a hidden leading 1).
 *   R6  NaN in either input gives NaN (0x7FC00000); infinity times zero gives
 *       NaN; infinity times a non-zero gives a signed infinity. Otherwise a
 *       zero input gives a signed zero.
 *   R7  Algorithm 1 supports products whose mantissa lies in [1, 4): the
 *       product exponent equals the un-normalised exponent (carry 0) or
 *       exceeds it by one (carry 1). Anything else is rejected.
 *   R8  Convolution padding and dilation slots are zero operands that are
 *       multiplied (the IM2COL buffer holds zeros there), not omitted terms.
 *   R13 Sums are taken in double precision here; the sum of absolute
 *       products is returned beside each output for the error gate.
 *   R20 The FP32 order (the *_f32 functions below): the sum the library
 *       documents for its outputs, taken in single precision. The reduction
 *       sequence of an output is cut into chunks of L consecutive positions;
 *       each chunk is summed from +0 in ascending order, then the chunk sums
 *       are added from +0 in ascending order (one chunk when L covers the
 *       sequence). Every addition rounds to nearest even; with the native
 *       multiplier each step is a fused multiply-add (one rounding). The
 *       chunk length of each output is an input (the library reports it).
 *   R17 The native multiplier (Section V: the simulator can call the
 *       hardware multiplication instead of the table, the reference point
 *       of Fig. 6) is the exact product of the two floats, rounded only when
 *       it is added to a sum. The sums take it when no table is given.
 *   R19 Formats (1, E, M) with E = 1..8 exponent bits (Section V allows any
 *       exponent width from 1 to 8 once an exponent cast is supplied, and
 *       gives no cast). The
 *       format's exponent has bias b = 2^(E-1) - 1 and normal unbiased
 *       exponents 1-b .. b, IEEE style, without subnormals (the table
 *       assumes a hidden 1). Cast of an operand: a normal FP32 value whose
 *       unbiased exponent is below 1-b becomes a signed zero, above b a
 *       signed infinity; zero, Inf and NaN stay. Algorithm 2's underflow and
 *       overflow tests then use the format's range: the product's unbiased
 *       exponent (with the carry) below 1-b gives a signed zero, above b a
 *       signed infinity. E = 8 is FP32's range, so nothing changes there.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bit views of a float                                               */
/* ------------------------------------------------------------------ */
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t sign_of(uint32_t u) { return u >> 31; }
static uint32_t exp_of(uint32_t u) { return (u >> 23) & 0xFFu; }
static uint32_t frac_of(uint32_t u) { return u & 0x7FFFFFu; }

/* ------------------------------------------------------------------ */
/* C models of multipliers (the user-supplied approx_mul of Fig. 7)    */
/* ------------------------------------------------------------------ */

/* The exact multiplier: the hardware FP32 product. With M-bit operand
 * mantissas (M <= 11) the product of the two significands needs at most
 * 2M+2 <= 24 bits, so it is exact in FP32. */
float orc_mul_exact(float a, float b) { return a * b; }

/* Mitchell's logarithmic multiplier (J. N. Mitchell, "Computer
 * multiplication and division using binary logarithms", 1962), applied to
 * the significands of two normal floats. With a = (1+x)2^ea and
 * b = (1+y)2^eb, log2 is approximated by its chord: log2(1+x) ~ x. The
 * antilogarithm of ea+eb+x+y is then (1+x+y)2^(ea+eb) when x+y < 1, and
 * 2(x+y)2^(ea+eb) = (1+(x+y-1))2^(ea+eb+1) when x+y >= 1. Zero, subnormal,
 * infinite and NaN operands are not modelled: Algorithm 1 never passes them. */
float orc_mul_mitchell(float a, float b)
{
    uint32_t ua = bits_of(a), ub = bits_of(b);
    int ea = (int)exp_of(ua) - 127, eb = (int)exp_of(ub) - 127;
    double x = (double)frac_of(ua) / 8388608.0;
    double y = (double)frac_of(ub) / 8388608.0;
    double sig = (x + y < 1.0) ? 1.0 + x + y : 2.0 * (x + y);
    double v = ldexp(sig, ea + eb);
    if (sign_of(ua) ^ sign_of(ub)) v = -v;
    return (float)v;
}

/* ------------------------------------------------------------------ */
/* Algorithm 1: mantissa-product lookup table generation (Section V-A) */
/* ------------------------------------------------------------------ */

/* Fills lut[(ia << M) | ib] for every pair of M-bit mantissas. Returns 0, or
 * -1 for M out of [1, 11], or -2 when the model's product falls outside the
 * supported shape (reading R7).
 *
 * The operands are built with sign + and biased exponent 127 (value in
 * [1, 2)), so neither they nor their product can be a special case. The
 * un-normalised exponent of the product is 127 + 127 - 127 = 127; the carry
 * is set when the model's product has a larger exponent. */
int orc_lut_generate(int M, float (*approx_mul)(float, float), uint16_t *lut)
{
    if (M < 1 || M > 11) return -1;
    const uint32_t n = 1u << M;
    const uint32_t exp_a = 127, exp_b = 127;
    const int un_normalized_exp = (int)exp_a + (int)exp_b - 127;
    for (uint32_t ia = 0; ia < n; ++ia) {
        for (uint32_t ib = 0; ib < n; ++ib) {
            float A = float_of((exp_a << 23) | (ia << (23 - M)));
            float B = float_of((exp_b << 23) | (ib << (23 - M)));
            uint32_t c = bits_of(approx_mul(A, B));
            int real_exp = (int)exp_of(c);
            uint32_t carry;
            if (sign_of(c) != 0) return -2;
            if (real_exp == un_normalized_exp) carry = 0;
            else if (real_exp == un_normalized_exp + 1) carry = 1;
            else return -2;
            uint32_t mantissa15 = frac_of(c) >> 8; /* top 15 fraction bits */
            lut[(ia << M) | ib] = (uint16_t)((carry << 15) | mantissa15);
        }
    }
    return 0;
}

/* A synthetic multiplier: a table whose every entry's 15-bit mantissa field
 * is moved by delta[i] (+1 or -1 units of the field), saturating at 0 and
 * 0x7FFF; the carry bit is left as it is. delta comes from the caller. */
void orc_lut_perturb(int M, uint16_t *lut, const int8_t *delta)
{
    const uint32_t n = 1u << (2 * M);
    for (uint32_t i = 0; i < n; ++i) {
        int carry = lut[i] >> 15;
        int mant = lut[i] & 0x7FFF;
        mant += delta[i];
        if (mant < 0) mant = 0;
        if (mant > 0x7FFF) mant = 0x7FFF;
        lut[i] = (uint16_t)((carry << 15) | mant);
    }
}

/* ------------------------------------------------------------------ */
/* Exponent cast to a (1, E, M) format (reading R19)                   */
/* ------------------------------------------------------------------ */
/* FP32 biased exponents of the format's normal range: lowest and highest. */
static int fmt_lo(int E) { return 127 + 1 - ((1 << (E - 1)) - 1); }
static int fmt_hi(int E) { return 127 + ((1 << (E - 1)) - 1); }

uint32_t orc_cast_bits(uint32_t x, int E)
{
    uint32_t e = exp_of(x);
    if (e == 0 || e == 255) return x;                              /* zero, subnormal, Inf, NaN */
    if ((int)e < fmt_lo(E)) return sign_of(x) << 31;               /* below the format: zero */
    if ((int)e > fmt_hi(E)) return (sign_of(x) << 31) | 0x7F800000u;   /* above: infinity */
    return x;
}

/* ------------------------------------------------------------------ */
/* Algorithm 2: AMSim, one approximate product (Section V)             */
/* ------------------------------------------------------------------ */
/* The product of a and b in the format (1, E, M): both operands are cast to
 * the format first (R19), then Algorithm 2 runs with the format's range. */
uint32_t orc_amsim_bits_fmt(uint32_t a, uint32_t b, const uint16_t *lut, int M, int E)
{
    a = orc_cast_bits(a, E);
    b = orc_cast_bits(b, E);
    /* extract the mantissas (top M fraction bits) and form the index */
    uint32_t mant_a = frac_of(a) >> (23 - M);
    uint32_t mant_b = frac_of(b) >> (23 - M);
    uint32_t index = (mant_a << M) | mant_b;
    /* decouple the table entry into mantissa and carry; sign is the XOR */
    uint32_t entry = lut[index];
    uint32_t mantissa = entry & 0x7FFFu;
    uint32_t carry = entry >> 15;
    uint32_t sign = sign_of(a) ^ sign_of(b);

    /* classes (readings R5, R6) */
    uint32_t ea = exp_of(a), eb = exp_of(b);
    int a_nan = (ea == 255) && frac_of(a) != 0, b_nan = (eb == 255) && frac_of(b) != 0;
    int a_inf = (ea == 255) && frac_of(a) == 0, b_inf = (eb == 255) && frac_of(b) == 0;
    int a_zero = (ea == 0), b_zero = (eb == 0);
    if (a_nan || b_nan) return 0x7FC00000u;
    if (a_inf || b_inf) {
        if (a_zero || b_zero) return 0x7FC00000u;
        return (sign << 31) | 0x7F800000u;
    }
    if (a_zero || b_zero) return sign << 31;

    /* normal case: biased exponent with the carry (reading R4), tested
     * against the format's range (R19; FP32: 1..254) */
    int e = (int)ea + (int)eb - 127 + (int)carry;
    if (e < fmt_lo(E)) return sign << 31;
    if (e > fmt_hi(E)) return (sign << 31) | 0x7F800000u;
    return (sign << 31) | ((uint32_t)e << 23) | (mantissa << 8);
}

/* FP32 operands (E = 8) */
uint32_t orc_amsim_bits(uint32_t a, uint32_t b, const uint16_t *lut, int M)
{
    return orc_amsim_bits_fmt(a, b, lut, M, 8);
}

float orc_amsim(float a, float b, const uint16_t *lut, int M)
{
    return float_of(orc_amsim_bits(bits_of(a), bits_of(b), lut, M));
}

/* ------------------------------------------------------------------ */
/* The native multiplier (reading R17)                                 */
/* ------------------------------------------------------------------ */
/* Exact: two 24-bit significands give at most 48 bits (double holds 53),
 * and every product of two floats, subnormals included, lies inside
 * double's normal range. Inf * 0 and NaN inputs give NaN, as in IEEE-754. */
double orc_mul_native(float a, float b) { return (double)a * (double)b; }

/* the product the sums below use: Algorithm 2 with a table in the format
 * (1, E, M), the native multiplier when there is none (lut == NULL; E is
 * then unused) */
static double product(float a, float b, const uint16_t *lut, int M, int E)
{
    if (lut == NULL) return orc_mul_native(a, b);
    return (double)float_of(orc_amsim_bits_fmt(bits_of(a), bits_of(b), lut, M, E));
}

/* element-wise products of two bit arrays (for exhaustive checks) */
void orc_amsim_many(int64_t count, const uint32_t *a, const uint32_t *b,
                    const uint16_t *lut, int M, int E, uint32_t *out)
{
    for (int64_t t = 0; t < count; ++t) out[t] = orc_amsim_bits_fmt(a[t], b[t], lut, M, E);
}

/* ------------------------------------------------------------------ */
/* GEMM: C = op(A) op(B) with every product approximate                */
/* ------------------------------------------------------------------ */
/* Row-major operands. op(A)(i,p) = transA ? A[p*lda+i] : A[i*lda+p];
 * op(B)(p,j) = transB ? B[j*ldb+p] : B[p*ldb+j]. The first operand of each
 * product is op(A)(i,p), the second op(B)(p,j) (reading R3). */
static void gemm_one(int transA, int transB, int i, int j, int k,
                     const float *A, long lda, const float *B, long ldb,
                     const uint16_t *lut, int M, int E, double *r, double *s)
{
    double sum = 0.0, abs_sum = 0.0;
    for (int p = 0; p < k; ++p) {
        float a = transA ? A[(long)p * lda + i] : A[(long)i * lda + p];
        float b = transB ? B[(long)j * ldb + p] : B[(long)p * ldb + j];
        double prod = product(a, b, lut, M, E);
        sum += prod;
        abs_sum += fabs(prod);
    }
    *r = sum;
    *s = abs_sum;
}

void orc_gemm(int transA, int transB, int m, int n, int k,
              const float *A, int lda, const float *B, int ldb,
              const uint16_t *lut, int M, int E, double *R, double *S)
{
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j)
            gemm_one(transA, transB, i, j, k, A, lda, B, ldb, lut, M, E,
                     &R[(long)i * n + j], &S[(long)i * n + j]);
}

/* the same sums at chosen (row, column) pairs only */
void orc_gemm_at(int transA, int transB, int m, int n, int k,
                 const float *A, int lda, const float *B, int ldb,
                 const uint16_t *lut, int M, int E,
                 int64_t count, const int32_t *rows, const int32_t *cols,
                 double *R, double *S)
{
    (void)m; (void)n;
    for (int64_t t = 0; t < count; ++t)
        gemm_one(transA, transB, rows[t], cols[t], k, A, lda, B, ldb, lut, M, E, &R[t], &S[t]);
}

/* ------------------------------------------------------------------ */
/* Conv2D, NHWC activations and RSCK (HWIO) weights                    */
/* ------------------------------------------------------------------ */
typedef struct {
    int N, H, W, C, K, R, S, sh, sw, ph, pw, P, Q;
} geom;

static geom make_geom(int N, int H, int W, int C, int K, int R, int S,
                      int sh, int sw, int ph, int pw)
{
    geom g = {N, H, W, C, K, R, S, sh, sw, ph, pw, 0, 0};
    g.P = (H + 2 * ph - R) / sh + 1;
    g.Q = (W + 2 * pw - S) / sw + 1;
    return g;
}

/* activation value with zero padding outside the image (reading R8) */
static float x_at(const geom *g, const float *x, int n, int h, int w, int c)
{
    if (h < 0 || h >= g->H || w < 0 || w >= g->W) return 0.0f;
    return x[(((long)n * g->H + h) * g->W + w) * g->C + c];
}

/* Padded, dilated errors (Section VI-B, the IM2COL_PLG input): at an input
 * coordinate offset hh = h + ph - r the error of output row hh / sh is used
 * when hh is a multiple of the stride and in range, and zero otherwise. */
static float dilated_dy_at(const geom *g, const float *dy, int n, int hh, int ww, int k)
{
    if (hh < 0 || ww < 0) return 0.0f;
    if (hh % g->sh != 0 || ww % g->sw != 0) return 0.0f;
    int p = hh / g->sh, q = ww / g->sw;
    if (p >= g->P || q >= g->Q) return 0.0f;
    return dy[(((long)n * g->P + p) * g->Q + q) * g->K + k];
}

static float w_at(const geom *g, const float *w, int r, int s, int c, int k)
{
    return w[(((long)r * g->S + s) * g->C + c) * g->K + k];
}

/* forward: y[n,p,q,k] = sum_{r,s,c} approx(x[n, p*sh-ph+r, q*sw-pw+s, c], w[r,s,c,k]) */
static void fwd_one(const geom *g, const float *x, const float *w, long idx,
                    const uint16_t *lut, int M, int E, double *r_out, double *s_out)
{
    int k = (int)(idx % g->K); idx /= g->K;
    int q = (int)(idx % g->Q); idx /= g->Q;
    int p = (int)(idx % g->P);
    int n = (int)(idx / g->P);
    double sum = 0.0, abs_sum = 0.0;
    for (int r = 0; r < g->R; ++r)
        for (int s = 0; s < g->S; ++s)
            for (int c = 0; c < g->C; ++c) {
                float a = x_at(g, x, n, p * g->sh - g->ph + r, q * g->sw - g->pw + s, c);
                double prod = product(a, w_at(g, w, r, s, c, k), lut, M, E);
                sum += prod;
                abs_sum += fabs(prod);
            }
    *r_out = sum;
    *s_out = abs_sum;
}

/* preceding-layer gradient:
 * dx[n,h,w,c] = sum_{r,s,k} approx(D[n, h+ph-r, w+pw-s, k], w[r,s,c,k])
 * with D the padded, dilated errors above. */
static void dgrad_one(const geom *g, const float *dy, const float *w, long idx,
                      const uint16_t *lut, int M, int E, double *r_out, double *s_out)
{
    int c = (int)(idx % g->C); idx /= g->C;
    int ww = (int)(idx % g->W); idx /= g->W;
    int h = (int)(idx % g->H);
    int n = (int)(idx / g->H);
    double sum = 0.0, abs_sum = 0.0;
    for (int r = 0; r < g->R; ++r)
        for (int s = 0; s < g->S; ++s)
            for (int k = 0; k < g->K; ++k) {
                float a = dilated_dy_at(g, dy, n, h + g->ph - r, ww + g->pw - s, k);
                double prod = product(a, w_at(g, w, r, s, c, k), lut, M, E);
                sum += prod;
                abs_sum += fabs(prod);
            }
    *r_out = sum;
    *s_out = abs_sum;
}

/* weight gradient:
 * dw[r,s,c,k] = sum_{n,p,q} approx(x[n, p*sh-ph+r, q*sw-pw+s, c], dy[n,p,q,k]) */
static void wgrad_one(const geom *g, const float *x, const float *dy, long idx,
                      const uint16_t *lut, int M, int E, double *r_out, double *s_out)
{
    int k = (int)(idx % g->K); idx /= g->K;
    int c = (int)(idx % g->C); idx /= g->C;
    int s = (int)(idx % g->S);
    int r = (int)(idx / g->S);
    double sum = 0.0, abs_sum = 0.0;
    for (int n = 0; n < g->N; ++n)
        for (int p = 0; p < g->P; ++p)
            for (int q = 0; q < g->Q; ++q) {
                float a = x_at(g, x, n, p * g->sh - g->ph + r, q * g->sw - g->pw + s, c);
                float b = dy[(((long)n * g->P + p) * g->Q + q) * g->K + k];
                double prod = product(a, b, lut, M, E);
                sum += prod;
                abs_sum += fabs(prod);
            }
    *r_out = sum;
    *s_out = abs_sum;
}

/* Full passes (idx == NULL: every output in order) or chosen outputs (flat
 * indices into the NHWC / RSCK output). */
void orc_conv2d_fwd(int N, int H, int W, int C, int K, int R, int S,
                    int sh, int sw, int ph, int pw,
                    const float *x, const float *w, const uint16_t *lut, int M, int E,
                    int64_t count, const int64_t *idx, double *Y, double *YS)
{
    geom g = make_geom(N, H, W, C, K, R, S, sh, sw, ph, pw);
    long total = (long)N * g.P * g.Q * K;
    long cnt = idx ? (long)count : total;
    for (long t = 0; t < cnt; ++t)
        fwd_one(&g, x, w, idx ? (long)idx[t] : t, lut, M, E, &Y[t], &YS[t]);
}

void orc_conv2d_dgrad(int N, int H, int W, int C, int K, int R, int S,
                      int sh, int sw, int ph, int pw,
                      const float *dy, const float *w, const uint16_t *lut, int M, int E,
                      int64_t count, const int64_t *idx, double *DX, double *DXS)
{
    geom g = make_geom(N, H, W, C, K, R, S, sh, sw, ph, pw);
    long total = (long)N * H * W * C;
    long cnt = idx ? (long)count : total;
    for (long t = 0; t < cnt; ++t)
        dgrad_one(&g, dy, w, idx ? (long)idx[t] : t, lut, M, E, &DX[t], &DXS[t]);
}

void orc_conv2d_wgrad(int N, int H, int W, int C, int K, int R, int S,
                      int sh, int sw, int ph, int pw,
                      const float *x, const float *dy, const uint16_t *lut, int M, int E,
                      int64_t count, const int64_t *idx, double *DW, double *DWS)
{
    geom g = make_geom(N, H, W, C, K, R, S, sh, sw, ph, pw);
    long total = (long)R * S * C * K;
    long cnt = idx ? (long)count : total;
    for (long t = 0; t < cnt; ++t)
        wgrad_one(&g, x, dy, idx ? (long)idx[t] : t, lut, M, E, &DW[t], &DWS[t]);
}

/* ------------------------------------------------------------------ */
/* The same sums in FP32, in the documented order (reading R20)        */
/* ------------------------------------------------------------------ */
/* Running state of one FP32 sum: `total` holds the finished chunks, `part`
 * the chunk in progress, which is chunk number `cur` (position t lies in
 * chunk t / L). Positions must come in ascending order. */
typedef struct {
    float total, part;
    int64_t L, cur;
} f32sum;

static void f32_begin(f32sum *f, int64_t L)
{
    f->total = 0.0f;
    f->part = 0.0f;
    f->L = L > 0 ? L : 1;
    f->cur = 0;
}

/* position t of the sequence: when it lies past the chunk in progress, that
 * chunk's sum is added to the total and a new chunk starts from +0 (a chunk
 * with no product in between adds +0, which changes nothing) */
static void f32_at(f32sum *f, int64_t t)
{
    while (t / f->L > f->cur) {
        f->total = f->total + f->part;
        f->part = 0.0f;
        ++f->cur;
    }
}

/* add the product of a and b (approximate, or native: fused) at position t */
static void f32_add(f32sum *f, int64_t t, float a, float b, const uint16_t *lut, int M, int E)
{
    f32_at(f, t);
    if (lut == NULL)
        f->part = fmaf(a, b, f->part);
    else
        f->part = f->part + float_of(orc_amsim_bits_fmt(bits_of(a), bits_of(b), lut, M, E));
}

static float f32_end(f32sum *f)
{
    f->total = f->total + f->part;
    return f->total;
}

/* GEMM outputs (rows[t], cols[t]) with reduction chunks of chunk[t]
 * positions of the reduction index p */
void orc_gemm_f32_at(int transA, int transB, int m, int n, int k,
                     const float *A, int lda, const float *B, int ldb,
                     const uint16_t *lut, int M, int E,
                     int64_t count, const int32_t *rows, const int32_t *cols,
                     const int64_t *chunk, float *out)
{
    (void)m; (void)n;
    for (int64_t t = 0; t < count; ++t) {
        int i = rows[t], j = cols[t];
        f32sum f;
        f32_begin(&f, chunk[t]);
        for (int p = 0; p < k; ++p) {
            float a = transA ? A[(long)p * lda + i] : A[(long)i * lda + p];
            float b = transB ? B[(long)j * ldb + p] : B[(long)p * ldb + j];
            f32_add(&f, p, a, b, lut, M, E);
        }
        out[t] = f32_end(&f);
    }
}

/* Conv2D outputs at flat indices idx[t] with chunks of chunk[t] positions.
 * Reduction sequences (positions in ascending order; C4 and K4 are C and K
 * rounded up to a multiple of 4, the positions past C or K holding no
 * product):
 *   fwd:   (r, s, c) at position (r*S + s)*C4 + c;
 *   dgrad: (r, s, k) at position ((R-1-r)*S + (S-1-s))*K4 + k, i.e. the
 *          filter taps in reverse order (the transposed, reversed filter of
 *          Section VI-B), channels ascending;
 *   wgrad: (n, p, q) at position (n*P + p)*Q + q. */
void orc_conv2d_f32(int pass, int N, int H, int W, int C, int K, int R, int S,
                    int sh, int sw, int ph, int pw,
                    const float *t1, const float *t2, const uint16_t *lut, int M, int E,
                    int64_t count, const int64_t *idx, const int64_t *chunk, float *out)
{
    geom g = make_geom(N, H, W, C, K, R, S, sh, sw, ph, pw);
    const int C4 = (C + 3) / 4 * 4, K4 = (K + 3) / 4 * 4;
    for (int64_t t = 0; t < count; ++t) {
        long o = (long)idx[t];
        f32sum f;
        f32_begin(&f, chunk[t]);
        if (pass == 0) {                         /* y[n,p,q,k]: t1 = x, t2 = w */
            int k = (int)(o % K); o /= K;
            int q = (int)(o % g.Q); o /= g.Q;
            int p = (int)(o % g.P);
            int n = (int)(o / g.P);
            for (int r = 0; r < R; ++r)
                for (int s = 0; s < S; ++s)
                    for (int c = 0; c < C; ++c) {
                        float a = x_at(&g, t1, n, p * sh - ph + r, q * sw - pw + s, c);
                        f32_add(&f, ((int64_t)r * S + s) * C4 + c, a, w_at(&g, t2, r, s, c, k), lut, M, E);
                    }
        } else if (pass == 1) {                  /* dx[n,h,w,c]: t1 = dy, t2 = w */
            int c = (int)(o % C); o /= C;
            int ww = (int)(o % W); o /= W;
            int h = (int)(o % H);
            int n = (int)(o / H);
            for (int r = R - 1; r >= 0; --r)
                for (int s = S - 1; s >= 0; --s)
                    for (int k = 0; k < K; ++k) {
                        float a = dilated_dy_at(&g, t1, n, h + ph - r, ww + pw - s, k);
                        int64_t pos = ((int64_t)(R - 1 - r) * S + (S - 1 - s)) * K4 + k;
                        f32_add(&f, pos, a, w_at(&g, t2, r, s, c, k), lut, M, E);
                    }
        } else {                                 /* dw[r,s,c,k]: t1 = x, t2 = dy */
            int k = (int)(o % K); o /= K;
            int c = (int)(o % C); o /= C;
            int s = (int)(o % S);
            int r = (int)(o / S);
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < g.P; ++p)
                    for (int q = 0; q < g.Q; ++q) {
                        float a = x_at(&g, t1, n, p * sh - ph + r, q * sw - pw + s, c);
                        float b = t2[(((long)n * g.P + p) * g.Q + q) * K + k];
                        f32_add(&f, ((int64_t)n * g.P + p) * g.Q + q, a, b, lut, M, E);
                    }
        }
        out[t] = f32_end(&f);
    }
}
