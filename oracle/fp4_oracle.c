/*
 * fp4_oracle.c -- plain, slow, obviously-correct CPU oracle for block-wise
 * microscaling FP4 quantization (MXFP4, NVFP4), its dequantization, the error
 * metrics, and the FP4 x FP4 block-scaled matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library, and it is never on
 * the product path.
 *
 * Every function states the passage it follows.  Pages are cited by title:
 *   [MRGPTQ]  "Bridging the Gap Between Promise and Performance for Microscaling
 *             FP4 Quantization"
 *   [VS]      "NVFP4 vs MXFP4: 4-Bit Floating Point for LLM Training and
 *             Inference (2026)"
 *   [PORT]    "Portable FP4 Quantization for Heterogeneous Accelerators"
 *   [PROD]    "Microscaling Formats in Production LLM Inference: NVFP4 vs. MXFP4
 *             Architecture, Block Quantization, Kernel Scaling, and Perplexity
 *             Degradation"
 *
 * Readings where the pages are silent or disagree (each one is listed with its
 * reason in the design notes of the repository):
 *   - E2M1 ties go to the even code (round-to-nearest-even), following [VS]
 *     "The training recipe, piece by piece" and [PROD] "Microscaled Residual
 *     GPTQ"; [VS]'s emulation breaks ties toward zero but says it ignores the
 *     tie rules.
 *   - Values beyond 6 saturate to +-6 ([VS] emulation clips to [0, 6]).
 *   - MXFP4 exponent = floor(log2(block amax)) - 2, taken exactly from the
 *     binary exponent, clamped to [-127, 127]; an all-zero block gets code 0.
 *   - NVFP4: ts = amax_tensor / (6*448) in fp32; block scale code =
 *     E4M3(RNE, saturating at 448) of (amax_block / 6) / ts, all in fp32 in that
 *     order; elements use q = fl32(x / s) with s = fl32(e4m3 * ts).  A block whose
 *     s is zero stores all-zero element codes.
 *   - Hadamard: Sylvester order, normalised by 1/sqrt(n), n = block size.
 *   - Element 2i goes in the low nibble of byte i.
 *   - The sign bit of an element code is the sign bit of q, so a negative value
 *     that rounds to zero stores code 0x8.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * Floating point follows IEEE-754 binary32/binary64 exactly as written: no
 * contraction into FMA, no reassociation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_MXFP4 0
#define ORA_NVFP4 1
#define ORA_MXINT4 2
#define ORA_NVINT4 3

#define ORA_OK 0
#define ORA_EINVAL -1

int ora_dequantize_rot(int fmt, const uint8_t *codes, const uint8_t *scales, float ts,
                       long rows, long cols, int rot_n, const uint32_t *signs, float *y);

/* ------------------------------------------------------------------------ */
/* E2M1 element ([MRGPTQ] format definitions; [VS] "The E2M1 element: only   */
/* eight magnitudes"; [PROD] "The Numerical Ceiling of Standard 4-Bit        */
/* Floating Point", bit layout: 1 sign bit, 2 exponent bits with bias 1,     */
/* 1 mantissa bit).                                                          */
/* ------------------------------------------------------------------------ */

/* Value of a 4-bit code, decoded from its fields. */
double ora_e2m1_decode(int code)
{
    int sign = (code >> 3) & 1;
    int exp_field = (code >> 1) & 3;
    int man = code & 1;
    double mag;
    if (exp_field == 0)            /* subnormal: 0.m x 2^(1-bias) */
        mag = 0.5 * man;
    else                           /* normal: 1.m x 2^(e-bias) */
        mag = ldexp(1.0 + 0.5 * man, exp_field - 1);
    return sign ? -mag : mag;
}

/* Code of the grid point nearest to q.  |q| > 6 saturates to 6.  Ties go to
 * the even code (mantissa bit 0).  The sign bit is signbit(q). */
int ora_e2m1_encode(float q)
{
    int neg = signbit(q) ? 1 : 0;
    double a = fabs((double)q);
    if (a > 6.0)
        a = 6.0;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - ora_e2m1_decode(c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (neg << 3) | best;
}

/* ------------------------------------------------------------------------ */
/* E4M3 scale ([MRGPTQ] NVFP4 definition; [VS] "Why the scale format matters */
/* more than the element" (maximum 448) and the emulation's e4m3 rounding:   */
/* 3 mantissa bits, minimum normal exponent -6, subnormal step 2^-9).        */
/* OCP E4M3 "FN": bias 7, no infinities, 0x7F / 0xFF are NaN.                */
/* ------------------------------------------------------------------------ */

double ora_e4m3_decode(int code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);              /* 0.mmm x 2^(1-7) */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);       /* 1.mmm x 2^(e-7) */
    return sign ? -mag : mag;
}

/* Code of the non-negative E4M3 value nearest to t, after clipping t to
 * [0, 448].  Ties go to the even code.  t must be >= 0 (or +inf). */
int ora_e4m3_encode(float t)
{
    double a = (double)t;
    if (!(a > 0.0))
        return 0;
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(a - ora_e4m3_decode(c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* E8M0 scale value 2^(code-127) ([MRGPTQ] MXFP4 definition; [PROD] "Format  */
/* Specifications": exponent-only, bias 127).  Code 255 is not produced.     */
double ora_e8m0_decode(int code)
{
    return ldexp(1.0, code - 127);
}

/* ------------------------------------------------------------------------ */
/* INT4 element ([MRGPTQ] "MXINT4 and NVINT4": the MXFP4 / NVFP4 layouts     */
/* with a 4-bit integer element).  Reading: a signed two's-complement nibble */
/* used symmetrically, values -7 .. 7 (the pattern 0x8 = -8 is never         */
/* produced), nearest integer with ties to even, saturating at +-7.  There  */
/* is no negative zero.                                                      */
/* ------------------------------------------------------------------------ */

double ora_int4_decode(int code)
{
    int c = code & 15;
    return c >= 8 ? (double)(c - 16) : (double)c;
}

int ora_int4_encode(float q)
{
    double a = fabs((double)q);
    if (a > 7.0)
        a = 7.0;
    int best = 0;
    double bestd = INFINITY;
    for (int m = 0; m <= 7; ++m) {
        double d = fabs(a - (double)m);
        if (d < bestd || (d == bestd && (m & 1) == 0)) {
            best = m;
            bestd = d;
        }
    }
    int v = signbit(q) ? -best : best;
    return v & 15;
}

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers for stochastic rounding: Philox4x32-10       */
/* (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as     */
/* easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64-bit multiplies and  */
/* xors with the key, the key advanced by two Weyl constants between rounds. */
/* ------------------------------------------------------------------------ */

void ora_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The uniform number in [0, 1) of element e of a tensor for stochastic
 * rounding: counter (e / 4 low word, e / 4 high word, 0, 0), key = seed, word
 * e % 4 of the output, top 24 bits times 2^-24 (exact). */
static double sr_uniform(uint64_t e, const uint32_t seed[2])
{
    uint32_t ctr[4] = {(uint32_t)(e >> 2), (uint32_t)(e >> 34), 0u, 0u};
    uint32_t out[4];
    ora_philox4x32_10(ctr, seed, out);
    return (double)(out[e & 3] >> 8) * 0x1p-24;
}

/* Stochastic rounding onto the E2M1 grid ([VS] "Stochastic rounding": up or
 * down with probability proportional to proximity, so the expected value is
 * the input): a = min(|q|, 6) between neighbours lo <= a < hi rounds up when
 * u < (a - lo) / (hi - lo).  Grid points stay put; the sign bit is signbit(q). */
int ora_e2m1_encode_sr(float q, double u)
{
    int neg = signbit(q) ? 1 : 0;
    double a = fabs((double)q);
    if (a > 6.0)
        a = 6.0;
    int lo = 0;
    for (int c = 0; c < 8; ++c)
        if (ora_e2m1_decode(c) <= a)
            lo = c;
    int mag = lo;
    if (lo < 7 && ora_e2m1_decode(lo) < a) {
        double glo = ora_e2m1_decode(lo), ghi = ora_e2m1_decode(lo + 1);
        double p = (a - glo) / (ghi - glo);
        if (u < p)
            mag = lo + 1;
    }
    return (neg << 3) | mag;
}

/* Block size of a format (0: not a format). */
static int fmt_block(int fmt)
{
    if (fmt == ORA_MXFP4 || fmt == ORA_MXINT4)
        return 32;
    if (fmt == ORA_NVFP4 || fmt == ORA_NVINT4)
        return 16;
    return 0;
}

/* E8M0 block scales (MX) rather than E4M3 block scales and a tensor scale. */
static int fmt_mx(int fmt)
{
    return fmt == ORA_MXFP4 || fmt == ORA_MXINT4;
}

static int fmt_int(int fmt)
{
    return fmt == ORA_MXINT4 || fmt == ORA_NVINT4;
}

static double elem_decode(int fmt, int code)
{
    return fmt_int(fmt) ? ora_int4_decode(code) : ora_e2m1_decode(code);
}

static int elem_encode(int fmt, float q)
{
    return fmt_int(fmt) ? ora_int4_encode(q) : ora_e2m1_encode(q);
}

/* ------------------------------------------------------------------------ */
/* Block Hadamard rotation ([MRGPTQ]: rotations at the group level, matching */
/* the quantization group size, Q(W H_k) Q(X H_k)^T; [PORT] section 2.3:     */
/* block-local orthogonal transform, norm preserving, eq. (2)).              */
/* ------------------------------------------------------------------------ */

/* Entry (i, j) of the unnormalised Sylvester Hadamard matrix of order 2^m. */
static int had_entry(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* Sign of element i of a rotation group: bit i of the 128-bit mask (word
 * i / 32, bit i % 32) set means negative ("randomized Hadamard": a random
 * diagonal of +-1 before the transform, [PROD] "Orthogonal Rotations" and
 * [VS] "Random Hadamard transforms").  A NULL mask is all positive. */
static double sign_of(const uint32_t *signs, int i)
{
    if (!signs)
        return 1.0;
    return ((signs[i >> 5] >> (i & 31)) & 1u) ? -1.0 : 1.0;
}

/* Forward (inverse = 0): y = fl32( (H D x) / sqrt(n) ) per group of n, with D
 * the sign diagonal; inverse = 1: y = D fl32( (H x) / sqrt(n) ), the inverse
 * of the forward map (H symmetric, H H = n I, D D = I).  Sums and the division
 * in double, one rounding.  n a power of two dividing cols; no aliasing. */
int ora_rotate_signed(const float *x, float *y, long rows, long cols, int n,
                      const uint32_t *signs, int inverse)
{
    if (n <= 0 || n > 128 || (n & (n - 1)) != 0 || cols % n != 0)
        return ORA_EINVAL;
    double root = sqrt((double)n);
    for (long r = 0; r < rows; ++r) {
        for (long b = 0; b < cols / n; ++b) {
            const float *xb = x + r * cols + b * n;
            float *yb = y + r * cols + b * n;
            for (int j = 0; j < n; ++j) {
                double s = 0.0;
                for (int i = 0; i < n; ++i) {
                    double xi = (double)xb[i];
                    if (!inverse)
                        xi *= sign_of(signs, i);
                    s += xi * had_entry(i, j);
                }
                float v = (float)(s / root);
                yb[j] = inverse ? (float)(sign_of(signs, j) * v) : v;
            }
        }
    }
    return ORA_OK;
}

/* y[r, b*n + j] = fl32( (sum_i x[r, b*n + i] * H[i][j]) / sqrt(n) ), the sum
 * and the division carried out in double.  n must be a power of two and
 * divide cols.  x and y may not alias. */
int ora_rotate(const float *x, float *y, long rows, long cols, int n)
{
    return ora_rotate_signed(x, y, rows, cols, n, NULL, 0);
}

/* ------------------------------------------------------------------------ */
/* Quantization.                                                             */
/* ------------------------------------------------------------------------ */

static float block_amax(const float *v, int n)
{
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m)
            m = a;
    }
    return m;
}

/* MXFP4 shared exponent of a block: floor(log2(amax)) - 2, clamped to
 * [-127, 127] ([VS] "A worked example, by hand" and the emulation's mxfp4;
 * [VS] "Why the scale format matters": E8M0 spans 2^-127 .. 2^127).
 * floor(log2(amax)) is read from frexp, which is exact: amax = f * 2^E with
 * f in [0.5, 1), so floor(log2(amax)) = E - 1. */
static int mx_exponent(float amax)
{
    if (amax == 0.0f)
        return -127;
    int E;
    (void)frexp((double)amax, &E);
    int e = (E - 1) - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

static void put_code(uint8_t *row_codes, long k, int code)
{
    if ((k & 1) == 0)
        row_codes[k >> 1] = (uint8_t)((row_codes[k >> 1] & 0xF0) | (code & 0xF));
    else
        row_codes[k >> 1] = (uint8_t)((row_codes[k >> 1] & 0x0F) | ((code & 0xF) << 4));
}

static int get_code(const uint8_t *row_codes, long k)
{
    return (k & 1) ? (row_codes[k >> 1] >> 4) & 0xF : row_codes[k >> 1] & 0xF;
}

/* Scale-selection rules ([MRGPTQ] section 4.1 and the W4A4 baselines:
 * absmax scales for RTN, "MSE scale optimization" / "format-specific scale
 * search" for MR-GPTQ's weights; [VS] "The E2M1 element": the best scale does
 * not always put the block maximum on 6, and "Follow-on research": Four Over
 * Six maps the maximum of some blocks to 4 instead of 6). */
#define ORA_SCALE_ABSMAX 0
#define ORA_SCALE_MSE 1
#define ORA_SCALE_FOUR_OVER_SIX 2

/* Element codes of the G values yb at scale code sc: q = fl32(y / s) rounded
 * onto the E2M1 grid.  MXFP4: s = 2^(sc-127).  NVFP4: s = fl32(e4m3(sc) * ts);
 * a zero s gives all-zero codes. */
static void block_encode(int fmt, const float *yb, int G, int sc, float tsv, int *code)
{
    float s = fmt_mx(fmt) ? ldexpf(1.0f, sc - 127) : (float)ora_e4m3_decode(sc) * tsv;
    for (int i = 0; i < G; ++i)
        code[i] = s != 0.0f ? elem_encode(fmt, yb[i] / s) : 0;
}

/* Dequantized value of one element (as ora_dequantize computes it, in fp32). */
static float element_value(int fmt, int code, int sc, float tsv)
{
    if (fmt_mx(fmt))
        return (float)elem_decode(fmt, code) * ldexpf(1.0f, sc - 127);
    float inner = (float)(elem_decode(fmt, code) * ora_e4m3_decode(sc));
    return inner * tsv;
}

/* Squared reconstruction error of a block quantized at scale code sc, in
 * fp32: d = fl32(y - y^), acc = fma(d, d, acc) in element order.  This is
 * the number the search compares, so the decision is taken in the precision
 * the GPU kernel uses (one lane holds one block). */
static float block_sse(int fmt, const float *yb, int G, int sc, float tsv, const int *code)
{
    float acc = 0.0f;
    for (int i = 0; i < G; ++i) {
        float d = yb[i] - element_value(fmt, code[i], sc, tsv);
        acc = fmaf(d, d, acc);
    }
    return acc;
}

/* NVFP4 E4M3 block-scale code that maps the block maximum amax onto `top`
 * (6 for the standard rule, 4 for the alternative of Four Over Six):
 * E4M3(fl32(fl32(amax / top) / ts)). */
static int nv_scale_code(float amax, float top, float tsv)
{
    float t = (amax / top) / tsv;
    return ora_e4m3_encode(t);
}

/* NV per-tensor scale of the n (rotated) values y ([VS] Figure 2: the global
 * amax sets the fp32 tensor scale): amax / (6 * 448) for NVFP4, amax /
 * (7 * 448) for NVINT4. */
static float tensor_scale(int fmt, const float *y, long n)
{
    float gamax = 0.0f;
    for (long i = 0; i < n; ++i) {
        float a = fabsf(y[i]);
        if (a > gamax)
            gamax = a;
    }
    float tsv;
    if (fmt == ORA_NVFP4)
        tsv = gamax / 2688.0f;          /* 6 * 448 */
    else
        tsv = gamax / 3136.0f;          /* 7 * 448: the INT4 maximum */
    return tsv;
}

/*
 * Quantize x [rows, cols] (fp32, row-major, blocks run along cols).
 *   fmt     ORA_MXFP4 (block 32, E8M0) or ORA_NVFP4 (block 16, E4M3 x fp32),
 *           or their INT4-element twins ORA_MXINT4 / ORA_NVINT4 ([MRGPTQ]:
 *           identical except for the element; the NVINT4 tensor scale is
 *           amax / (7 * 448) and its block scale maps the block maximum onto 7;
 *           only the absmax rule).
 *   rotate  0, or 1 for a block Hadamard of the block size applied first.
 *   rule    ORA_SCALE_ABSMAX: the block maximum sets the scale.
 *           ORA_SCALE_MSE: among candidate scale codes around the absmax code
 *             c0, the one whose block has the smallest squared error
 *             (block_sse).  MXFP4 candidates: c0, c0 + 1.  NVFP4: c0, c0 + 1,
 *             c0 - 1, c0 + 2, c0 - 2, c0 + 3, c0 + 4, c0 + 5, c0 + 6 (codes
 *             outside 0 .. 0x7E skipped).  A later candidate replaces the best
 *             one only with a strictly smaller error, so ties keep the
 *             earliest (the absmax code first).
 *           ORA_SCALE_FOUR_OVER_SIX (NVFP4 only): candidates c0 (maximum onto
 *             6), then the code that maps the maximum onto 4; the smaller
 *             error wins, ties keep c0.
 *   codes   out, [rows, cols/2] bytes, element 2i in the low nibble.
 *   scales  out, [rows, cols/G] bytes, row-major.
 *   ts      NVFP4 per-tensor scale: written (gs_given = 0) or read (= 1).
 *           Every rule uses the same tensor scale, amax / (6 * 448).
 * MXFP4 follows [VS] "A worked example, by hand" and the emulation's mxfp4;
 * NVFP4 follows [VS] Figure 2 (global amax -> fp32 tensor scale -> block amax
 * -> E4M3 -> E2M1 -> pack) and the emulation's nvfp4.
 */
/* Quantization specification of the oracle (its own struct).
 *   rot_n       0, or the Hadamard size: the block size (16 or 32); MX
 *               formats also 64 or 128 ([MRGPTQ]: larger rotations help
 *               MXFP4).  A rotation group of rot_n elements along the row.
 *   signs       the sign diagonal applied before the Hadamard (bit i: element
 *               i of the group negated); all zero = the plain transform.
 *   rule        ORA_SCALE_* (searching rules: FP4 elements, block_rows 1).
 *   rounding    0: nearest, ties to even; 1: stochastic (E2M1 elements,
 *               absmax rule), uniform numbers from sr_uniform(seed).
 *   block_rows  1, or 16 for NVFP4: the scale of a 16x16 tile (16 rows x one
 *               16-column block) is taken from the tile's maximum and stored
 *               for each of its rows ([VS] "Two-dimensional weight scaling":
 *               a tile and its transpose share one scale). */
typedef struct {
    int fmt;
    int rot_n;
    uint32_t signs[4];
    int rule;
    int rounding;
    uint32_t seed[2];
    int block_rows;
} ora_qspec;

int ora_quantize_spec(const ora_qspec *q, const float *x, long rows, long cols,
                      uint8_t *codes, uint8_t *scales, float *ts, int gs_given)
{
    int fmt = q->fmt, rule = q->rule;
    int G = fmt_block(fmt);
    if (G == 0)
        return ORA_EINVAL;
    if (rows < 0 || cols < 0 || cols % G != 0)
        return ORA_EINVAL;
    if (!fmt_mx(fmt) && ts == NULL)
        return ORA_EINVAL;
    if (rule != ORA_SCALE_ABSMAX && (fmt_int(fmt) || (rule != ORA_SCALE_MSE &&
        !(rule == ORA_SCALE_FOUR_OVER_SIX && fmt == ORA_NVFP4))))
        return ORA_EINVAL;
    int rn = q->rot_n;
    if (rn != 0 && rn != G && !(fmt_mx(fmt) && (rn == 64 || rn == 128)))
        return ORA_EINVAL;
    if (rn != 0 && cols % rn != 0)
        return ORA_EINVAL;
    if (q->rounding != 0 && (q->rounding != 1 || fmt_int(fmt) || rule != ORA_SCALE_ABSMAX))
        return ORA_EINVAL;
    if (q->block_rows != 1 && (q->block_rows != 16 || fmt != ORA_NVFP4 || rn != 0 ||
                               rule != ORA_SCALE_ABSMAX))
        return ORA_EINVAL;

    long n = rows * cols;
    const float *y = x;
    float *ybuf = NULL;
    if (rn) {
        ybuf = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        if (!ybuf)
            return ORA_EINVAL;
        ora_rotate_signed(x, ybuf, rows, cols, rn, q->signs, 0);
        y = ybuf;
    }

    float tsv = 0.0f;
    if (!fmt_mx(fmt)) {
        if (gs_given) {
            tsv = *ts;
        } else {
            tsv = tensor_scale(fmt, y, n);
            *ts = tsv;
        }
    }

    static const int nv_window[9] = {0, 1, -1, 2, -2, 3, 4, 5, 6};
    long nb = cols / G;
    int code[32], cand_code[32];
    for (long r = 0; r < rows; ++r) {
        uint8_t *rc = codes + r * (cols / 2);
        for (long b = 0; b < nb; ++b) {
            const float *yb = y + r * cols + b * G;
            float amax = block_amax(yb, G);
            if (q->block_rows > 1) {           /* the 16x16 tile's maximum */
                long r0 = r - r % q->block_rows;
                for (long rr = r0; rr < r0 + q->block_rows && rr < rows; ++rr) {
                    float m = block_amax(y + rr * cols + b * G, G);
                    if (m > amax)
                        amax = m;
                }
            }
            int sc;
            if (fmt_mx(fmt)) {
                /* floor(log2 amax) - 2 for both elements: 4 = 2^2 is the
                 * largest power of two of E2M1 (max 6) and of INT4 (max 7) */
                sc = mx_exponent(amax) + 127;
            } else {
                sc = 0;
                if (tsv > 0.0f) {
                    if (fmt == ORA_NVFP4) {
                        float t = (amax / 6.0f) / tsv;
                        sc = ora_e4m3_encode(t);
                    } else {
                        float t = (amax / 7.0f) / tsv;
                        sc = ora_e4m3_encode(t);
                    }
                }
            }
            block_encode(fmt, yb, G, sc, tsv, code);
            if (q->rounding == 1) {
                float s = fmt_mx(fmt) ? ldexpf(1.0f, sc - 127) : (float)ora_e4m3_decode(sc) * tsv;
                for (int i = 0; i < G; ++i) {
                    double u = sr_uniform((uint64_t)r * (uint64_t)cols + (uint64_t)(b * G + i), q->seed);
                    code[i] = s != 0.0f ? ora_e2m1_encode_sr(yb[i] / s, u) : 0;
                }
            }
            if (rule != ORA_SCALE_ABSMAX && !(!fmt_mx(fmt) && !(tsv > 0.0f))) {
                int cands[9], nc = 0;
                if (rule == ORA_SCALE_MSE && fmt == ORA_MXFP4) {
                    cands[nc++] = sc + 1;
                } else if (rule == ORA_SCALE_MSE) {
                    for (int w = 1; w < 9; ++w)
                        cands[nc++] = sc + nv_window[w];
                } else {
                    cands[nc++] = nv_scale_code(amax, 4.0f, tsv);
                }
                int maxcode = fmt_mx(fmt) ? 254 : 0x7E;
                float best = block_sse(fmt, yb, G, sc, tsv, code);
                for (int k = 0; k < nc; ++k) {
                    int c = cands[k];
                    if (c < 0 || c > maxcode)
                        continue;
                    block_encode(fmt, yb, G, c, tsv, cand_code);
                    float e = block_sse(fmt, yb, G, c, tsv, cand_code);
                    if (e < best) {
                        best = e;
                        sc = c;
                        memcpy(code, cand_code, sizeof(int) * (size_t)G);
                    }
                }
            }
            scales[r * nb + b] = (uint8_t)sc;
            for (int i = 0; i < G; ++i)
                put_code(rc, b * G + i, code[i]);
        }
    }
    free(ybuf);
    return ORA_OK;
}

/* The NV per-tensor scale alone, exactly as ora_quantize_spec computes it
 * without a given scale: x rotated by rot_n (0 or the block size) with the
 * sign mask `signs` (may be NULL), then tensor_scale.  Returns ORA_EINVAL
 * for MX formats or bad sizes. */
int ora_tensor_scale(int fmt, int rot_n, const uint32_t *signs, const float *x, long rows,
                     long cols, float *ts)
{
    int G = fmt_block(fmt);
    if (G == 0 || fmt_mx(fmt) || ts == NULL || rows < 0 || cols < 0 || cols % G != 0)
        return ORA_EINVAL;
    if (rot_n != 0 && rot_n != G)
        return ORA_EINVAL;
    long n = rows * cols;
    if (!rot_n) {
        *ts = tensor_scale(fmt, x, n);
        return ORA_OK;
    }
    float *y = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!y)
        return ORA_EINVAL;
    ora_rotate_signed(x, y, rows, cols, rot_n, signs, 0);
    *ts = tensor_scale(fmt, y, n);
    free(y);
    return ORA_OK;
}

/* A block-size rotation (or none), nearest rounding, one-row blocks. */
int ora_quantize_rule(int fmt, int rotate, int rule, const float *x, long rows, long cols,
                      uint8_t *codes, uint8_t *scales, float *ts, int gs_given)
{
    if (rotate != 0 && rotate != 1)
        return ORA_EINVAL;
    ora_qspec q;
    memset(&q, 0, sizeof q);
    q.fmt = fmt;
    q.rot_n = rotate ? fmt_block(fmt) : 0;
    q.rule = rule;
    q.block_rows = 1;
    return ora_quantize_spec(&q, x, rows, cols, codes, scales, ts, gs_given);
}

/* The absmax rule ([VS] "A worked example, by hand"; Figure 2). */
int ora_quantize(int fmt, int rotate, const float *x, long rows, long cols,
                 uint8_t *codes, uint8_t *scales, float *ts, int gs_given)
{
    return ora_quantize_rule(fmt, rotate, ORA_SCALE_ABSMAX, x, rows, cols, codes, scales, ts,
                             gs_given);
}

/*
 * Dequantize codes/scales back to fp32 y [rows, cols] ([VS] Figure 1: element
 * times scale, NVFP4 applying the per-tensor factor on top; [PROD] "Format
 * Specifications").  MXFP4: y = e2m1 * 2^(c-127).  NVFP4: y = fl32(fl32(e2m1 *
 * e4m3) * ts) -- the inner product is exact in fp32.  inverse_rotate = 1 then
 * applies the (self-inverse) normalised block Hadamard of the block size.
 */
int ora_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, float ts,
                   long rows, long cols, int inverse_rotate, float *y)
{
    return ora_dequantize_rot(fmt, codes, scales, ts, rows, cols,
                              inverse_rotate ? fmt_block(fmt) : 0, NULL, y);
}

/* As ora_dequantize, with the inverse of a rotation of size rot_n (0: none)
 * and sign mask signs (see ora_rotate_signed). */
int ora_dequantize_rot(int fmt, const uint8_t *codes, const uint8_t *scales, float ts,
                       long rows, long cols, int rot_n, const uint32_t *signs, float *y)
{
    int inverse_rotate = rot_n != 0;
    int G = fmt_block(fmt);
    if (G == 0)
        return ORA_EINVAL;
    if (rows < 0 || cols < 0 || cols % G != 0)
        return ORA_EINVAL;
    long nb = cols / G;
    float *tmp = NULL;
    float *dst = y;
    if (inverse_rotate) {
        tmp = (float *)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
        if (!tmp)
            return ORA_EINVAL;
        dst = tmp;
    }
    for (long r = 0; r < rows; ++r) {
        const uint8_t *rc = codes + r * (cols / 2);
        for (long k = 0; k < cols; ++k) {
            double m = elem_decode(fmt, get_code(rc, k));
            int sc = scales[r * nb + k / G];
            if (fmt_mx(fmt)) {
                dst[r * cols + k] = (float)(m * ora_e8m0_decode(sc));
            } else {
                float inner = (float)(m * ora_e4m3_decode(sc));
                dst[r * cols + k] = inner * ts;
            }
        }
    }
    if (inverse_rotate) {
        int rc = ora_rotate_signed(tmp, y, rows, cols, rot_n, signs, 1);
        free(tmp);
        return rc;
    }
    return ORA_OK;
}

/*
 * Error sums over n values in double ([PORT] section 3.2: NMSE = ||x - x^||^2
 * / ||x||^2 and cosine similarity; [VS] emulation: MSE and SQNR = 10 log10(
 * mean x^2 / MSE)).  out[0] = sum (x - x^)^2, out[1] = sum x^2,
 * out[2] = sum x * x^, out[3] = sum x^^2.
 */
void ora_error_sums(const float *x, const float *xhat, long n, double *out)
{
    double se = 0.0, sx = 0.0, sxy = 0.0, sy = 0.0;
    for (long i = 0; i < n; ++i) {
        double a = x[i], b = xhat[i];
        se += (a - b) * (a - b);
        sx += a * a;
        sxy += a * b;
        sy += b * b;
    }
    out[0] = se;
    out[1] = sx;
    out[2] = sxy;
    out[3] = sy;
}

/*
 * Selected entries of Y = A * B^T ([MRGPTQ]: the kernels compute
 * Q(W H_k) Q(X H_k)^T; [VS] "Hardware execution": scales applied inside the
 * product, accumulation at higher precision).  A is [M, K] and B is [N, K],
 * both as packed codes (row-major, K/2 bytes per row) with row-major scales
 * (K/G per row).  For each requested (row, col):
 *   y    = sum_k a^[row][k] * b^[col][k]  in double;
 *   absy = sum_k |a^[row][k]| * |b^[col][k]|.
 * MXFP4: a^ = e2m1 * 2^(c-127).  NVFP4: the sum runs over (e2m1 * e4m3)
 * products and is multiplied by a_ts * b_ts at the end.
 */
int ora_gemm_entries(int fmt, long K,
                     const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                     const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                     long nent, const long *rows, const long *cols,
                     double *y, double *absy)
{
    int G = fmt_block(fmt);
    if (G == 0)
        return ORA_EINVAL;
    if (K < 0 || K % G != 0)
        return ORA_EINVAL;
    long nb = K / G;
    for (long e = 0; e < nent; ++e) {
        const uint8_t *ac = a_codes + rows[e] * (K / 2);
        const uint8_t *bc = b_codes + cols[e] * (K / 2);
        const uint8_t *as = a_scales + rows[e] * nb;
        const uint8_t *bs = b_scales + cols[e] * nb;
        double s = 0.0, sa = 0.0;
        for (long b = 0; b < nb; ++b) {
            double asv, bsv;            /* the two block scales */
            if (fmt_mx(fmt)) {
                asv = ora_e8m0_decode(as[b]);
                bsv = ora_e8m0_decode(bs[b]);
            } else {
                asv = ora_e4m3_decode(as[b]);
                bsv = ora_e4m3_decode(bs[b]);
            }
            for (long k = b * G; k < (b + 1) * G; ++k) {
                double av = elem_decode(fmt, get_code(ac, k)) * asv;
                double bv = elem_decode(fmt, get_code(bc, k)) * bsv;
                s += av * bv;
                sa += fabs(av) * fabs(bv);
            }
        }
        if (!fmt_mx(fmt)) {
            double g = (double)a_ts * (double)b_ts;
            s *= g;
            sa *= fabs(g);
        }
        y[e] = s;
        absy[e] = sa;
    }
    return ORA_OK;
}

/*
 * Weight-only GEMM entries ("Bridging the Gap Between Promise and Performance
 * for Microscaling FP4 Quantization", W4A16: 16-bit activations times FP4
 * weights).  The plain definition:
 *   y    = sum_k a[row][k] * b^[col][k]  in double;
 *   absy = sum_k |a[row][k]| * |b^[col][k]|,
 * with a[M, K] given as fp32 values (the bf16 activations, exactly) and
 * b^ the dequantized weights (MXFP4: e2m1 * 2^(c-127); NVFP4: e2m1 * e4m3,
 * the sum multiplied by b_ts at the end).  b_scales row-major [N, K/G].
 */
int ora_gemm_w4a16_entries(int fmt, long K, const float *a, long lda,
                           const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                           long nent, const long *rows, const long *cols,
                           double *y, double *absy)
{
    int G = fmt_block(fmt);
    if (G == 0)
        return ORA_EINVAL;
    if (K < 0 || K % G != 0 || lda < K)
        return ORA_EINVAL;
    long nb = K / G;
    for (long e = 0; e < nent; ++e) {
        const float *ar = a + rows[e] * lda;
        const uint8_t *bc = b_codes + cols[e] * (K / 2);
        const uint8_t *bs = b_scales + cols[e] * nb;
        double s = 0.0, sa = 0.0;
        for (long b = 0; b < nb; ++b) {
            double bsv = fmt_mx(fmt) ? ora_e8m0_decode(bs[b]) : ora_e4m3_decode(bs[b]);
            for (long k = b * G; k < (b + 1) * G; ++k) {
                double bv = elem_decode(fmt, get_code(bc, k)) * bsv;
                s += (double)ar[k] * bv;
                sa += fabs((double)ar[k]) * fabs(bv);
            }
        }
        if (!fmt_mx(fmt)) {
            s *= (double)b_ts;
            sa *= fabs((double)b_ts);
        }
        y[e] = s;
        absy[e] = sa;
    }
    return ORA_OK;
}

/* Array forms of the codecs, for exhaustive checks. */
void ora_e2m1_encode_array(const float *q, long n, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = (uint8_t)ora_e2m1_encode(q[i]);
}

void ora_int4_encode_array(const float *q, long n, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = (uint8_t)ora_int4_encode(q[i]);
}

void ora_e4m3_encode_array(const float *t, long n, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = (uint8_t)ora_e4m3_encode(t[i]);
}

/* ------------------------------------------------------------------------ */
/* Tiled code layout.  No page fixes a storage order for packed codes; this is
 * the library's own FP4_CODES_TILED layout, written here from its definition:
 * the code bytes of a [rows, row_bytes] row-major matrix (rows a multiple of
 * 128, row_bytes of 64) go into 8192-byte tiles of 128 rows x 64 bytes,
 * row-major inside a tile; the tiles of one 128-row panel follow each other
 * along the row, and the panels follow each other.  A pure permutation. */
int ora_tile_codes(const uint8_t *src, long rows, long row_bytes, uint8_t *dst)
{
    if (rows < 0 || row_bytes < 0 || rows % 128 != 0 || row_bytes % 64 != 0)
        return ORA_EINVAL;
    const long tiles_per_panel = row_bytes / 64;
    for (long r = 0; r < rows; ++r) {
        for (long b = 0; b < row_bytes; ++b) {
            long panel = r / 128, tile = b / 64;
            long start = (panel * tiles_per_panel + tile) * 8192;
            dst[start + (r % 128) * 64 + (b % 64)] = src[r * row_bytes + b];
        }
    }
    return ORA_OK;
}
