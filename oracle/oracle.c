/*
 * oracle.c -- plain scalar CPU reference for the fine-grained FP8 linear.
 *
 * TEST INFRASTRUCTURE: see oracle.h for who may use it.  Written for a
 * reader who checks it against the pages by eye: no blocking, no fusion,
 * one group at a time.  Build: gcc -O2 -fopenmp -ffp-contract=off (no
 * fast-math, so every float operation below is one IEEE round-to-nearest
 * operation).
 *
 * What is computed, and where the pages say so:
 *  - Online fine-grained quantisation: the max absolute value of each small
 *    group gives the group's scaling factor, and the values are quantised to
 *    FP8 on the fly ([qna-131281] and [why-be-59061], passages on the
 *    fine-grained quantisation strategy; [cameseeing-1171527], passage on
 *    aligning the max absolute value with the largest FP8 value).
 *  - Power-of-two scales for some activations ([why-be-59061], passage on the
 *    activations after attention and before the MoE down-projection).
 *  - 128x1 tiles for the backward pass ([hacks-368261], passage on the
 *    dequantise / transpose / re-quantise round trip).
 *  - GEMMs take FP8 inputs and give BF16 or FP32 outputs; partial sums are
 *    promoted to FP32 every 128 elements of K ([qna-131281], passage on FP8
 *    GEMM inputs and outputs; [why-be-59061], passage on the 128-element
 *    interval and the copy to FP32 registers; [cameseeing-1171527],
 *    Figure 7(b)).
 *  - The GEMM reference itself is the FP64 dequantised dot product, reached
 *    exactly per 128-element group (a group partial is an integer multiple
 *    of 2^-18 below 2^25 in magnitude, so int64 holds it exactly).
 *
 * Readings where the pages are silent (E4M3 "FN", round-half-even, the
 * amax floor, rounding the scaled value to fp32 before encoding, rounding
 * power-of-two scales up) are stated at each function.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------
 * E4M3 codec.  Format (OCP FP8, E4M3 "FN"): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9;
 * field 15 with mantissa 7 is NaN; there is no infinity; the largest
 * finite value is 1.75 * 2^8 = 448 (code 0x7E).  The pages say only "FP8"
 * with few exponent bits ([cameseeing-1171527], passage on overflow and
 * underflow); E4M3 with saturation is the reading taken.
 * ------------------------------------------------------------------------ */

/* Round a non-negative double to the nearest integer, halves to even. */
static double round_half_even(double x)
{
    double f = floor(x);
    double frac = x - f; /* exact for the magnitudes used here */
    if (frac > 0.5)
        return f + 1.0;
    if (frac < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);

    /* Saturate: anything at or above the largest finite value becomes it. */
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);

    /* Subnormal range (below the smallest normal 2^-6): the representable
     * values are m * 2^-9, m = 0..7; m = 8 is the smallest normal, whose
     * code 0x08 is the same integer. */
    if (a < ldexp(1.0, -6)) {
        double m = round_half_even(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }

    /* Normal range: a = mant * 2^e with mant in [1, 2). */
    int e2;
    double fr = frexp(a, &e2); /* a = fr * 2^e2, fr in [0.5, 1) */
    int e = e2 - 1;
    double mant = 2.0 * fr;                         /* [1, 2)   */
    double f = round_half_even((mant - 1.0) * 8.0); /* 0 .. 8   */
    if (f == 8.0) {
        e += 1;
        f = 0.0;
    }
    /* e in [-6, 8]; at e = 8, a < 448 keeps f <= 6 (0x7F is NaN). */
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)f);
}

double orc_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = (double)m * ldexp(1.0, -9);
    else
        v = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; i++)
        out[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------------
 * Group scale.
 * FP32 mode: the group's amax is mapped onto the largest E4M3 value, so the
 * stored dequantisation scale is s = amax / 448 and the elements are
 * multiplied by inv = 448 / amax (each a single fp32 division).
 * POW2 mode: s is the smallest integral power of two with amax <= 448 * s,
 * so no element is clipped (reading: the pages say "integral power of 2"
 * without a direction; rounding up is the one that never saturates).
 * Both modes clamp amax from below at 448 * 2^-126 (reading: the pages do
 * not treat an all-zero group; the floor keeps s a normal float and inv
 * finite).
 * ------------------------------------------------------------------------ */
float orc_amax_floor(void)
{
    return (float)(448.0 * ldexp(1.0, -126)); /* 1.75 * 2^-118, exact */
}

void orc_group_scale(float amax, int pow2, float *s, float *inv)
{
    float floor_a = orc_amax_floor();
    float a = amax > floor_a ? amax : floor_a;
    if (!pow2) {
        *s = a / 448.0f;
        *inv = 448.0f / a;
        return;
    }
    /* Smallest k with a <= 448 * 2^k, found by walking k up from -126
     * (where the floor already satisfies it).  Exact in double. */
    int k = -126;
    while ((double)a > 448.0 * ldexp(1.0, k))
        k++;
    *s = (float)ldexp(1.0, k);
    *inv = (float)ldexp(1.0, -k);
}

/* bf16 (as uint16) to float: the bf16 bits are the top half of an fp32. */
static float bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Quantise one group of n elements read through (base, stride) and write
 * codes through (out, ostride).  Returns the stored scale.  The scaled value
 * is rounded to fp32 (x * inv is one fp32 multiply) before it is encoded;
 * reading: the pages do not say in which precision the scaling happens, and
 * fp32 is the precision of the scaling factor itself. */
static float quantise_group(const uint16_t *base, int64_t stride, int64_t n,
                            int pow2, uint8_t *out, int64_t ostride)
{
    float amax = 0.0f;
    int64_t i;
    for (i = 0; i < n; i++) {
        float v = fabsf(bf16_value(base[i * stride]));
        if (v > amax)
            amax = v;
    }
    float s, inv;
    orc_group_scale(amax, pow2, &s, &inv);
    for (i = 0; i < n; i++) {
        float x = bf16_value(base[i * stride]);
        float y = x * inv; /* one fp32 rounding */
        out[i * ostride] = orc_e4m3_encode(y);
    }
    return s;
}

int orc_quant_tile(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                   int axis, int pow2, uint8_t *q, int64_t ldq, float *s,
                   int64_t lds)
{
    if (!x || !q || !s || rows < 0 || cols < 0 || (axis != 0 && axis != 1))
        return ORC_ERR_ARG;
    if (axis == 0) {
        /* 1x128 groups along each row. */
        if (cols % 128 != 0)
            return ORC_ERR_SHAPE;
        if (ldx < cols || ldq < cols || lds < rows)
            return ORC_ERR_ARG;
        int64_t r;
#pragma omp parallel for schedule(static)
        for (r = 0; r < rows; r++) {
            for (int64_t g = 0; g < cols / 128; g++) {
                s[g * lds + r] = quantise_group(x + r * ldx + g * 128, 1, 128,
                                                pow2, q + r * ldq + g * 128, 1);
            }
        }
    } else {
        /* 128x1 groups down each column; codes written transposed. */
        if (rows % 128 != 0)
            return ORC_ERR_SHAPE;
        if (ldx < cols || ldq < rows || lds < cols)
            return ORC_ERR_ARG;
        int64_t c;
#pragma omp parallel for schedule(static)
        for (c = 0; c < cols; c++) {
            for (int64_t g = 0; g < rows / 128; g++) {
                s[g * lds + c] =
                    quantise_group(x + (g * 128) * ldx + c, ldx, 128, pow2,
                                   q + c * ldq + g * 128, 1);
            }
        }
    }
    return ORC_OK;
}

/* 128x1 groups restarted at every expert boundary (reading: the pages give
 * the 128x1 tiles of the backward pass for one matrix; for tokens routed to
 * experts a group must not mix two experts' tokens, so each expert's tokens
 * are grouped from its first token and its last group may be partial).
 * Transposed output on a padded token axis so that every expert starts on
 * a 128-element boundary. */
int orc_quant_tile_grouped_col(const uint16_t *x, int64_t T, int64_t C,
                               int64_t ldx, int G, const int32_t *offsets,
                               int pow2, uint8_t *q, int64_t ldq, float *s,
                               int64_t lds, int64_t *tp)
{
    if (!x || !offsets || !q || !s || !tp || T < 0 || C < 0 || G < 0 ||
        ldx < C || lds < C)
        return ORC_ERR_ARG;
    if (offsets[0] != 0 || offsets[G] > T)
        return ORC_ERR_ARG;
    int64_t pad = 0;
    for (int e = 0; e < G; e++) {
        int64_t n = (int64_t)offsets[e + 1] - offsets[e];
        if (n < 0)
            return ORC_ERR_ARG;
        pad += (n + 127) / 128 * 128;
    }
    *tp = pad;
    if (ldq < pad)
        return ORC_ERR_ARG;
    int64_t start = 0; /* padded position of the current expert */
    for (int e = 0; e < G; e++) {
        int64_t r0 = offsets[e], n = (int64_t)offsets[e + 1] - offsets[e];
        int64_t ng = (n + 127) / 128;
        int64_t c;
#pragma omp parallel for schedule(static)
        for (c = 0; c < C; c++) {
            for (int64_t j = 0; j < ng; j++) {
                int64_t len = n - j * 128 < 128 ? n - j * 128 : 128;
                uint8_t *out = q + c * ldq + start + j * 128;
                s[(start / 128 + j) * lds + c] =
                    quantise_group(x + (r0 + j * 128) * ldx + c, ldx, len, pow2, out, 1);
                for (int64_t i = len; i < 128; i++)
                    out[i] = 0; /* padding */
            }
        }
        start += ng * 128;
    }
    return ORC_OK;
}

int orc_quant_block(const uint16_t *w, int64_t rows, int64_t cols, int64_t ldw,
                    int pow2, uint8_t *q, int64_t ldq, uint8_t *qt,
                    int64_t ldqt, float *s, int64_t lds)
{
    if (!w || !q || !s || rows < 0 || cols < 0)
        return ORC_ERR_ARG;
    if (cols % 128 != 0)
        return ORC_ERR_SHAPE;
    int64_t nbr = (rows + 127) / 128, nbc = cols / 128;
    if (ldw < cols || ldq < cols || lds < nbc || (qt && ldqt < rows))
        return ORC_ERR_ARG;
    int64_t bi;
#pragma omp parallel for schedule(static)
    for (bi = 0; bi < nbr; bi++) {
        int64_t r0 = bi * 128;
        int64_t nr = rows - r0 < 128 ? rows - r0 : 128;
        for (int64_t bj = 0; bj < nbc; bj++) {
            int64_t c0 = bj * 128;
            /* amax over the whole block */
            float amax = 0.0f;
            for (int64_t r = 0; r < nr; r++)
                for (int64_t c = 0; c < 128; c++) {
                    float v = fabsf(bf16_value(w[(r0 + r) * ldw + c0 + c]));
                    if (v > amax)
                        amax = v;
                }
            float sc, inv;
            orc_group_scale(amax, pow2, &sc, &inv);
            s[bi * lds + bj] = sc;
            for (int64_t r = 0; r < nr; r++)
                for (int64_t c = 0; c < 128; c++) {
                    float xv = bf16_value(w[(r0 + r) * ldw + c0 + c]);
                    float y = xv * inv;
                    uint8_t code = orc_e4m3_encode(y);
                    q[(r0 + r) * ldq + c0 + c] = code;
                    if (qt)
                        qt[(c0 + c) * ldqt + r0 + r] = code;
                }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Backward re-tiling ([hacks-368261], the hardware-suggestions passage on
 * the backward pass): a matrix held as FP8 codes in 1x128 row groups is read
 * back, dequantised, transposed and quantised again in 128x1 groups.
 * Readings (the pages give the four steps only): the dequantised element is
 * the fp32 product fl32(dec(q) * s), fp32 being the precision of the stored
 * scale; the new groups take their amax over those fp32 values and follow
 * the same scale rule, amax floor and rounding as the quantisers above.
 * ------------------------------------------------------------------------ */
int orc_requant_col(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                    const float *s, int64_t lds, int pow2, uint8_t *qt,
                    int64_t ldqt, float *st, int64_t ldst)
{
    if (!q || !s || !qt || !st || rows < 0 || cols < 0)
        return ORC_ERR_ARG;
    if (rows % 128 != 0 || cols % 128 != 0)
        return ORC_ERR_SHAPE;
    if (ldq < cols || lds < rows || ldqt < rows || ldst < cols)
        return ORC_ERR_ARG;
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < cols; c++) {
        float x[128];
        for (int64_t g = 0; g < rows / 128; g++) {
            /* read back and dequantise the column's 128 elements of group g */
            float amax = 0.0f;
            for (int64_t i = 0; i < 128; i++) {
                int64_t r = g * 128 + i;
                float d = (float)orc_e4m3_decode(q[r * ldq + c]); /* exact */
                x[i] = d * s[(c / 128) * lds + r];                /* fp32 */
                if (fabsf(x[i]) > amax)
                    amax = fabsf(x[i]);
            }
            /* quantise again as a 128x1 group, written transposed */
            float sc, inv;
            orc_group_scale(amax, pow2, &sc, &inv);
            st[g * ldst + c] = sc;
            for (int64_t i = 0; i < 128; i++)
                qt[c * ldqt + g * 128 + i] = orc_e4m3_encode(x[i] * inv);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * GEMM reference.  Every finite E4M3 value is an integer multiple of 2^-9
 * with magnitude at most 448 = 229376 * 2^-9, so dec(a) * dec(b) is an
 * integer multiple of 2^-18 below 2^36 in units, and a 128-term group sum is
 * below 2^43 units: int64 holds each group partial exactly.  The partial is
 * then scaled by sa * SB (an exact fp64 product of two floats) and the
 * groups are summed in fp64.
 * ------------------------------------------------------------------------ */

/* Code -> value in units of 2^-9 (exact integer); NaN codes give 0 and are
 * rejected by callers never producing them (quantisers never emit 0x7F). */
static int32_t dec_units[256];
static int dec_units_ready = 0;

static void init_dec_units(void)
{
    if (dec_units_ready)
        return;
    for (int c = 0; c < 256; c++) {
        double v = orc_e4m3_decode((uint8_t)c);
        dec_units[c] = isnan(v) ? 0 : (int32_t)(v * 512.0);
    }
    dec_units_ready = 1;
}

static double sb_at(const float *sb, int kind, int64_t s0, int64_t s1,
                    int64_t n, int64_t g)
{
    if (kind == 0)
        return (double)sb[(n / 128) * s0 + g * s1];
    return (double)sb[g * s0 + n];
}

/* One output element. */
static double gemm_one(int64_t K, const uint8_t *arow, const float *sa,
                       int64_t ldsa, int64_t m, const uint8_t *brow,
                       const float *sb, int kind, int64_t s0, int64_t s1,
                       int64_t n)
{
    double acc = 0.0;
    for (int64_t g = 0; g < K / 128; g++) {
        int64_t p = 0; /* group partial in units of 2^-18 */
        for (int64_t k = g * 128; k < g * 128 + 128; k++)
            p += (int64_t)dec_units[arow[k]] * (int64_t)dec_units[brow[k]];
        double scale = (double)sa[g * ldsa + m] * sb_at(sb, kind, s0, s1, n, g);
        acc += ldexp((double)p, -18) * scale;
    }
    return acc;
}

int orc_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a, int64_t lda,
             const float *sa, int64_t ldsa, const uint8_t *b, int64_t ldb,
             const float *sb, int bscale_kind, int64_t sb_s0, int64_t sb_s1,
             double *d, int64_t ldd)
{
    if (!a || !sa || !b || !sb || !d || M < 0 || N < 0 || K < 0 ||
        (bscale_kind != 0 && bscale_kind != 1))
        return ORC_ERR_ARG;
    if (K % 128 != 0)
        return ORC_ERR_SHAPE;
    init_dec_units();
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            d[m * ldd + n] = gemm_one(K, a + m * lda, sa, ldsa, m, b + n * ldb,
                                      sb, bscale_kind, sb_s0, sb_s1, n);
    return ORC_OK;
}

int orc_gemm_entries(int64_t M, int64_t N, int64_t K, const uint8_t *a,
                     int64_t lda, const float *sa, int64_t ldsa,
                     const uint8_t *b, int64_t ldb, const float *sb,
                     int bscale_kind, int64_t sb_s0, int64_t sb_s1,
                     int64_t count, const int64_t *mi, const int64_t *ni,
                     double *out)
{
    if (!a || !sa || !b || !sb || !out || !mi || !ni || K % 128 != 0)
        return ORC_ERR_ARG;
    init_dec_units();
    int64_t i;
    for (i = 0; i < count; i++)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N)
            return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; i++)
        out[i] = gemm_one(K, a + mi[i] * lda, sa, ldsa, mi[i],
                          b + ni[i] * ldb, sb, bscale_kind, sb_s0, sb_s1,
                          ni[i]);
    return ORC_OK;
}

/* Grouped GEMM: each expert's rows are a dense GEMM against that expert's
 * weights (reading: the pages describe expert GEMMs in FP8 but no grouped
 * kernel; grouping is only a batching of independent dense GEMMs). */
int orc_grouped_gemm(int G, int64_t N, int64_t K, const int32_t *offsets,
                     const uint8_t *a, int64_t lda, const float *sa,
                     int64_t ldsa, const uint8_t *b, const float *sb,
                     double *d, int64_t ldd)
{
    if (G < 0 || !offsets || N % 128 != 0 || K % 128 != 0)
        return G < 0 || !offsets ? ORC_ERR_ARG : ORC_ERR_SHAPE;
    for (int e = 0; e < G; e++) {
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
        if (r1 < r0)
            return ORC_ERR_ARG;
        if (r1 == r0)
            continue;
        const uint8_t *be = b + (int64_t)e * N * K;
        const float *sbe = sb + (int64_t)e * (N / 128) * (K / 128);
        /* rows r0..r1-1 of a and of sa (sa's row index is the global row) */
        int rc = orc_gemm(r1 - r0, N, K, a + r0 * lda, lda, sa + r0, ldsa, be,
                          K, sbe, 0, K / 128, 1, d + r0 * ldd, ldd);
        if (rc)
            return rc;
    }
    return ORC_OK;
}

int orc_grouped_gemm_entries(int G, int64_t N, int64_t K,
                             const int32_t *offsets, const uint8_t *a,
                             int64_t lda, const float *sa, int64_t ldsa,
                             const uint8_t *b, const float *sb, int64_t count,
                             const int64_t *mi, const int64_t *ni,
                             double *out)
{
    if (G < 0 || !offsets || !out || N % 128 != 0 || K % 128 != 0)
        return ORC_ERR_ARG;
    init_dec_units();
    for (int64_t i = 0; i < count; i++) {
        int e = -1;
        for (int j = 0; j < G; j++)
            if (mi[i] >= offsets[j] && mi[i] < offsets[j + 1]) {
                e = j;
                break;
            }
        if (e < 0 || ni[i] < 0 || ni[i] >= N)
            return ORC_ERR_ARG;
        const uint8_t *be = b + (int64_t)e * N * K;
        const float *sbe = sb + (int64_t)e * (N / 128) * (K / 128);
        out[i] = gemm_one(K, a + mi[i] * lda, sa, ldsa, mi[i], be + ni[i] * K,
                          sbe, 0, K / 128, 1, ni[i]);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Limited-precision accumulation: a model for the large-K study, not part of
 * the reference result above.  The pages report that the FP8 GEMM of their
 * tensor cores keeps only about 14 bits while it accumulates
 * ([cameseeing-1171527], passage on the accumulation precision of FP8
 * GEMM), that this reached a relative error of nearly 2% at K = 4096
 * ([qna-131281], passage on the preliminary test), and that copying the
 * partial sums to FP32 registers every 128 elements removes the problem
 * ([why-be-59061], passage on the 128-element interval).  They give no
 * model of that accumulator.  Reading taken: the running sum is held with
 * `bits` significant bits; `chunk` consecutive products are added exactly
 * (one instruction's worth), then the running sum is cut toward zero to
 * `bits` significant bits (the bits a fixed-width aligned adder shifts out
 * are dropped).
 *   interval 0: never promoted -- one limited sum over all of K of the
 *     dequantised products (dec(a) * sa) * (dec(b) * SB), each in fp64;
 *   interval I (dividing 128): promoted every I elements -- each interval's
 *     partial of code products dec(a) * dec(b) is formed in the limited sum
 *     from zero, then multiplied by sa * SB of its group and added to an fp64
 *     accumulator (fp64 standing in for the FP32 registers, whose rounding
 *     is far below the limited sum's).
 * ------------------------------------------------------------------------ */

/* v cut toward zero to `bits` significant bits (bits >= 53: unchanged). */
static double chop_bits(double v, int bits)
{
    if (v == 0.0 || bits >= 53)
        return v;
    int e;
    double fr = frexp(fabs(v), &e);   /* |v| = fr * 2^e, fr in [0.5, 1) */
    double t = floor(ldexp(fr, bits)); /* the top `bits` bits as an integer */
    double r = ldexp(t, e - bits);
    return v < 0 ? -r : r;
}

/* Add products p[0..n-1] to acc in chunks of `chunk`: each chunk is summed
 * exactly (fp64; the products here are exact and a chunk's sum of at most 128
 * of them is too), then the running sum is cut to `bits` bits. */
static double limited_sum(double acc, const double *p, int64_t n, int chunk,
                          int bits)
{
    for (int64_t i = 0; i < n; i += chunk) {
        double c = 0.0;
        for (int64_t j = i; j < i + chunk && j < n; j++)
            c += p[j];
        acc = chop_bits(acc + c, bits);
    }
    return acc;
}

int orc_gemm_limited(int64_t M, int64_t N, int64_t K, const uint8_t *a,
                     int64_t lda, const float *sa, int64_t ldsa,
                     const uint8_t *b, int64_t ldb, const float *sb,
                     int bscale_kind, int64_t sb_s0, int64_t sb_s1, int bits,
                     int chunk, int interval, double *d, int64_t ldd)
{
    if (!a || !sa || !b || !sb || !d || M < 0 || N < 0 || K < 0 ||
        (bscale_kind != 0 && bscale_kind != 1) || bits < 2 || chunk < 1 ||
        interval < 0)
        return ORC_ERR_ARG;
    if (K % 128 != 0 || (interval > 0 && (128 % interval != 0 || interval % chunk != 0)))
        return ORC_ERR_SHAPE;
    double dec[256]; /* decoded values, so the loops below stay cheap */
    for (int c = 0; c < 256; c++)
        dec[c] = orc_e4m3_decode((uint8_t)c);
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; m++) {
        double *prod = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        const uint8_t *arow = a + m * lda;
        for (int64_t n = 0; n < N; n++) {
            const uint8_t *brow = b + n * ldb;
            double out;
            if (interval == 0) {
                for (int64_t k = 0; k < K; k++) {
                    int64_t g = k / 128;
                    double x = dec[arow[k]] * (double)sa[g * ldsa + m];
                    double y = dec[brow[k]] * sb_at(sb, bscale_kind, sb_s0, sb_s1, n, g);
                    prod[k] = x * y;
                }
                out = limited_sum(0.0, prod, K, chunk, bits);
            } else {
                out = 0.0;
                for (int64_t k0 = 0; k0 < K; k0 += interval) {
                    int64_t g = k0 / 128;
                    for (int64_t k = k0; k < k0 + interval; k++)
                        prod[k - k0] = dec[arow[k]] * dec[brow[k]];
                    double part = limited_sum(0.0, prod, interval, chunk, bits);
                    out += part * ((double)sa[g * ldsa + m] * sb_at(sb, bscale_kind, sb_s0, sb_s1, n, g));
                }
            }
            d[m * ldd + n] = out;
        }
        free(prod);
    }
    return ORC_OK;
}

/* Threads for the OpenMP loops of later calls (n < 1 restores the default). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0)
        dflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : dflt);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
