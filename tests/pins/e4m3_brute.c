/*
 * e4m3_brute.c -- brute-force check of an E4M3 encoder over fp32 bit
 * patterns.  Test code only; it knows nothing of the oracle's encoder except
 * its signature, passed in as a function pointer.
 *
 * The candidate set is the E4M3 format written as integer significands:
 * subnormals m * 2^-9 (m = 0..7) and normals (8 + m) * 2^(e - 10) for
 * exponent field e = 1..15 and m = 0..7, without e = 15, m = 7 (NaN).  In
 * code order 0x00..0x7E these values increase, so the code of a candidate is
 * its index.  For |v| the expected code is the index of the nearest
 * candidate, the even index on a tie, 0x7E at or above 448; the sign bit of
 * v is copied to bit 7.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*encode_fn)(float);

static double cand[127];

static void build_candidates(void)
{
    for (int c = 0; c < 127; c++) {
        int e = c >> 3, m = c & 7;
        cand[c] = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    }
}

/* Candidate values, for the caller to compare with the oracle's table. */
void brute_candidates(double *out)
{
    build_candidates();
    memcpy(out, cand, sizeof cand);
}

static uint8_t brute_code(float v)
{
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (a >= cand[126])
        return sign | 126;
    int lo = 0, hi = 126; /* cand[lo] <= a < cand[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (cand[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dl = a - cand[lo], dh = cand[hi] - a;
    int pick;
    if (dl < dh)
        pick = lo;
    else if (dh < dl)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)pick;
}

/* Check every `stride`-th fp32 bit pattern starting at `start` (NaN and
 * infinity skipped).  Returns the number of mismatches; the first one found
 * (by any thread) is stored in *bad_bits / *got / *want. */
int64_t brute_check(encode_fn enc, uint64_t start, uint64_t stride,
                    uint32_t *bad_bits, uint8_t *got, uint8_t *want)
{
    build_candidates();
    int64_t bad = 0;
    int64_t i;
    int64_t n = (int64_t)((0x100000000ULL - start + stride - 1) / stride);
    *bad_bits = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (i = 0; i < n; i++) {
        uint32_t u = (uint32_t)(start + (uint64_t)i * stride);
        if (((u >> 23) & 0xFF) == 0xFF)
            continue;
        float v;
        memcpy(&v, &u, sizeof v);
        uint8_t w = brute_code(v), g = enc(v);
        if (w != g) {
            bad++;
#pragma omp critical
            {
                if (*bad_bits == 0) {
                    *bad_bits = u;
                    *got = g;
                    *want = w;
                }
            }
        }
    }
    return bad;
}
