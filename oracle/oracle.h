/*
 * oracle.h -- plain scalar CPU reference for the fine-grained FP8 linear.
 *
 * TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and
 * the CPU-baseline leg of bench.py may load, call or link this library. The
 * product library (block_scaled_gemm_amd/) never does, and the two share no
 * source, header, table or constant.
 *
 * Pages are cited by host and post id:
 *   [qna-131281]          xn--9g3bo1gtkw0l8ubf92bgle.kr, qna post 131281
 *   [hacks-368261]        "9 Amazing Deepseek Hacks", xn--jj0bz6z98ct0a29q.com post 368261
 *   [cameseeing-1171527]  blog.cameseeing.com, freeboard post 1171527
 *   [why-be-59061]        why-be.why-be.co.kr, as_center post 59061
 *   [why-be-50529]        why-be.why-be.co.kr, as_center post 50529
 * followed by the passage (figure, heading or topic) the statement comes from.
 *
 * Every function states the reading it takes where the pages are silent.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes (0 = ok). */
#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_SHAPE 2

/* ---- E4M3 (OCP "FN" variant: bias 7, no infinities, max 448) ---------- */

/* Nearest E4M3 code to a finite float, ties to the even code, |v| >= 448
 * saturating to +-448.  The sign of v is kept, so negative values that round
 * to zero give 0x80. */
uint8_t orc_e4m3_encode(float v);

/* Exact value of an E4M3 code (NaN for 0x7F / 0xFF). */
double orc_e4m3_decode(uint8_t code);

/* Array form of orc_e4m3_encode. */
void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out);

/* ---- scale of one group --------------------------------------------------
 * amax is the group's max |x|; pow2 = 0 gives the FP32 scale, 1 the
 * power-of-two scale.  s is the dequantisation scale that is stored, inv the
 * factor the elements are multiplied by before rounding. */
void orc_group_scale(float amax, int pow2, float *s, float *inv);

/* The amax floor that keeps s normal and inv finite: 448 * 2^-126. */
float orc_amax_floor(void);

/* ---- quantisers ----------------------------------------------------------
 * x is bf16 stored as uint16, row-major with leading dimension ldx.
 * axis 0 (row): groups are 1x128 runs along the contiguous dimension;
 *   q is [rows][ldq]; the scale of group g of row r is s[g*lds + r].
 * axis 1 (col): groups are 128x1 runs down a column; q is written
 *   transposed, [cols][ldq], so that the 128 codes of a group are contiguous;
 *   the scale of group g of column c is s[g*lds + c].
 * Returns ORC_ERR_SHAPE when the grouped dimension is not a multiple of 128. */
int orc_quant_tile(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                   int axis, int pow2, uint8_t *q, int64_t ldq, float *s,
                   int64_t lds);

/* 128x128 blocks of w [rows][ldw]; cols must be a multiple of 128, a last
 * partial block-row holds the rows present.  q is [rows][ldq]; qt, when not
 * NULL, is the transposed copy [cols][ldqt]; the scale of block (i, j) is
 * s[i*lds + j]. */
int orc_quant_block(const uint16_t *w, int64_t rows, int64_t cols, int64_t ldw,
                    int pow2, uint8_t *q, int64_t ldq, uint8_t *qt,
                    int64_t ldqt, float *s, int64_t lds);

/* 128x1 groups along the tokens of each expert.  x [T][ldx] holds the
 * tokens of G experts back to back: expert e owns rows offsets[e] ..
 * offsets[e+1]-1.  Each expert's tokens are cut into groups of 128 starting
 * at its first token; the last group holds the n_e mod 128 remaining tokens
 * (its amax is taken over those only).  Codes are written transposed into a
 * padded token axis where expert e starts at P_e = 128 * sum_{e'<e}
 * ceil(n_e'/128): q[c*ldq + P_e + i] for token offsets[e] + i, zero codes in
 * the padding; the scale of padded group p of column c is s[p*lds + c]
 * (padded groups of the padding tail of an expert do not exist: every
 * padded group holds at least one token).  Returns the padded length in *tp. */
int orc_quant_tile_grouped_col(const uint16_t *x, int64_t T, int64_t C,
                               int64_t ldx, int G, const int32_t *offsets,
                               int pow2, uint8_t *q, int64_t ldq, float *s,
                               int64_t lds, int64_t *tp);

/* ---- backward re-tiling ----------------------------------------------------
 * q [rows][ldq] holds codes quantised in 1x128 row groups with scales
 * s[g*lds + r] (the layout orc_quant_tile writes for axis 0).  The matrix is
 * dequantised (x = fl32(dec(q) * s)), transposed and quantised again in
 * 128x1 groups down its columns: qt [cols][ldqt], scale of group g of column
 * c in st[g*ldst + c] (the layout of axis 1).  rows and cols must be
 * multiples of 128; the dequantised values must be finite in fp32. */
int orc_requant_col(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                    const float *s, int64_t lds, int pow2, uint8_t *qt,
                    int64_t ldqt, float *st, int64_t ldst);

/* ---- block-scaled GEMM ---------------------------------------------------
 * R[m][n] = sum_g sa[g*ldsa+m] * SB(n,g) * P_g[m][n], with
 *   P_g[m][n] = sum_{k in group g} dec(a[m*lda+k]) * dec(b[n*ldb+k])
 * computed exactly, and SB(n,g) = sb[(n/128)*sb_s0 + g*sb_s1] for
 * bscale_kind 0 (128x128 weight blocks) or sb[g*sb_s0 + n] for kind 1
 * (a per-column scale, as for 128x1 token tiles).  The result is fp64,
 * d[m*ldd + n].  K must be a multiple of 128. */
int orc_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a, int64_t lda,
             const float *sa, int64_t ldsa, const uint8_t *b, int64_t ldb,
             const float *sb, int bscale_kind, int64_t sb_s0, int64_t sb_s1,
             double *d, int64_t ldd);

/* The same sum for the listed (m, n) pairs only. */
int orc_gemm_entries(int64_t M, int64_t N, int64_t K, const uint8_t *a,
                     int64_t lda, const float *sa, int64_t ldsa,
                     const uint8_t *b, int64_t ldb, const float *sb,
                     int bscale_kind, int64_t sb_s0, int64_t sb_s1,
                     int64_t count, const int64_t *mi, const int64_t *ni,
                     double *out);

/* Grouped GEMM: rows offsets[e] .. offsets[e+1]-1 of a use expert e, whose
 * codes are b[e][N][K] and block scales sb[e][N/128][K/128].  d has
 * offsets[G] rows.  N and K must be multiples of 128. */
int orc_grouped_gemm(int G, int64_t N, int64_t K, const int32_t *offsets,
                     const uint8_t *a, int64_t lda, const float *sa,
                     int64_t ldsa, const uint8_t *b, const float *sb,
                     double *d, int64_t ldd);

/* Sampled form of orc_grouped_gemm: row mi[i] (a global row of a), column
 * ni[i]; the expert is found from offsets. */
int orc_grouped_gemm_entries(int G, int64_t N, int64_t K,
                             const int32_t *offsets, const uint8_t *a,
                             int64_t lda, const float *sa, int64_t ldsa,
                             const uint8_t *b, const float *sb, int64_t count,
                             const int64_t *mi, const int64_t *ni,
                             double *out);

/* A model of FP8 GEMM accumulation with limited precision, for the large-K
 * study (not the reference result): the running sum keeps `bits`
 * significant bits, `chunk` products are added exactly and the sum is then
 * cut toward zero to `bits` bits.  interval 0: one such sum over all of K
 * of the dequantised products (never promoted); interval I (dividing 128,
 * a multiple of chunk): each I-element partial of code products is such a
 * sum from zero, then scaled by its group's sa * SB and added in fp64
 * (promoted every I elements).  Arguments otherwise as orc_gemm. */
int orc_gemm_limited(int64_t M, int64_t N, int64_t K, const uint8_t *a,
                     int64_t lda, const float *sa, int64_t ldsa,
                     const uint8_t *b, int64_t ldb, const float *sb,
                     int bscale_kind, int64_t sb_s0, int64_t sb_s1, int bits,
                     int chunk, int interval, double *d, int64_t ldd);

/* Number of OpenMP threads the GEMM and quantiser loops use (1 when the
 * library was built without OpenMP). */
int orc_num_threads(void);

/* Threads the OpenMP loops of later calls use (n < 1: the default). */
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif /* FP8_ORACLE_H */
