/*
 * fp8bs.h -- C ABI of libfp8bs.so: fine-grained FP8 quantisation and the
 * block-scaled FP8 GEMM on AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by host and post id, then the passage):
 *  - Activations and weights are quantised online: each small group's
 *    maximum absolute value gives its scaling factor, and the group is then
 *    cast to FP8 ([qna-131281], passage on deriving the scaling factor and
 *    quantising online; [why-be-59061], passage on adapting the scale to
 *    smaller groups to absorb outliers).  The maximum absolute value is
 *    mapped onto the largest FP8 value ([cameseeing-1171527], passage on
 *    aligning the input distribution with the FP8 range).
 *  - Some activations use scales that are integral powers of two
 *    ([why-be-59061], passage on the input of the Linear after attention and
 *    the gradient before the MoE down-projection).
 *  - The backward pass needs activations re-tiled as 128x1 groups along the
 *    token dimension ([hacks-368261], passage on reading, dequantising,
 *    transposing and re-quantising activations into 128x1 tiles).
 *  - All three GEMMs of a Linear -- Fprop, Dgrad, Wgrad -- run in FP8
 *    ([why-be-59061], Figure 6 passage), taking FP8 inputs and producing
 *    BF16 or FP32 ([qna-131281], passage on the FP8 Wgrad GEMM).
 *  - Partial sums are promoted to FP32 every 128 elements of K, where the
 *    per-group dequantisation is applied ([why-be-59061], passage on the
 *    128-element interval and the copy of partial results to FP32
 *    registers; [cameseeing-1171527], Figure 7(b) passage).
 *  - In decoding, experts see few tokens each and the GEMM is bound by
 *    memory ([why-be-59061], passage on the decoding stage).
 *
 * Page keys: [qna-131281] xn--9g3bo1gtkw0l8ubf92bgle.kr qna post 131281;
 * [hacks-368261] "9 Amazing Deepseek Hacks", xn--jj0bz6z98ct0a29q.com post
 * 368261; [cameseeing-1171527] blog.cameseeing.com freeboard post 1171527;
 * [why-be-59061] and [why-be-50529] why-be.why-be.co.kr as_center posts.
 *
 * Conventions for every call:
 *  - bf16 tensors are passed as their 16-bit patterns (uint16_t); FP8 codes
 *    are OCP E4M3 ("FN": bias 7, max 448, 0x7F/0xFF NaN, never produced);
 *    scales are fp32 dequantisation factors: value ~= decode(code) * scale.
 *  - Every pointer argument except `stream` is DEVICE memory allocated and
 *    owned by the caller.  The library never allocates, frees or
 *    synchronises; each call validates its arguments on the host, enqueues
 *    its kernels on `stream` (a hipStream_t, NULL = the null stream) and
 *    returns.  Device faults surface at the caller's next synchronisation.
 *  - Inputs are read only; outputs are completely overwritten; inputs and
 *    outputs must not overlap.
 *  - On any error the call returns a nonzero status and enqueues nothing.
 *  - Calls are reentrant; calls on different streams may run concurrently.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_ABI_VERSION 5

/* Largest lda / ldb (bytes) the GEMMs take: the kernels address the rows of
 * a 256-row tile with 32-bit offsets (255 * 2^24 + 127 < 2^32). */
#define FP8BS_MAX_LD (1LL << 24)

/* Status codes. */
enum {
    FP8BS_OK = 0,
    FP8BS_ERR_ARG = 1,       /* null pointer, bad enum, negative size, ld too small */
    FP8BS_ERR_SHAPE = 2,     /* a grouped dimension is not a multiple of 128, or a
                                GEMM code stride is above FP8BS_MAX_LD */
    FP8BS_ERR_ALIGN = 3,     /* pointer or leading dimension misaligned */
    FP8BS_ERR_WORKSPACE = 4, /* workspace missing or too small */
    FP8BS_ERR_DEVICE = 5,    /* current device is not gfx950 / no device */
    FP8BS_ERR_HIP = 6        /* a HIP launch reported an error */
};

/* Group orientation of fp8_quant_tile. */
enum {
    FP8BS_AXIS_ROW = 0, /* 1x128 groups along the contiguous dimension */
    FP8BS_AXIS_COL = 1  /* 128x1 groups down the columns; codes transposed */
};

/* Scale mode. */
enum {
    FP8BS_SCALE_FP32 = 0, /* s = amax/448 (fp32 division), codes of x*(448/amax) */
    FP8BS_SCALE_POW2 = 1  /* s = smallest power of two with amax <= 448*s */
};

/* GEMM output type. */
enum { FP8BS_OUT_BF16 = 0, FP8BS_OUT_F32 = 1 };

/* How each 128-element group partial is formed before its FP32 promotion.
 *  FP8BS_ACCUM_FP32:  products exact and summed at FP32 accuracy.  The E4M3
 *    operands are widened exactly to f16 and multiplied on the f16 matrix
 *    cores (half the FP8 matrix-core rate).
 *  FP8BS_ACCUM_MFMA8: the FP8 matrix cores' own sum of the group (full FP8
 *    rate).  On gfx950 that sum is not FP32-accurate: it loses up to about
 *    2^-12 of the largest product in the instruction -- the same limited
 *    accumulation the pages report for their tensor cores.  Contract:
 *    |D - exact| <= 2^-10 * sum_g |sa*SB| * sum_k |dec(a)*dec(b)|, plus the
 *    output rounding.
 *  FP8BS_ACCUM_MFMA8_POW2: for power-of-two scales only (both operands
 *    quantised with FP8BS_SCALE_POW2): the scales enter the FP8 matrix cores
 *    as E8M0 block scales and each group is summed straight into the FP32
 *    accumulator, with no promotion step -- the block-scaled
 *    microscaling form of the method ([cameseeing-1171527], passage relating
 *    the fine-grained scaling to microscaling formats).  Scales that are not
 *    powers of two give wrong results without an error
 *    (fp8_scales_are_pow2 checks them); the error contract is that of
 *    FP8BS_ACCUM_MFMA8. */
enum { FP8BS_ACCUM_FP32 = 0, FP8BS_ACCUM_MFMA8 = 1, FP8BS_ACCUM_MFMA8_POW2 = 2 };

/* How the B operand's scales are addressed (SB(n, g) for column n of the
 * output and K group g). */
enum {
    FP8BS_BSCALE_BLOCK = 0, /* 128x128 blocks: SB(n,g) = sb[(n/128)*sb_s0 + g*sb_s1] */
    FP8BS_BSCALE_TILE = 1   /* 128x1 tiles:    SB(n,g) = sb[g*sb_s0 + n]            */
};

/* Version of this ABI (FP8BS_ABI_VERSION). */
int fp8bs_abi_version(void);

/* Static text for a status code (never NULL). */
const char *fp8bs_status_string(int status);

/*
 * fp8_cast_e4m3 -- q[i] = E4M3 code of x[i] for i < n: nearest value, ties
 * to the even code, |x| >= 448 saturating to +-448, sign kept for values
 * that round to zero.  This is the final rounding step of every quantiser
 * (the cast to FP8 of [qna-131281]'s online quantisation), exposed on its
 * own.  x: fp32 [n], finite, 16-byte aligned; q: uint8 [n], 4-byte aligned.
 * Errors: ERR_ARG (null pointer with n > 0, n < 0), ERR_DEVICE, ERR_HIP.
 */
int fp8_cast_e4m3(const float *x, int64_t n, uint8_t *q, void *stream);

/*
 * fp8_quant_tile -- online quantisation of activations in 1x128 or 128x1
 * groups ([qna-131281] fine-grained quantisation passage; [hacks-368261]
 * 128x1 tiles for the backward pass).
 *
 *   x      bf16 bits [rows][ldx], row-major.
 *   axis   FP8BS_AXIS_ROW: group (r, g) = x[r][128g .. 128g+127];
 *            q is [rows][ldq] (same orientation as x);
 *            s[g*lds + r] is the scale of group (r, g), g < cols/128.
 *            cols must be a multiple of 128; rows is any value >= 0.
 *          FP8BS_AXIS_COL: group (g, c) = x[128g .. 128g+127][c];
 *            q is written TRANSPOSED, [cols][ldq], so q[c][128g + i] is the
 *            code of x[128g + i][c] and each group is 128 contiguous bytes;
 *            s[g*lds + c] is the scale of group (g, c), g < rows/128.
 *            rows must be a multiple of 128; cols is any value >= 0.
 *   scale_mode  FP8BS_SCALE_FP32 or FP8BS_SCALE_POW2.
 *   Group amax is floored at 448*2^-126 so an all-zero group gets
 *   s = 2^-126 and zero codes.
 *
 * Alignment: x and q 16-byte aligned; ldx a multiple of 8 elements; ldq a
 * multiple of 16 bytes; s 4-byte aligned.  ldx >= cols; ldq >= cols (ROW)
 * or >= rows (COL); lds >= rows (ROW) or >= cols (COL).
 * Errors: ERR_ARG, ERR_SHAPE (grouped dimension % 128 != 0), ERR_ALIGN,
 * ERR_DEVICE, ERR_HIP.
 */
int fp8_quant_tile(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                   int axis, int scale_mode, uint8_t *q, int64_t ldq, float *s,
                   int64_t lds, void *stream);

/*
 * fp8_quant_block -- online quantisation of a weight matrix in 128x128
 * blocks (the weight grouping of the fine-grained quantisation,
 * [qna-131281] and [why-be-59061] passages on fine-grained scaling).
 *
 *   w     bf16 bits [rows][ldw]; cols must be a multiple of 128; a last
 *         partial block-row (rows % 128 != 0) holds only the rows present.
 *   q     codes [rows][ldq].
 *   qt    optional (NULL = skip) transposed copy of the codes, [cols][ldqt]:
 *         qt[c][r] == q[r][c].  A 128x128 block's scale does not depend on
 *         orientation, so qt with the transposed scales is the quantised W^T
 *         that Dgrad multiplies by.
 *   s     s[(r/128)*lds + c/128] is the scale of the block holding (r, c).
 *
 * Alignment: w, q, qt 16-byte aligned; ldw a multiple of 8; ldq and ldqt
 * multiples of 16; ldw, ldq >= cols; ldqt >= rows; lds >= cols/128.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_quant_block(const uint16_t *w, int64_t rows, int64_t cols,
                    int64_t ldw, int scale_mode, uint8_t *q, int64_t ldq,
                    uint8_t *qt, int64_t ldqt, float *s, int64_t lds,
                    void *stream);

/*
 * fp8_quant_tile_grouped_col -- 128x1 groups along the tokens of each MoE
 * expert, for the K-grouped expert Wgrad ([hacks-368261] 128x1 tiles of the
 * backward pass; [why-be-59061] expert GEMMs in FP8).  Reading: a group
 * never mixes two experts' tokens.
 *
 *   x        bf16 bits [T][ldx]: the tokens of G experts back to back,
 *            expert e owning rows offsets[e] .. offsets[e+1]-1.
 *   offsets  DEVICE int32 [G+1], offsets[0] = 0, non-decreasing,
 *            offsets[G] <= T (read only on the device).
 *   Each expert's tokens form groups of 128 from its first token, the last
 *   group holding the n_e mod 128 remaining ones (its amax over those
 *   only).  Groups are numbered on a padded token axis on which expert e
 *   starts at P_e = 128 * sum_{e'<e} ceil(n_e'/128):
 *   q        codes [cols][ldq], TRANSPOSED: q[c][P_e + i] encodes
 *            x[offsets[e] + i][c]; the padding of each expert's last group
 *            holds zero codes; bytes past the last group are not written.
 *   s        s[p*lds + c] is the scale of padded group p of column c.
 *   ldq must be >= fp8_grouped_col_bound(T, G) and s must hold
 *   fp8_grouped_col_bound(T, G)/128 rows.
 * Alignment: x, q 16-byte aligned; ldx a multiple of 8; ldq a multiple of
 * 16; s 4-byte aligned.  ldx >= cols, lds >= cols.
 * Errors: ERR_ARG, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_quant_tile_grouped_col(const uint16_t *x, int64_t T, int64_t cols,
                               int64_t ldx, int G, const int32_t *offsets,
                               int scale_mode, uint8_t *q, int64_t ldq,
                               float *s, int64_t lds, void *stream);

/* Padded token bound of fp8_quant_tile_grouped_col: 128 * (ceil(T/128) + G),
 * which is >= 128 * sum_e ceil(n_e/128) for any split of T tokens. */
int64_t fp8_grouped_col_bound(int64_t T, int G);

/*
 * fp8_quant_dual -- both activation groupings from one read of x: the 1x128
 * groups (as fp8_quant_tile with FP8BS_AXIS_ROW) and the 128x1 groups (as
 * FP8BS_AXIS_COL), for a gradient that feeds both Dgrad and Wgrad
 * ([hacks-368261], passage on the backward pass needing 128x1 tiles next
 * to the 1x128 tiles, and on the HBM round trips quantisation costs).
 * Outputs equal the two fp8_quant_tile calls bit for bit.
 *
 *   x      bf16 bits [rows][ldx]; rows and cols multiples of 128.
 *   qr, sr the ROW outputs: qr [rows][ldqr], sr[g*ldsr + r].
 *   qc, sc the COL outputs: qc [cols][ldqc] (transposed), sc[g*ldsc + c].
 *
 * Alignment: x, qr, qc 16-byte aligned; ldx a multiple of 8; ldqr and ldqc
 * multiples of 16; sr, sc 4-byte aligned.  ldx, ldqr >= cols; ldqc >= rows;
 * ldsr >= rows; ldsc >= cols.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_quant_dual(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                   int scale_mode, uint8_t *qr, int64_t ldqr, float *sr,
                   int64_t ldsr, uint8_t *qc, int64_t ldqc, float *sc,
                   int64_t ldsc, void *stream);

/*
 * fp8_requant_col -- backward re-tiling ([hacks-368261], passage on the
 * backward pass reading the FP8 activations back, dequantising them,
 * transposing them and re-quantising them into 128x1 tiles).
 *
 *   q     codes [rows][ldq] quantised in 1x128 row groups, with
 *   s     their scales s[g*lds + r] (g < cols/128) -- the layout
 *         fp8_quant_tile writes for FP8BS_AXIS_ROW.
 *   The matrix is dequantised element by element as the fp32 product
 *   x = decode(q) * s (one rounding), transposed, and quantised again in
 *   128x1 groups down its columns with `scale_mode`:
 *   qt    codes [cols][ldqt], written TRANSPOSED: qt[c][128g + i] encodes
 *         x[128g + i][c];
 *   st    st[g*ldst + c] is the scale of group (g, c), g < rows/128 -- the
 *         layout fp8_quant_tile writes for FP8BS_AXIS_COL.
 *   rows and cols must be multiples of 128.  The dequantised values must be
 *   finite fp32: codes 0x7F / 0xFF (NaN, never produced by the quantisers)
 *   and power-of-two scales of groups whose amax lies within 1/16 of the
 *   fp32 maximum (their largest code times the scale overflows) are
 *   outside the contract.
 *
 * Alignment: q and qt 16-byte aligned, ldq and ldqt multiples of 16; s
 * 16-byte aligned with lds a multiple of 4; st 4-byte aligned.  ldq >= cols,
 * lds >= rows, ldqt >= rows, ldst >= cols.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_requant_col(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                    const float *s, int64_t lds, int scale_mode, uint8_t *qt,
                    int64_t ldqt, float *st, int64_t ldst, void *stream);

/*
 * fp8_scales_are_pow2 -- whether every scale of a power-of-two
 * quantisation really is one.  FP8BS_ACCUM_MFMA8_POW2 hands the scales to
 * the matrix cores as E8M0 exponents ([cameseeing-1171527], passage
 * relating the fine-grained scaling to microscaling formats), which keep
 * only the exponent: any other scale gives wrong products without an
 * error.  This check lets a caller (or a debug build of its own) verify
 * the scales first.
 *
 *   s      fp32 array, entry (r, c) at s[r*ld_r + c*ld_c], r < rows, c < cols
 *          (ld_r, ld_c >= 0; e.g. fp8_quant_tile's row scales: rows = K/128,
 *          cols = M, ld_r = lds, ld_c = 1; block scales addressed as the
 *          GEMM's SB: rows = ceil(N/128), cols = K/128, ld_r = sb_s0,
 *          ld_c = sb_s1).
 *   flag   one int32 in device memory, written on the stream: 1 when every
 *          entry is a positive normal power of two (sign 0, exponent field
 *          1..254, mantissa 0), else 0; an empty array gives 1.  The caller
 *          reads it after synchronising the stream.
 * Alignment: s and flag 4-byte aligned.
 * Errors: ERR_ARG (negative size or stride, null pointer), ERR_ALIGN,
 * ERR_DEVICE, ERR_HIP.
 */
int fp8_scales_are_pow2(const float *s, int64_t rows, int64_t cols,
                        int64_t ld_r, int64_t ld_c, int32_t *flag,
                        void *stream);

/*
 * fp8_gemm_blockscaled -- block-scaled FP8 GEMM with FP32 promotion every
 * 128-element K group ([why-be-59061] 128-element interval passage;
 * [cameseeing-1171527] Figure 7(b) passage; [why-be-59061] Figure 6
 * passage for Fprop / Dgrad / Wgrad):
 *
 *   D[m][n] = sum_{g < K/128} sa[g*ldsa + m] * SB(n, g) *
 *             sum_{k = 128g}^{128g+127} dec(a[m*lda + k]) * dec(b[n*ldb + k])
 *
 * Each group's inner sum is formed on the matrix cores (see FP8BS_ACCUM_*)
 * and multiplied by its two scales into an FP32 accumulator, which is
 * rounded once to the output type (bf16: round to nearest even).
 *   a      E4M3 codes [M][lda], K contiguous.
 *   sa     per-row scale of each K group of a: sa[g*ldsa + m].
 *   b      E4M3 codes [N][ldb], K contiguous ("TN": both operands K-major).
 *   sb, bscale_kind, sb_s0, sb_s1   scales of b, addressed as SB(n, g)
 *          above.  Fprop (B = W from fp8_quant_block):  BLOCK, s0 = lds, s1 = 1.
 *          Dgrad (B = qt of W, its scales transposed): BLOCK, s0 = 1, s1 = lds.
 *          Wgrad (B from fp8_quant_tile COL):          TILE,  s0 = lds.
 *   d      output [M][ldd], bf16 bits (FP8BS_OUT_BF16) or fp32 (FP8BS_OUT_F32).
 *   accum  FP8BS_ACCUM_FP32, FP8BS_ACCUM_MFMA8 or FP8BS_ACCUM_MFMA8_POW2.
 *   workspace  device scratch of at least fp8_gemm_workspace_bytes(M, N, K)
 *          bytes (may be NULL when that is 0); it holds split-K partials
 *          when K is long and the output small.  The reduction over splits
 *          is in a fixed order, so results are run-to-run deterministic.
 * K must be a multiple of 128 (K == 0 writes zeros); M, N >= 0 (0 = no-op).
 * Alignment: a, b 16-byte aligned, lda and ldb multiples of 16 (when
 * K > 0); d 16-byte
 * aligned, ldd a multiple of 4 elements; sa, sb 4-byte aligned.
 * lda, ldb >= K; ldd >= N; ldsa >= M; lda, ldb <= FP8BS_MAX_LD (every GEMM
 * call below has the same bound).
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DEVICE, ERR_HIP.
 */
int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t *a,
                         int64_t lda, const float *sa, int64_t ldsa,
                         const uint8_t *b, int64_t ldb, const float *sb,
                         int bscale_kind, int64_t sb_s0, int64_t sb_s1,
                         void *d, int64_t ldd, int out_dtype, int accum,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/* Workspace bytes fp8_gemm_blockscaled needs for this shape (0 = none). */
size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Size of the device scratch array each GPU holds for
 * fp8_gemm_blockscaled_noalloc: 16 MiB (the split-K partials of a
 * 256 x 256 output over K = 65536). */
#define FP8BS_NOALLOC_SCRATCH_BYTES (16LL << 20)

/*
 * fp8_gemm_blockscaled_noalloc -- fp8_gemm_blockscaled for callers that
 * cannot allocate device memory: code under HIP graph capture, serving
 * loops that must not call the allocator, harnesses that forbid it.  It
 * takes no workspace: the split-K partials that fp8_gemm_blockscaled keeps
 * in the caller's workspace go to a device array of
 * FP8BS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, at the
 * first call on that device).  The call allocates and frees nothing and
 * gives the same results as fp8_gemm_blockscaled (the same kernels and split
 * count).  Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (different streams, or several host threads)
 * race on it and give undefined results; calls on one stream are ordered.
 * Arguments, layouts and alignment as fp8_gemm_blockscaled.
 * Errors: as fp8_gemm_blockscaled; ERR_WORKSPACE when the shape needs more
 * than FP8BS_NOALLOC_SCRATCH_BYTES (fp8_gemm_workspace_bytes(M, N, K)
 * above it); ERR_HIP when the array's address cannot be obtained.
 */
int fp8_gemm_blockscaled_noalloc(int64_t M, int64_t N, int64_t K,
                                 const uint8_t *a, int64_t lda,
                                 const float *sa, int64_t ldsa,
                                 const uint8_t *b, int64_t ldb,
                                 const float *sb, int bscale_kind,
                                 int64_t sb_s0, int64_t sb_s1, void *d,
                                 int64_t ldd, int out_dtype, int accum,
                                 void *stream);

/*
 * fp8_gemm_blockscaled_quant -- the block-scaled GEMM with its output
 * quantised in the epilogue, so a layer's activation leaves the kernel that
 * produces it already in FP8 and never makes a BF16 round trip through HBM
 * (the pages name that round trip -- read BF16 back, quantise, write FP8,
 * read again for the next MMA -- as the cost to remove: [hacks-368261],
 * passages on fusing FP8 casting with memory access).  The result is
 * exactly what fp8_gemm_blockscaled with FP8BS_OUT_BF16 followed by
 * fp8_quant_tile(FP8BS_AXIS_ROW, scale_mode) of that bf16 matrix would give:
 *   q   codes [M][ldq]; s[g*lds + m] the scale of row m, columns 128g..128g+127.
 * Other arguments as fp8_gemm_blockscaled.  N must be a multiple of 128.
 * The K loop is never split (long-K shapes with few output tiles run at
 * lower occupancy than in fp8_gemm_blockscaled).
 * Alignment: q 4-byte aligned, ldq a multiple of 4; s 4-byte aligned;
 * ldq >= N; lds >= M; otherwise as fp8_gemm_blockscaled.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_gemm_blockscaled_quant(int64_t M, int64_t N, int64_t K,
                               const uint8_t *a, int64_t lda, const float *sa,
                               int64_t ldsa, const uint8_t *b, int64_t ldb,
                               const float *sb, int bscale_kind, int64_t sb_s0,
                               int64_t sb_s1, int scale_mode, uint8_t *q,
                               int64_t ldq, float *s, int64_t lds, int accum,
                               void *stream);

/*
 * fp8_grouped_gemm -- the block-scaled GEMM for a group of MoE experts
 * (expert GEMMs in FP8, [why-be-59061] passage on the activation gradient
 * before the MoE down-projection; few, memory-bound tokens per expert in
 * decoding, [why-be-59061] decoding passage).  Rows offsets[e] ..
 * offsets[e+1]-1 of a (and of d) belong to expert e:
 *
 *   D[m][n] = sum_g sa[g*ldsa + m] * sb[e][n/128][g] *
 *             sum_{k in g} dec(a[m*lda + k]) * dec(b[e][n][k])
 *
 *   offsets  DEVICE int32 [G+1], offsets[0] = 0, non-decreasing,
 *            offsets[G] <= rows_bound.  Read only on the device, so no host
 *            synchronisation is needed; offsets that break this contract
 *            give undefined results.  Empty experts are allowed.
 *   rows_bound  host-side upper bound of offsets[G] (rows of a, sa, d).
 *   a, sa    codes [rows][lda] and scales sa[g*ldsa + m] of all rows
 *            (fp8_quant_tile ROW of the rows gathered per expert).
 *   b        codes [G][N][K] (contiguous), sb  block scales [G][N/128][K/128].
 *   d        output [rows][ldd], bf16 or fp32 as out_dtype.
 *   accum    one of FP8BS_ACCUM_*, as for the dense GEMM.
 * N and K must be multiples of 128.  Alignment as fp8_gemm_blockscaled;
 * ldsa >= rows_bound.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_grouped_gemm(int G, int64_t rows_bound, int64_t N, int64_t K,
                     const int32_t *offsets, const uint8_t *a, int64_t lda,
                     const float *sa, int64_t ldsa, const uint8_t *b,
                     const float *sb, void *d, int64_t ldd, int out_dtype,
                     int accum, void *stream);

/*
 * fp8_grouped_gemm_kgrouped -- the K-grouped expert GEMM of the MoE
 * backward pass: expert e's weight gradient sums over its own tokens,
 *
 *   D_e[m][n] = sum_{p = P_e/128}^{P_e/128 + ceil(n_e/128) - 1}
 *               sa[p*ldsa + m] * sb[p*ldsb + n] *
 *               sum_{k in p} dec(a[m*lda + k]) * dec(b[n*ldb + k])
 *
 * with a, sa and b, sb both from fp8_quant_tile_grouped_col (dY and X of the
 * expert-sorted tokens; padded token axis, zero codes in the padding, so
 * partial groups add nothing extra).  D_e is [M][ldd] at d + e*d_estride
 * elements; an expert without tokens gets zeros.
 *   offsets  the same DEVICE token offsets [G+1] the quantiser used.
 *   K        the padded token bound the operands were laid out for
 *            (a multiple of 128, >= 128 * sum_e ceil(n_e/128)).
 * Alignment as fp8_gemm_blockscaled; lda, ldb >= K; ldsa >= M; ldsb >= N;
 * d_estride >= M*ldd and a multiple of 4.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_grouped_gemm_kgrouped(int G, int64_t M, int64_t N, int64_t K,
                              const int32_t *offsets, const uint8_t *a,
                              int64_t lda, const float *sa, int64_t ldsa,
                              const uint8_t *b, int64_t ldb, const float *sb,
                              int64_t ldsb, void *d, int64_t ldd,
                              int64_t d_estride, int out_dtype, int accum,
                              void *stream);

/*
 * fp8_grouped_gemm_strided -- fp8_grouped_gemm with the experts' B codes and
 * scales addressed by strides, so the same call serves the MoE backward
 * GEMMs that read the forward weights transposed (M-grouped Dgrad:
 * dX_e = dY_e * W_e from the transposed copy of the stacked weight
 * quantisation; all three GEMMs in FP8, [why-be-59061] Figure 6 passage):
 *
 *   D[m][n] = sum_g sa[g*ldsa + m] * SB_e(n, g) *
 *             sum_{k in g} dec(a[m*lda + k]) * dec(b[e*b_estride + n*ldb + k])
 *   SB_e(n, g) = sb[e*sb_estride + (n/128)*sb_s0 + g*sb_s1]   (BLOCK)
 *              = sb[e*sb_estride + g*sb_s0 + n]              (TILE)
 *
 * for rows m of expert e (offsets[e] <= m < offsets[e+1]); other arguments
 * as fp8_grouped_gemm.  K must be a multiple of 128 (N any); b_estride a
 * multiple of 16; alignment otherwise as fp8_gemm_blockscaled.
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP.
 */
int fp8_grouped_gemm_strided(int G, int64_t rows_bound, int64_t N, int64_t K,
                             const int32_t *offsets, const uint8_t *a,
                             int64_t lda, const float *sa, int64_t ldsa,
                             const uint8_t *b, int64_t ldb, int64_t b_estride,
                             const float *sb, int bscale_kind, int64_t sb_s0,
                             int64_t sb_s1, int64_t sb_estride, void *d,
                             int64_t ldd, int out_dtype, int accum,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8BS_H */
