// kernels.h -- internal launch interface between the C ABI (api.cpp) and the
// HIP kernels.  Launchers assume their arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bs {

hipError_t launch_cast(const float* x, int64_t n, uint8_t* q, hipStream_t st);

hipError_t launch_quant_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                             bool pow2, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             hipStream_t st);

hipError_t launch_quant_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw, bool pow2,
                              uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s,
                              int64_t lds, hipStream_t st);

// Padded token bound of the per-expert 128x1 grouping: 128 * (ceil(T/128) + G).
inline int64_t grouped_col_bound(int64_t T, int G) { return 128 * ((T + 127) / 128 + G); }

hipError_t launch_quant_grouped_col(const uint16_t* x, int64_t T, int64_t cols, int64_t ldx, int G,
                                    const int32_t* offsets, bool pow2, uint8_t* q, int64_t ldq, float* s,
                                    int64_t lds, hipStream_t st);

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool pow2, uint8_t* qr,
                             int64_t ldqr, float* sr, int64_t ldsr, uint8_t* qc, int64_t ldqc, float* sc,
                             int64_t ldsc, hipStream_t st);

hipError_t launch_scales_pow2_check(const float* s, int64_t rows, int64_t cols, int64_t ld_r, int64_t ld_c,
                                    int32_t* flag, hipStream_t st);
hipError_t launch_requant_col(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                              int64_t lds, bool pow2, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                              hipStream_t st_);

// Everything a block-scaled GEMM launch needs.  For a grouped launch,
// `offsets` is non-null, `G` experts share N and K, expert e's codes start at
// b + e*b_estride (rows ldb apart) and its B scales at sb + e*sb_estride
// (addressed through bscale_kind, sb_s0, sb_s1 as in a dense launch).
struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    const float* sb;
    int bscale_kind;  // 0 block, 1 tile
    int64_t sb_s0, sb_s1;
    void* d;
    int64_t ldd;
    int out_f32;  // 0 bf16, 1 fp32
    // fused quantisation of the bf16 result in 1x128 groups along n
    // (0 off, 1 FP32 scales, 2 power-of-two scales): codes to d, scales to
    // qs[(n/128)*qlds + m]
    int out_quant;
    float* qs;
    int64_t qlds;
    int accum;    // 0 FP32-accurate group partials (f16 matrix cores), 1 FP8 matrix cores,
                  // 2 FP8 matrix cores with the power-of-two scales inside the MFMA
    // split-K (dense only): partials in `ws`, row stride ws_ld floats
    float* ws;
    int splits;
    int64_t ws_ld;
    // grouped
    const int32_t* offsets;
    int G;
    int64_t b_estride, sb_estride;
    int64_t d_estride;  // K-grouped: expert e writes d + e*d_estride elements
};

// Split count the dense GEMM uses for this shape (1 = no split).
int gemm_splits(int64_t M, int64_t N, int64_t K);
// Workspace bytes the dense GEMM needs for this shape.
size_t gemm_workspace(int64_t M, int64_t N, int64_t K);
// Output columns the FP8 dense paths run on 256 x 256 tiles (the rest on
// 256 x 128 tiles), given the device's compute units; *cost_out, if given,
// receives the split's cost in rounds of 256 x 256 tiles.
int64_t wide_columns(int64_t M, int64_t N, int cus, double* cost_out = nullptr);

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st);
// K-grouped: expert e sums the K groups of its tokens on the padded token
// axis of the per-expert 128x1 grouping; B scales are per column (tile kind).
hipError_t launch_kgrouped_gemm(const GemmArgs& g, hipStream_t st);

}  // namespace fp8bs
