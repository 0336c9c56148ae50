// api.cpp -- the C ABI of libfp8bs.so (declared in include/fp8bs.h).
//
// Every entry point validates its arguments on the host first (no HIP call
// is made for a rejected call), then checks that the current device is a
// gfx950, then enqueues its kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/fp8bs.h"
#include "kernels.h"

#define FP8BS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// gfx950 check, cached per device ordinal.
int check_device() {
    static std::mutex mu;
    static int cache[64];  // 0 unknown, 1 ok, 2 not ok
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8BS_ERR_DEVICE;
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(mu);
        if (cache[dev] == 1) return FP8BS_OK;
        if (cache[dev] == 2) return FP8BS_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BS_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(mu);
        cache[dev] = ok ? 1 : 2;
    }
    return ok ? FP8BS_OK : FP8BS_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_HIP; }

}  // namespace

FP8BS_EXPORT int fp8bs_abi_version(void) { return FP8BS_ABI_VERSION; }

FP8BS_EXPORT const char* fp8bs_status_string(int status) {
    switch (status) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_ARG: return "invalid argument (null pointer, bad enum, negative size or leading dimension too small)";
        case FP8BS_ERR_SHAPE: return "a grouped dimension is not a multiple of 128";
        case FP8BS_ERR_ALIGN: return "pointer or leading dimension misaligned";
        case FP8BS_ERR_WORKSPACE: return "workspace missing or too small";
        case FP8BS_ERR_DEVICE: return "current device is not a gfx950 GPU";
        case FP8BS_ERR_HIP: return "HIP reported an error while launching";
        default: return "unknown status";
    }
}

FP8BS_EXPORT int fp8_cast_e4m3(const float* x, int64_t n, uint8_t* q, void* stream) {
    if (n < 0 || (n > 0 && (!x || !q))) return FP8BS_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 4)) return FP8BS_ERR_ALIGN;
    if (n == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_cast(x, n, q, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_quant_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                                int scale_mode, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                void* stream) {
    if (axis != FP8BS_AXIS_ROW && axis != FP8BS_AXIS_COL) return FP8BS_ERR_ARG;
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (rows < 0 || cols < 0) return FP8BS_ERR_ARG;
    if (rows > 0 && cols > 0 && (!x || !q || !s)) return FP8BS_ERR_ARG;
    if (ldx < cols) return FP8BS_ERR_ARG;
    if (axis == FP8BS_AXIS_ROW) {
        if (cols % 128 != 0) return FP8BS_ERR_SHAPE;
        if (ldq < cols || lds < rows) return FP8BS_ERR_ARG;
    } else {
        if (rows % 128 != 0) return FP8BS_ERR_SHAPE;
        if (ldq < rows || lds < cols) return FP8BS_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || ldx % 8 != 0 || ldq % 16 != 0)
        return FP8BS_ERR_ALIGN;
    if (rows == 0 || cols == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_quant_tile(x, rows, cols, ldx, axis, scale_mode == FP8BS_SCALE_POW2, q,
                                               ldq, s, lds, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_quant_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw, int scale_mode,
                                 uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s, int64_t lds,
                                 void* stream) {
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (rows < 0 || cols < 0) return FP8BS_ERR_ARG;
    if (rows > 0 && cols > 0 && (!w || !q || !s)) return FP8BS_ERR_ARG;
    if (cols % 128 != 0) return FP8BS_ERR_SHAPE;
    if (ldw < cols || ldq < cols || lds < cols / 128 || (qt && ldqt < rows)) return FP8BS_ERR_ARG;
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(qt, 16) || !aligned(s, 4) || ldw % 8 != 0 ||
        ldq % 16 != 0 || (qt && ldqt % 16 != 0))
        return FP8BS_ERR_ALIGN;
    if (rows == 0 || cols == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_quant_block(w, rows, cols, ldw, scale_mode == FP8BS_SCALE_POW2, q, ldq, qt,
                                                ldqt, s, lds, (hipStream_t)stream));
}

FP8BS_EXPORT int64_t fp8_grouped_col_bound(int64_t T, int G) {
    if (T < 0 || G < 0) return 0;
    return fp8bs::grouped_col_bound(T, G);
}

FP8BS_EXPORT int fp8_quant_tile_grouped_col(const uint16_t* x, int64_t T, int64_t cols, int64_t ldx, int G,
                                            const int32_t* offsets, int scale_mode, uint8_t* q, int64_t ldq,
                                            float* s, int64_t lds, void* stream) {
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (T < 0 || cols < 0 || G < 0) return FP8BS_ERR_ARG;
    if (G > 0 && cols > 0 && (!x || !offsets || !q || !s)) return FP8BS_ERR_ARG;
    if (ldx < cols || lds < cols || ldq < fp8bs::grouped_col_bound(T, G)) return FP8BS_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(offsets, 4) || ldx % 8 != 0 ||
        ldq % 16 != 0)
        return FP8BS_ERR_ALIGN;
    if (G == 0 || cols == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_quant_grouped_col(x, T, cols, ldx, G, offsets, scale_mode == FP8BS_SCALE_POW2, q,
                                                      ldq, s, lds, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int scale_mode,
                                uint8_t* qr, int64_t ldqr, float* sr, int64_t ldsr, uint8_t* qc, int64_t ldqc,
                                float* sc, int64_t ldsc, void* stream) {
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (rows < 0 || cols < 0) return FP8BS_ERR_ARG;
    if (rows > 0 && cols > 0 && (!x || !qr || !sr || !qc || !sc)) return FP8BS_ERR_ARG;
    if (rows % 128 != 0 || cols % 128 != 0) return FP8BS_ERR_SHAPE;
    if (ldx < cols || ldqr < cols || ldqc < rows || ldsr < rows || ldsc < cols) return FP8BS_ERR_ARG;
    if (!aligned(x, 16) || !aligned(qr, 16) || !aligned(qc, 16) || !aligned(sr, 4) || !aligned(sc, 4) ||
        ldx % 8 != 0 || ldqr % 16 != 0 || ldqc % 16 != 0)
        return FP8BS_ERR_ALIGN;
    if (rows == 0 || cols == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_quant_dual(x, rows, cols, ldx, scale_mode == FP8BS_SCALE_POW2, qr, ldqr, sr,
                                               ldsr, qc, ldqc, sc, ldsc, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_requant_col(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                                 int64_t lds, int scale_mode, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                                 void* stream) {
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (rows < 0 || cols < 0) return FP8BS_ERR_ARG;
    if (rows > 0 && cols > 0 && (!q || !s || !qt || !st)) return FP8BS_ERR_ARG;
    if (rows % 128 != 0 || cols % 128 != 0) return FP8BS_ERR_SHAPE;
    if (ldq < cols || lds < rows || ldqt < rows || ldst < cols) return FP8BS_ERR_ARG;
    if (!aligned(q, 16) || !aligned(qt, 16) || !aligned(s, 16) || !aligned(st, 4) || ldq % 16 != 0 ||
        ldqt % 16 != 0 || lds % 4 != 0)
        return FP8BS_ERR_ALIGN;
    if (rows == 0 || cols == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_requant_col(q, rows, cols, ldq, s, lds, scale_mode == FP8BS_SCALE_POW2, qt,
                                                ldqt, st, ldst, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_scales_are_pow2(const float* s, int64_t rows, int64_t cols, int64_t ld_r, int64_t ld_c,
                                     int32_t* flag, void* stream) {
    if (rows < 0 || cols < 0 || ld_r < 0 || ld_c < 0 || !flag) return FP8BS_ERR_ARG;
    if (rows > 0 && cols > 0 && !s) return FP8BS_ERR_ARG;
    if (!aligned(s, 4) || !aligned(flag, 4)) return FP8BS_ERR_ALIGN;
    if (int r = check_device()) return r;
    return hip_status(fp8bs::launch_scales_pow2_check(s, rows, cols, ld_r, ld_c, flag, (hipStream_t)stream));
}

FP8BS_EXPORT size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) return 0;
    return fp8bs::gemm_workspace(M, N, K);
}

namespace {

int check_gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                      int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb, void* d, int64_t ldd,
                      int out_dtype) {
    if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return FP8BS_ERR_ARG;
    if (M > 0 && N > 0) {
        if (!d) return FP8BS_ERR_ARG;
        if (K > 0 && (!a || !sa || !b || !sb)) return FP8BS_ERR_ARG;
    }
    if (K % 128 != 0) return FP8BS_ERR_SHAPE;
    if (lda > FP8BS_MAX_LD || ldb > FP8BS_MAX_LD) return FP8BS_ERR_SHAPE;  // 32-bit per-lane row offsets
    if (lda < K || ldb < K || ldd < N || ldsa < M) return FP8BS_ERR_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
        (K > 0 && (lda % 16 != 0 || ldb % 16 != 0)) || ldd % 4 != 0)
        return FP8BS_ERR_ALIGN;
    return FP8BS_OK;
}

}  // namespace

namespace {

// Argument checks of the dense GEMM apart from the workspace.
int check_gemm_dense(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                     const uint8_t* b, int64_t ldb, const float* sb, int bscale_kind, void* d, int64_t ldd,
                     int out_dtype, int accum) {
    if (bscale_kind != FP8BS_BSCALE_BLOCK && bscale_kind != FP8BS_BSCALE_TILE) return FP8BS_ERR_ARG;
    if (accum != FP8BS_ACCUM_FP32 && accum != FP8BS_ACCUM_MFMA8 && accum != FP8BS_ACCUM_MFMA8_POW2)
        return FP8BS_ERR_ARG;
    return check_gemm_common(M, N, K, a, lda, sa, ldsa, b, ldb, sb, d, ldd, out_dtype);
}

// Enqueue a validated dense GEMM; `ws` holds fp8_gemm_workspace_bytes(M, N, K)
// bytes (unused when that is 0).
int launch_dense_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                      int64_t ldsa, const uint8_t* b, int64_t ldb, const float* sb, int bscale_kind, int64_t sb_s0,
                      int64_t sb_s1, void* d, int64_t ldd, int out_dtype, int accum, void* ws, size_t need,
                      void* stream) {
    fp8bs::GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = a;
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
    g.b = b;
    g.ldb = ldb;
    g.sb = sb;
    g.bscale_kind = bscale_kind;
    g.sb_s0 = sb_s0;
    g.sb_s1 = sb_s1;
    g.d = d;
    g.ldd = ldd;
    g.out_f32 = out_dtype == FP8BS_OUT_F32;
    g.accum = accum;
    g.splits = need > 0 ? fp8bs::gemm_splits(M, N, K) : 1;
    g.ws = (float*)ws;
    g.ws_ld = (N + 3) / 4 * 4;
    return hip_status(fp8bs::launch_gemm(g, (hipStream_t)stream));
}

}  // namespace

FP8BS_EXPORT int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                      const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                                      const float* sb, int bscale_kind, int64_t sb_s0, int64_t sb_s1, void* d,
                                      int64_t ldd, int out_dtype, int accum, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (int r = check_gemm_dense(M, N, K, a, lda, sa, ldsa, b, ldb, sb, bscale_kind, d, ldd, out_dtype, accum))
        return r;
    if (M == 0 || N == 0) return FP8BS_OK;
    const size_t need = fp8_gemm_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || workspace_bytes < need)) return FP8BS_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
    if (int r = check_device()) return r;
    return launch_dense_gemm(M, N, K, a, lda, sa, ldsa, b, ldb, sb, bscale_kind, sb_s0, sb_s1, d, ldd, out_dtype,
                             accum, workspace, need, stream);
}

// ---- the dense GEMM without a caller workspace ---------------------------------------
//
// For callers that cannot allocate device memory: the split-K partials live
// in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a host-side stand-in, so it is never used as
// an address: at the first call on a device (with that device current)
// hipGetSymbolAddress gives that device's copy, which is kept per device and
// passed to the kernels.  Nothing here needs to start at zero (every split
// writes its whole partial before the reduction reads it).
static __device__ __align__(256) uint8_t scratch[FP8BS_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex scratch_mu;
void* scratch_ptr[64];

int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8BS_ERR_DEVICE;
    if (dev >= 64) return FP8BS_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8BS_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return FP8BS_OK;
}

}  // namespace

FP8BS_EXPORT int fp8_gemm_blockscaled_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                              const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                                              const float* sb, int bscale_kind, int64_t sb_s0, int64_t sb_s1,
                                              void* d, int64_t ldd, int out_dtype, int accum, void* stream) {
    if (int r = check_gemm_dense(M, N, K, a, lda, sa, ldsa, b, ldb, sb, bscale_kind, d, ldd, out_dtype, accum))
        return r;
    if (M == 0 || N == 0) return FP8BS_OK;
    const size_t need = fp8_gemm_workspace_bytes(M, N, K);
    if (need > (size_t)FP8BS_NOALLOC_SCRATCH_BYTES) return FP8BS_ERR_WORKSPACE;
    if (int r = check_device()) return r;
    void* ws = nullptr;
    if (need > 0)
        if (int r = device_scratch(&ws)) return r;
    return launch_dense_gemm(M, N, K, a, lda, sa, ldsa, b, ldb, sb, bscale_kind, sb_s0, sb_s1, d, ldd, out_dtype,
                             accum, ws, need, stream);
}

FP8BS_EXPORT int fp8_gemm_blockscaled_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                            const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                                            const float* sb, int bscale_kind, int64_t sb_s0, int64_t sb_s1,
                                            int scale_mode, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                            int accum, void* stream) {
    if (bscale_kind != FP8BS_BSCALE_BLOCK && bscale_kind != FP8BS_BSCALE_TILE) return FP8BS_ERR_ARG;
    if (scale_mode != FP8BS_SCALE_FP32 && scale_mode != FP8BS_SCALE_POW2) return FP8BS_ERR_ARG;
    if (accum != FP8BS_ACCUM_FP32 && accum != FP8BS_ACCUM_MFMA8 && accum != FP8BS_ACCUM_MFMA8_POW2)
        return FP8BS_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return FP8BS_ERR_ARG;
    if (M > 0 && N > 0 && (!q || !s || (K > 0 && (!a || !sa || !b || !sb)))) return FP8BS_ERR_ARG;
    if (K % 128 != 0 || N % 128 != 0) return FP8BS_ERR_SHAPE;
    if (lda > FP8BS_MAX_LD || ldb > FP8BS_MAX_LD) return FP8BS_ERR_SHAPE;  // 32-bit per-lane row offsets
    if (lda < K || ldb < K || ldq < N || ldsa < M || lds < M) return FP8BS_ERR_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(q, 4) || !aligned(sa, 4) || !aligned(sb, 4) ||
        !aligned(s, 4) || (K > 0 && (lda % 16 != 0 || ldb % 16 != 0)) || ldq % 4 != 0)
        return FP8BS_ERR_ALIGN;
    if (M == 0 || N == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    fp8bs::GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = a;
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
    g.b = b;
    g.ldb = ldb;
    g.sb = sb;
    g.bscale_kind = bscale_kind;
    g.sb_s0 = sb_s0;
    g.sb_s1 = sb_s1;
    g.d = q;
    g.ldd = ldq;
    g.out_f32 = 0;
    g.out_quant = scale_mode == FP8BS_SCALE_POW2 ? 2 : 1;
    g.qs = s;
    g.qlds = lds;
    g.accum = accum;
    g.splits = 1;
    return hip_status(fp8bs::launch_gemm(g, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_grouped_gemm(int G, int64_t rows_bound, int64_t N, int64_t K, const int32_t* offsets,
                                  const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                                  const float* sb, void* d, int64_t ldd, int out_dtype, int accum,
                                  void* stream) {
    if (G < 0 || rows_bound < 0) return FP8BS_ERR_ARG;
    if (accum != FP8BS_ACCUM_FP32 && accum != FP8BS_ACCUM_MFMA8 && accum != FP8BS_ACCUM_MFMA8_POW2)
        return FP8BS_ERR_ARG;
    if (G > 0 && !offsets) return FP8BS_ERR_ARG;
    if (N % 128 != 0) return FP8BS_ERR_SHAPE;
    if (int r = check_gemm_common(rows_bound, N, K, a, lda, sa, ldsa, b, K, sb, d, ldd, out_dtype)) return r;
    if (!aligned(offsets, 4)) return FP8BS_ERR_ALIGN;
    if (G == 0 || N == 0 || rows_bound == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    fp8bs::GemmArgs g{};
    g.M = rows_bound;
    g.N = N;
    g.K = K;
    g.a = a;
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
    g.b = b;
    g.ldb = K;
    g.sb = sb;
    g.bscale_kind = FP8BS_BSCALE_BLOCK;
    g.d = d;
    g.ldd = ldd;
    g.out_f32 = out_dtype == FP8BS_OUT_F32;
    g.accum = accum;
    g.splits = 1;
    g.offsets = offsets;
    g.G = G;
    g.b_estride = N * K;
    g.sb_s0 = K / 128;
    g.sb_s1 = 1;
    g.sb_estride = (N / 128) * (K / 128);
    return hip_status(fp8bs::launch_grouped_gemm(g, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_grouped_gemm_kgrouped(int G, int64_t M, int64_t N, int64_t K, const int32_t* offsets,
                                           const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                           const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb, void* d,
                                           int64_t ldd, int64_t d_estride, int out_dtype, int accum,
                                           void* stream) {
    if (G < 0) return FP8BS_ERR_ARG;
    if (accum != FP8BS_ACCUM_FP32 && accum != FP8BS_ACCUM_MFMA8 && accum != FP8BS_ACCUM_MFMA8_POW2)
        return FP8BS_ERR_ARG;
    if (G > 0 && !offsets) return FP8BS_ERR_ARG;
    if (int r = check_gemm_common(M, N, K, a, lda, sa, ldsa, b, ldb, sb, d, ldd, out_dtype)) return r;
    if (ldsb < N || d_estride < M * ldd) return FP8BS_ERR_ARG;
    if (!aligned(offsets, 4) || d_estride % 4 != 0) return FP8BS_ERR_ALIGN;
    if (G == 0 || M == 0 || N == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    fp8bs::GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = a;
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
    g.b = b;
    g.ldb = ldb;
    g.sb = sb;
    g.bscale_kind = FP8BS_BSCALE_TILE;
    g.sb_s0 = ldsb;
    g.sb_s1 = 0;
    g.d = d;
    g.ldd = ldd;
    g.d_estride = d_estride;
    g.out_f32 = out_dtype == FP8BS_OUT_F32;
    g.accum = accum;
    g.splits = 1;
    g.offsets = offsets;
    g.G = G;
    return hip_status(fp8bs::launch_kgrouped_gemm(g, (hipStream_t)stream));
}

FP8BS_EXPORT int fp8_grouped_gemm_strided(int G, int64_t rows_bound, int64_t N, int64_t K, const int32_t* offsets,
                                          const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                          const uint8_t* b, int64_t ldb, int64_t b_estride, const float* sb,
                                          int bscale_kind, int64_t sb_s0, int64_t sb_s1, int64_t sb_estride,
                                          void* d, int64_t ldd, int out_dtype, int accum, void* stream) {
    if (G < 0 || rows_bound < 0 || b_estride < 0 || sb_estride < 0) return FP8BS_ERR_ARG;
    if (bscale_kind != FP8BS_BSCALE_BLOCK && bscale_kind != FP8BS_BSCALE_TILE) return FP8BS_ERR_ARG;
    if (accum != FP8BS_ACCUM_FP32 && accum != FP8BS_ACCUM_MFMA8 && accum != FP8BS_ACCUM_MFMA8_POW2)
        return FP8BS_ERR_ARG;
    if (G > 0 && !offsets) return FP8BS_ERR_ARG;
    if (int r = check_gemm_common(rows_bound, N, K, a, lda, sa, ldsa, b, ldb, sb, d, ldd, out_dtype)) return r;
    if (!aligned(offsets, 4) || (K > 0 && b_estride % 16 != 0)) return FP8BS_ERR_ALIGN;
    if (G == 0 || N == 0 || rows_bound == 0) return FP8BS_OK;
    if (int r = check_device()) return r;
    fp8bs::GemmArgs g{};
    g.M = rows_bound;
    g.N = N;
    g.K = K;
    g.a = a;
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
    g.b = b;
    g.ldb = ldb;
    g.sb = sb;
    g.bscale_kind = bscale_kind;
    g.sb_s0 = sb_s0;
    g.sb_s1 = sb_s1;
    g.d = d;
    g.ldd = ldd;
    g.out_f32 = out_dtype == FP8BS_OUT_F32;
    g.accum = accum;
    g.splits = 1;
    g.offsets = offsets;
    g.G = G;
    g.b_estride = b_estride;
    g.sb_estride = sb_estride;
    return hip_status(fp8bs::launch_grouped_gemm(g, (hipStream_t)stream));
}
