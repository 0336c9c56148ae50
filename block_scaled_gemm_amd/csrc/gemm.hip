// gemm.hip -- block-scaled FP8 GEMM for gfx950.
//
// D[m][n] = sum_g sa[g][m] * SB(n,g) * P_g[m][n], P_g the 128-element group
// partial.  Each group's partial is formed on the matrix cores from zero and
// promoted into an FP32 register accumulator with one FMA per output element
// (the per-group dequantisation rides on that FMA), as the pages' promotion
// every 128 elements does.
//
// Two ways of forming P_g (the `accum` argument):
//
//  ACC_F32 (default).  The gfx950 FP8 matrix cores do not add their products
//  at FP32 accuracy: on crafted inputs every FP8 MFMA form loses about 2^-12
//  of the largest product inside one instruction -- the limited accumulation
//  the pages measure on their own tensor cores.  This path therefore widens
//  the E4M3 tiles exactly to f16 while staging them into LDS
//  (v_cvt_scalef32_pk_f16_fp8 with scale 1 is exact for every finite code)
//  and forms P_g with v_mfma_f32_32x32x16_f16, whose products are exact and
//  whose sums are FP32-accurate.  Tiles 128x128 per 256-thread workgroup,
//  64x64 per wave as 2x2 sub-tiles of 32x32, 8 MFMAs per sub-tile per group.
//
//  ACC_MFMA8.  P_g straight from v_mfma_f32_16x16x128_f8f6f4 (one MFMA = one
//  K group for a 16x16 sub-tile), at twice the matrix-core rate, with the
//  matrix core's own limited accumulation inside the group.  Tiles 128x128,
//  64x64 per wave as 4x4 sub-tiles of 16x16.
//
// Both: the MFMA's first operand is the B (weight) tile and its second the
// A (activation) tile, so each result sub-tile is D^T and every lane ends
// with runs of four consecutive output columns of one row (one 8-byte bf16
// or 16-byte fp32 store) and needs a single activation scale per sub-tile.
// Both operands feed each lane the same k positions, so whatever order the
// hardware pairs elements in, it pairs equal k.
//
// Each K group of both tiles is staged global -> registers -> LDS, double-
// buffered (the next group's loads are in flight while the current one is
// multiplied), rows XOR-swizzled in 16-byte chunks so fragment reads of
// consecutive rows hit distinct banks.
#include "device.h"
#include "kernels.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int BM = 128;
constexpr int BN = 128;

// ---- tile description and workgroup -> tile order ---------------------------------

struct Tile {
    int64_t m0, m_end;  // rows [m0, min(m0+BM, m_end)) are real
    int64_t n0, n_end;
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    const float* sb;
    int64_t sb_s0, sb_s1;
};

// The 8 XCDs each take a contiguous range of the tile list (the hardware
// hands workgroups to XCDs round-robin), and inside it tiles walk down GM
// m-tiles before moving to the next n-tile, so the tiles resident on one
// XCD share A rows and B rows in its L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t wid, int64_t nwg) {
    if (nwg % 8 != 0) return wid;
    return (wid % 8) * (nwg / 8) + wid / 8;
}

__device__ __forceinline__ void tile_coords(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                            int64_t& tn) {
    constexpr int64_t GM = 8;
    const int64_t per = GM * tiles_n;
    const int64_t grp = t / per;
    const int64_t first = grp * GM;
    const int64_t gm = tiles_m - first < GM ? tiles_m - first : GM;
    const int64_t r = t % per;
    tm = first + r % gm;
    tn = r / gm;
}

// ---- staging: one K group of both tiles, global -> registers ----------------------------
//
// 1024 16-byte chunks per 128x128 FP8 tile: thread t takes chunks t + 256j,
// i.e. row (t + 256j) / 8 and k-chunk t % 8, so 8 lanes cover a 128-byte row.

struct Stage {
    uint4 a[4];
    uint4 b[4];
    float s;    // sa of row t (t < 128) or, for tile-kind B scales, sb of column t-128
    float sbk;  // block-kind B scale of this group (uniform)
};

template <int KIND>
__device__ __forceinline__ void load_stage(Stage& st, const Tile& T, int64_t g, int t) {
    const int64_t k0 = g * 128;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int cid = t + 256 * j;
        const int row = cid >> 3, kc = cid & 7;
        int64_t ma = T.m0 + row;
        ma = ma < T.m_end ? ma : T.m_end - 1;
        int64_t nb = T.n0 + row;
        nb = nb < T.n_end ? nb : T.n_end - 1;
        st.a[j] = *(const uint4*)(T.a + ma * T.lda + k0 + kc * 16);
        st.b[j] = *(const uint4*)(T.b + nb * T.ldb + k0 + kc * 16);
    }
    if (t < 128) {
        int64_t m = T.m0 + t;
        m = m < T.m_end ? m : T.m_end - 1;
        st.s = T.sa[g * T.ldsa + m];
    } else if (KIND == 1) {
        int64_t n = T.n0 + (t - 128);
        n = n < T.n_end ? n : T.n_end - 1;
        st.s = T.sb[g * T.sb_s0 + n];
    }
    if (KIND == 0) st.sbk = T.sb[(T.n0 >> 7) * T.sb_s0 + g * T.sb_s1];
}

template <int KIND>
__device__ __forceinline__ void store_scales(const Stage& st, float* lsa, float* lsb, int t) {
    if (t < 128)
        lsa[t] = st.s;
    else if (KIND == 1)
        lsb[t - 128] = st.s;
}

// ==== ACC_F32 path: exact f16 widening, f16 matrix cores =============================
//
// LDS tile: 128 rows x 128 f16 = 256 B per row, 16 chunks of 16 B, chunk c
// of row r stored at position c ^ (r & 15).

constexpr int F16_TILE = 128 * 256;  // bytes

__device__ __forceinline__ int f16_off(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// 16 E4M3 codes -> 16 f16 values (exact), as two 16-byte chunks.
__device__ __forceinline__ void widen16(uint4 v, uint4& lo, uint4& hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
        h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
    }
    lo = make_uint4(h[0], h[1], h[2], h[3]);
    hi = make_uint4(h[4], h[5], h[6], h[7]);
}

__device__ __forceinline__ void store_stage_f16(const Stage& st, uint8_t* la, uint8_t* lb, int t) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int cid = t + 256 * j;
        const int row = cid >> 3, kc = cid & 7;
        uint4 lo, hi;
        widen16(st.a[j], lo, hi);
        *(uint4*)(la + f16_off(row, 2 * kc)) = lo;
        *(uint4*)(la + f16_off(row, 2 * kc + 1)) = hi;
        widen16(st.b[j], lo, hi);
        *(uint4*)(lb + f16_off(row, 2 * kc)) = lo;
        *(uint4*)(lb + f16_off(row, 2 * kc + 1)) = hi;
    }
}

__device__ __forceinline__ v8h f16_frag(const uint8_t* tile, int row, int chunk) {
    return __builtin_bit_cast(v8h, *(const uint4*)(tile + f16_off(row, chunk)));
}

// acc[i][j]: 32x32 sub-tile (m-sub i, n-sub j) of this wave, D^T layout:
// register r of lane l is n = 32j + 8(r/4) + 4(l/32) + r%4, m = 32i + l%32.
template <int KIND>
__device__ __forceinline__ void mainloop_f32(const Tile& T, int64_t g0, int64_t g1, v16f (&acc)[2][2],
                                             uint8_t* smem, float* ssa, float* ssb) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    if (g0 >= g1) return;

    Stage st;
    load_stage<KIND>(st, T, g0, t);
    store_stage_f16(st, smem, smem + F16_TILE, t);
    store_scales<KIND>(st, ssa, ssb, t);
    float sbk = st.sbk;
    __syncthreads();

    for (int64_t g = g0; g < g1; g++) {
        const int buf = (int)((g - g0) & 1);
        const bool more = g + 1 < g1;
        if (more) load_stage<KIND>(st, T, g + 1, t);

        const uint8_t* la = smem + buf * 2 * F16_TILE;
        const uint8_t* lb = la + F16_TILE;
        const float* lsa = ssa + buf * 128;
        const float* lsb = ssb + buf * 128;

        v16f p[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) p[i][j][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int chunk = 2 * s + (lane >> 5);
            v8h af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; i++) af[i] = f16_frag(la, wm * 64 + 32 * i + (lane & 31), chunk);
#pragma unroll
            for (int j = 0; j < 2; j++) bf[j] = f16_frag(lb, wn * 64 + 32 * j + (lane & 31), chunk);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], p[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const float sam = lsa[wm * 64 + 32 * i + (lane & 31)];
            const float c = KIND == 0 ? sam * sbk : sam;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                if (KIND == 0) {
                    acc[i][j] += p[i][j] * c;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const v4f sbn = *(const v4f*)(lsb + wn * 64 + 32 * j + 8 * q + 4 * (lane >> 5));
#pragma unroll
                        for (int e = 0; e < 4; e++) acc[i][j][4 * q + e] += (p[i][j][4 * q + e] * c) * sbn[e];
                    }
                }
            }
        }

        if (more) {
            const int nb = buf ^ 1;
            uint8_t* na = smem + nb * 2 * F16_TILE;
            store_stage_f16(st, na, na + F16_TILE, t);
            store_scales<KIND>(st, ssa + nb * 128, ssb + nb * 128, t);
            sbk = st.sbk;
        }
        __syncthreads();
    }
}

// Store four consecutive columns n..n+3 of row m (masked at the edges).
template <int OUT_F32>
__device__ __forceinline__ void store4(void* d, int64_t ldd, int64_t m, int64_t n, int64_t n_end, float v0,
                                       float v1, float v2, float v3) {
    if (OUT_F32) {
        float* p = (float*)d + m * ldd + n;
        if (n + 4 <= n_end) {
            *(float4*)p = make_float4(v0, v1, v2, v3);
        } else {
            const float vv[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4 && n + e < n_end; e++) p[e] = vv[e];
        }
    } else {
        uint16_t* p = (uint16_t*)d + m * ldd + n;
        const uint32_t b0 = f32_to_bf16_bits(v0), b1 = f32_to_bf16_bits(v1);
        const uint32_t b2 = f32_to_bf16_bits(v2), b3 = f32_to_bf16_bits(v3);
        if (n + 4 <= n_end) {
            *(uint2*)p = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
            const uint32_t bb[4] = {b0, b1, b2, b3};
            for (int e = 0; e < 4 && n + e < n_end; e++) p[e] = (uint16_t)bb[e];
        }
    }
}

template <int OUT_F32>
__device__ __forceinline__ void store_tile_f32(const v16f (&acc)[2][2], int64_t m0, int64_t m_end, int64_t n0,
                                               int64_t n_end, void* d, int64_t ldd) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t m = m0 + wm * 64 + 32 * i + (lane & 31);
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t n = n0 + wn * 64 + 32 * j + 8 * q + 4 * (lane >> 5);
                if (n >= n_end) continue;
                store4<OUT_F32>(d, ldd, m, n, n_end, acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]);
            }
    }
}

// ==== ACC_MFMA8 path: FP8 matrix cores, one MFMA per K group =============================
//
// LDS tile: 128 rows x 128 B, 8 chunks of 16 B, chunk c of row r stored at
// position c ^ ((r ^ r>>3) & 7).

constexpr int F8_TILE = 128 * 128;

__device__ __forceinline__ int f8_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ void store_stage_f8(const Stage& st, uint8_t* la, uint8_t* lb, int t) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int cid = t + 256 * j;
        const int row = cid >> 3, kc = cid & 7;
        *(uint4*)(la + f8_off(row, kc)) = st.a[j];
        *(uint4*)(lb + f8_off(row, kc)) = st.b[j];
    }
}

__device__ __forceinline__ v8i f8_frag(const uint8_t* tile, int row, int c0) {
    const uint4 lo = *(const uint4*)(tile + f8_off(row, c0));
    const uint4 hi = *(const uint4*)(tile + f8_off(row, c0 + 1));
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ v4f mfma8_group(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // formats 0/0: both operands FP8 E4M3; no in-instruction scaling
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// acc[i][j]: 16x16 sub-tile (m-sub i, n-sub j), D^T layout: register e of
// lane l is n = 16j + 4(l/16) + e, m = 16i + l%16.
template <int KIND>
__device__ __forceinline__ void mainloop_mfma8(const Tile& T, int64_t g0, int64_t g1, v4f (&acc)[4][4],
                                               uint8_t* smem, float* ssa, float* ssb) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int c0 = 2 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (g0 >= g1) return;

    Stage st;
    load_stage<KIND>(st, T, g0, t);
    store_stage_f8(st, smem, smem + F8_TILE, t);
    store_scales<KIND>(st, ssa, ssb, t);
    float sbk = st.sbk;
    __syncthreads();

    for (int64_t g = g0; g < g1; g++) {
        const int buf = (int)((g - g0) & 1);
        const bool more = g + 1 < g1;
        if (more) load_stage<KIND>(st, T, g + 1, t);

        const uint8_t* la = smem + buf * 2 * F8_TILE;
        const uint8_t* lb = la + F8_TILE;
        const float* lsa = ssa + buf * 128;
        const float* lsb = ssb + buf * 128;

        v8i bf[4];
#pragma unroll
        for (int j = 0; j < 4; j++) bf[j] = f8_frag(lb, wn * 64 + 16 * j + (lane & 15), c0);
        v4f sbn[4];
        if (KIND == 1) {
#pragma unroll
            for (int j = 0; j < 4; j++) sbn[j] = *(const v4f*)(lsb + wn * 64 + 16 * j + 4 * (lane >> 4));
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int mrow = wm * 64 + 16 * i + (lane & 15);
            const v8i af = f8_frag(la, mrow, c0);
            const float sam = lsa[mrow];
            const float c = KIND == 0 ? sam * sbk : sam;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const v4f p = mfma8_group(bf[j], af);
                if (KIND == 0)
                    acc[i][j] += p * c;
                else
                    acc[i][j] += (p * c) * sbn[j];
            }
        }

        if (more) {
            const int nb = buf ^ 1;
            uint8_t* na = smem + nb * 2 * F8_TILE;
            store_stage_f8(st, na, na + F8_TILE, t);
            store_scales<KIND>(st, ssa + nb * 128, ssb + nb * 128, t);
            sbk = st.sbk;
        }
        __syncthreads();
    }
}

template <int OUT_F32>
__device__ __forceinline__ void store_tile_mfma8(const v4f (&acc)[4][4], int64_t m0, int64_t m_end, int64_t n0,
                                                 int64_t n_end, void* d, int64_t ldd) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t m = m0 + wm * 64 + 16 * i + (lane & 15);
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t n = n0 + wn * 64 + 16 * j + 4 * (lane >> 4);
            if (n >= n_end) continue;
            store4<OUT_F32>(d, ldd, m, n, n_end, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

// ==== kernels ==========================================================================

// LDS: two stages of both tiles plus two stages of 128 scales for A and B.
template <int ACC>
struct Smem {
    static constexpr int TILE = ACC == 0 ? F16_TILE : F8_TILE;
    static constexpr int BYTES = 2 * 2 * TILE;
};

// One tile over K groups [g0, g1), then its store.
template <int ACC, int KIND, int OUT_F32>
__device__ __forceinline__ void run_tile(const Tile& T, int64_t g0, int64_t g1, void* d, int64_t ldd,
                                         uint8_t* smem, float* ssa, float* ssb) {
    if (ACC == 0) {
        v16f acc[2][2];
        mainloop_f32<KIND>(T, g0, g1, acc, smem, ssa, ssb);
        store_tile_f32<OUT_F32>(acc, T.m0, T.m_end, T.n0, T.n_end, d, ldd);
    } else {
        v4f acc[4][4];
        mainloop_mfma8<KIND>(T, g0, g1, acc, smem, ssa, ssb);
        store_tile_mfma8<OUT_F32>(acc, T.m0, T.m_end, T.n0, T.n_end, d, ldd);
    }
}

template <int ACC, int KIND, int OUT_F32, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p, int64_t tiles_m, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<ACC>::BYTES];
    __shared__ __attribute__((aligned(16))) float ssa[2 * 128];
    __shared__ __attribute__((aligned(16))) float ssb[2 * 128];

    const int64_t ntiles = tiles_m * tiles_n;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t split = SPLIT ? wid / ntiles : 0;
    int64_t tm, tn;
    tile_coords(wid % ntiles, tiles_m, tiles_n, tm, tn);

    Tile T;
    T.m0 = tm * BM;
    T.m_end = p.M;
    T.n0 = tn * BN;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b;
    T.ldb = p.ldb;
    T.sb = p.sb;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = p.sb_s1;

    const int64_t groups = p.K / 128;
    int64_t g0 = 0, g1 = groups;
    if (SPLIT) {
        const int64_t per = (groups + p.splits - 1) / p.splits;
        g0 = split * per;
        g1 = g0 + per < groups ? g0 + per : groups;
        run_tile<ACC, KIND, 1>(T, g0, g1, p.ws + split * p.M * p.ws_ld, p.ws_ld, smem, ssa, ssb);
    } else {
        run_tile<ACC, KIND, OUT_F32>(T, g0, g1, p.d, p.ldd, smem, ssa, ssb);
    }
}

// Grouped: workgroup (expert e, n-tile) walks the expert's m-tiles.
template <int ACC, int OUT_F32>
__global__ __launch_bounds__(256) void grouped_kernel(GemmArgs p, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<ACC>::BYTES];
    __shared__ __attribute__((aligned(16))) float ssa[2 * 128];
    __shared__ __attribute__((aligned(16))) float ssb[2 * 128];

    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t e = wid / tiles_n;
    const int64_t tn = wid % tiles_n;
    const int64_t r0 = p.offsets[e], r1 = p.offsets[e + 1];

    Tile T;
    T.m_end = r1;
    T.n0 = tn * BN;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b + e * p.b_estride;
    T.ldb = p.K;
    T.sb = p.sb + e * p.sb_estride;
    T.sb_s0 = p.K / 128;
    T.sb_s1 = 1;
    for (int64_t m0 = r0; m0 < r1; m0 += BM) {
        T.m0 = m0;
        run_tile<ACC, 0, OUT_F32>(T, 0, p.K / 128, p.d, p.ldd, smem, ssa, ssb);
    }
}

// Sum split-K partials in split order and convert.
template <int OUT_F32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits,
                                                            int64_t M, int64_t N, int64_t ws_ld,
                                                            void* __restrict__ d, int64_t ldd) {
    const int64_t cols4 = (N + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * cols4) return;
    const int64_t m = idx / cols4, n = (idx % cols4) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; k++) {
        const float4 v = *(const float4*)(ws + (int64_t)k * M * ws_ld + m * ws_ld + n);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    store4<OUT_F32>(d, ldd, m, n, N, s.x, s.y, s.z, s.w);
}

// ==== host side ==========================================================================

int gemm_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t groups = K / 128;
    if (tiles == 0 || groups < 16 || tiles >= 256) return 1;
    int64_t s = 512 / tiles;         // aim for ~2 workgroups per CU
    const int64_t cap = groups / 8;  // at least 8 groups per split
    if (s > cap) s = cap;
    if (s > 256) s = 256;
    return s < 2 ? 1 : (int)s;
}

size_t gemm_workspace(int64_t M, int64_t N, int64_t K) {
    const int s = gemm_splits(M, N, K);
    if (s <= 1) return 0;
    return (size_t)s * (size_t)M * (size_t)((N + 3) / 4 * 4) * sizeof(float);
}

template <int ACC, int KIND, int OUT_F32, bool SPLIT>
static void launch_dense(const GemmArgs& g, int64_t tiles_m, int64_t tiles_n, int64_t wgs, hipStream_t st) {
    hipLaunchKernelGGL((gemm_kernel<ACC, KIND, OUT_F32, SPLIT>), dim3((unsigned)wgs), dim3(256), 0, st, g,
                       tiles_m, tiles_n);
}

template <int ACC>
static hipError_t launch_gemm_acc(const GemmArgs& g, hipStream_t st) {
    const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    if (g.splits > 1) {
        const int64_t wgs = tiles_m * tiles_n * g.splits;
        if (g.bscale_kind == 0)
            launch_dense<ACC, 0, 1, true>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<ACC, 1, 1, true>(g, tiles_m, tiles_n, wgs, st);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = g.M * ((g.N + 3) / 4);
        const dim3 grid((unsigned)((n + 255) / 256));
        if (g.out_f32)
            hipLaunchKernelGGL(splitk_reduce_kernel<1>, grid, dim3(256), 0, st, g.ws, g.splits, g.M, g.N, g.ws_ld,
                               g.d, g.ldd);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<0>, grid, dim3(256), 0, st, g.ws, g.splits, g.M, g.N, g.ws_ld,
                               g.d, g.ldd);
        return hipGetLastError();
    }
    const int64_t wgs = tiles_m * tiles_n;
    if (g.bscale_kind == 0) {
        if (g.out_f32)
            launch_dense<ACC, 0, 1, false>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<ACC, 0, 0, false>(g, tiles_m, tiles_n, wgs, st);
    } else {
        if (g.out_f32)
            launch_dense<ACC, 1, 1, false>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<ACC, 1, 0, false>(g, tiles_m, tiles_n, wgs, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    return g.accum == 0 ? launch_gemm_acc<0>(g, st) : launch_gemm_acc<1>(g, st);
}

template <int ACC>
static hipError_t launch_grouped_acc(const GemmArgs& g, hipStream_t st) {
    const int64_t tiles_n = g.N / BN;
    const dim3 grid((unsigned)(tiles_n * g.G));
    if (g.out_f32)
        hipLaunchKernelGGL((grouped_kernel<ACC, 1>), grid, dim3(256), 0, st, g, tiles_n);
    else
        hipLaunchKernelGGL((grouped_kernel<ACC, 0>), grid, dim3(256), 0, st, g, tiles_n);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.G == 0 || g.N == 0) return hipSuccess;
    return g.accum == 0 ? launch_grouped_acc<0>(g, st) : launch_grouped_acc<1>(g, st);
}

}  // namespace fp8bs
