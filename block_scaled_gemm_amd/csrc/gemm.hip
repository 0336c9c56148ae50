// gemm.hip -- block-scaled FP8 GEMM for gfx950.
//
// D[m][n] = sum_g sa[g][m] * SB(n,g) * P_g[m][n], P_g the 128-element group
// partial.  One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one K group for
// a 16x16 output sub-tile, so the group partial comes out of the matrix core
// in FP32 and is promoted into the FP32 accumulator with one FMA per element
// (the per-group dequantisation rides on that FMA).
//
// Operand roles: the MFMA's first operand is the B (weight) tile, its second
// the A (activation) tile, so the 16x16 result sub-tile is D^T: lane l holds
// outputs (n = 4*(l/16) + e, m = l%16), e = 0..3, i.e. four consecutive
// columns of one output row -- one 8-byte (bf16) or 16-byte (fp32) store.
//
// The K permutation inside a group does not matter as long as both operands
// use the same one: lane l feeds bytes [32*(l/16), 32*(l/16)+32) of its row
// of both tiles, so whatever order the hardware pairs bytes in, it pairs
// equal k.
//
// Tiles: 128 (m) x 128 (n) per 256-thread workgroup, 4 waves in a 2x2 grid,
// 64x64 per wave (16 MFMAs per group).  Each K group of both tiles is staged
// through LDS (2 x 16 KB, double-buffered), rows of 128 B with the 16-byte
// chunk index XOR-swizzled by (row ^ row>>3) & 7 so the fragment reads of
// 8 or 16 consecutive rows hit distinct banks.
#include "device.h"
#include "kernels.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int TILE_BYTES = 128 * 128;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int c0) {
    const int s = swz(row);
    const uint4 lo = *(const uint4*)(tile + row * 128 + ((c0 ^ s) << 4));
    const uint4 hi = *(const uint4*)(tile + row * 128 + (((c0 + 1) ^ s) << 4));
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ v4f mfma_group(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // formats 0/0: both operands FP8 E4M3; no in-instruction scaling
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Stage registers for one K group of one tile pair: 4 chunks of A and 4 of
// B per thread, plus one scale.
struct Stage {
    uint4 a[4];
    uint4 b[4];
    float s;
    float sbk;  // block-kind B scale of this group (uniform)
};

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
__device__ __forceinline__ void store_stage(const Stage& st, uint8_t* la, uint8_t* lb, float* lsa,
                                            float* lsb, int t) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int cid = t + 256 * j;
        const int row = cid >> 3, kc = cid & 7;
        const int off = row * 128 + ((kc ^ swz(row)) << 4);
        *(uint4*)(la + off) = st.a[j];
        *(uint4*)(lb + off) = st.b[j];
    }
    if (t < 128)
        lsa[t] = st.s;
    else if (KIND == 1)
        lsb[t - 128] = st.s;
}

// Accumulate one tile over K groups [g0, g1); acc[i][j] is the 16x16
// sub-tile (m-sub i, n-sub j) of this wave.
template <int KIND>
__device__ __forceinline__ void mainloop(const Tile& T, int64_t g0, int64_t g1, v4f (&acc)[4][4],
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
    store_stage<KIND>(st, smem, smem + TILE_BYTES, ssa, ssb, t);
    float sbk = st.sbk;
    __syncthreads();

    for (int64_t g = g0; g < g1; g++) {
        const int buf = (int)((g - g0) & 1);
        const bool more = g + 1 < g1;
        if (more) load_stage<KIND>(st, T, g + 1, t);

        const uint8_t* la = smem + buf * 2 * TILE_BYTES;
        const uint8_t* lb = la + TILE_BYTES;
        const float* lsa = ssa + buf * 128;
        const float* lsb = ssb + buf * 128;

        v8i bf[4];
#pragma unroll
        for (int j = 0; j < 4; j++) bf[j] = lds_frag(lb, wn * 64 + 16 * j + (lane & 15), c0);
        v4f sbn[4];
        if (KIND == 1) {
#pragma unroll
            for (int j = 0; j < 4; j++) sbn[j] = *(const v4f*)(lsb + wn * 64 + 16 * j + 4 * (lane >> 4));
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int mrow = wm * 64 + 16 * i + (lane & 15);
            const v8i af = lds_frag(la, mrow, c0);
            const float sam = lsa[mrow];
            const float c = KIND == 0 ? sam * sbk : sam;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const v4f p = mfma_group(bf[j], af);
                if (KIND == 0) {
                    acc[i][j] += p * c;
                } else {
                    acc[i][j] += (p * c) * sbn[j];
                }
            }
        }

        if (more) {
            const int nb = buf ^ 1;
            store_stage<KIND>(st, smem + nb * 2 * TILE_BYTES, smem + nb * 2 * TILE_BYTES + TILE_BYTES,
                              ssa + nb * 128, ssb + nb * 128, t);
            sbk = st.sbk;
        }
        __syncthreads();
    }
}

// Write the wave's 64x64 part of the tile: four consecutive columns per lane.
template <int OUT_F32>
__device__ __forceinline__ void store_tile(const v4f (&acc)[4][4], int64_t m0, int64_t m_end, int64_t n0,
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
            const v4f v = acc[i][j];
            if (OUT_F32) {
                float* p = (float*)d + m * ldd + n;
                if (n + 4 <= n_end) {
                    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    for (int e = 0; e < 4 && n + e < n_end; e++) p[e] = v[e];
                }
            } else {
                uint16_t* p = (uint16_t*)d + m * ldd + n;
                const uint32_t b0 = f32_to_bf16_bits(v[0]), b1 = f32_to_bf16_bits(v[1]);
                const uint32_t b2 = f32_to_bf16_bits(v[2]), b3 = f32_to_bf16_bits(v[3]);
                if (n + 4 <= n_end) {
                    *(uint2*)p = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                } else {
                    const uint32_t bb[4] = {b0, b1, b2, b3};
                    for (int e = 0; e < 4 && n + e < n_end; e++) p[e] = (uint16_t)bb[e];
                }
            }
        }
    }
}

// Workgroup -> tile order: the 8 XCDs each take a contiguous range of the
// tile list (the hardware hands workgroups to XCDs round-robin), and inside
// it tiles walk down GM m-tiles before moving to the next n-tile, so the
// tiles resident on one XCD share A rows and B rows in its L2.
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

template <int KIND, int OUT_F32, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs p, int64_t tiles_m, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * TILE_BYTES];
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
    }
    v4f acc[4][4];
    mainloop<KIND>(T, g0, g1, acc, smem, ssa, ssb);
    if (SPLIT)
        store_tile<1>(acc, T.m0, p.M, T.n0, p.N, p.ws + split * p.M * p.ws_ld, p.ws_ld);
    else
        store_tile<OUT_F32>(acc, T.m0, p.M, T.n0, p.N, p.d, p.ldd);
}

// Grouped: workgroup (expert e, n-tile) walks the expert's m-tiles.
template <int OUT_F32>
__global__ __launch_bounds__(256, 2) void grouped_kernel(GemmArgs p, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * TILE_BYTES];
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
        v4f acc[4][4];
        mainloop<0>(T, 0, p.K / 128, acc, smem, ssa, ssb);
        store_tile<OUT_F32>(acc, m0, r1, T.n0, p.N, p.d, p.ldd);
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
    const float r[4] = {s.x, s.y, s.z, s.w};
    for (int e = 0; e < 4 && n + e < N; e++) {
        if (OUT_F32)
            ((float*)d)[m * ldd + n + e] = r[e];
        else
            ((uint16_t*)d)[m * ldd + n + e] = (uint16_t)f32_to_bf16_bits(r[e]);
    }
}

int gemm_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t groups = K / 128;
    if (tiles == 0 || groups < 16 || tiles >= 256) return 1;
    int64_t s = 512 / tiles;              // aim for ~2 workgroups per CU
    const int64_t cap = groups / 8;       // at least 8 groups per split
    if (s > cap) s = cap;
    if (s > 256) s = 256;
    return s < 2 ? 1 : (int)s;
}

size_t gemm_workspace(int64_t M, int64_t N, int64_t K) {
    const int s = gemm_splits(M, N, K);
    if (s <= 1) return 0;
    return (size_t)s * (size_t)M * (size_t)((N + 3) / 4 * 4) * sizeof(float);
}

template <int KIND, int OUT_F32, bool SPLIT>
static void launch_dense(const GemmArgs& g, int64_t tiles_m, int64_t tiles_n, int64_t wgs, hipStream_t st) {
    hipLaunchKernelGGL((gemm_kernel<KIND, OUT_F32, SPLIT>), dim3((unsigned)wgs), dim3(256), 0, st, g, tiles_m,
                       tiles_n);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    if (g.splits > 1) {
        const int64_t wgs = tiles_m * tiles_n * g.splits;
        if (g.bscale_kind == 0)
            launch_dense<0, 1, true>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<1, 1, true>(g, tiles_m, tiles_n, wgs, st);
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
            launch_dense<0, 1, false>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<0, 0, false>(g, tiles_m, tiles_n, wgs, st);
    } else {
        if (g.out_f32)
            launch_dense<1, 1, false>(g, tiles_m, tiles_n, wgs, st);
        else
            launch_dense<1, 0, false>(g, tiles_m, tiles_n, wgs, st);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.G == 0 || g.N == 0) return hipSuccess;
    const int64_t tiles_n = g.N / BN;
    const dim3 grid((unsigned)(tiles_n * g.G));
    if (g.out_f32)
        hipLaunchKernelGGL(grouped_kernel<1>, grid, dim3(256), 0, st, g, tiles_n);
    else
        hipLaunchKernelGGL(grouped_kernel<0>, grid, dim3(256), 0, st, g, tiles_n);
    return hipGetLastError();
}

}  // namespace fp8bs
