// gemm.hip -- block-scaled FP8 GEMM for gfx950.
//
// D[m][n] = sum_g sa[g][m] * SB(n,g) * P_g[m][n], P_g the 128-element group
// partial.  Each group's partial is formed on the matrix cores from zero and
// promoted into an FP32 register accumulator with one FMA per output element
// (the per-group dequantisation rides on that FMA), as the pages' promotion
// every 128 elements does.
//
// Three ways of forming P_g (the `accum` argument):
//
//  ACC_F32 (0, default).  The gfx950 FP8 matrix cores do not add their
//  products at FP32 accuracy: on crafted inputs every FP8 MFMA form loses
//  about 2^-12 of the largest product inside one instruction -- the limited
//  accumulation the pages measure on their own tensor cores.  This path
//  widens each E4M3 fragment exactly to f16 right after reading it from LDS
//  (v_cvt_scalef32_pk_f16_fp8 with scale 1 is exact for every finite code)
//  and forms P_g with v_mfma_f32_32x32x16_f16, whose products are exact and
//  whose sums are FP32-accurate.  Workgroup tile 256 (m) x 128 (n); 8 waves
//  of 64x64, each 2x2 sub-tiles of 32x32, 8 MFMAs per sub-tile per group.
//
//  ACC_MFMA8 (1).  P_g straight from v_mfma_f32_16x16x128_f8f6f4 (one MFMA
//  is one K group of a 16x16 sub-tile) at twice the matrix-core rate, with
//  the matrix core's own limited accumulation inside the group.  Dense
//  launches: workgroup tile 256 (m) x 256 (n), 8 waves of 64x128 (4x8
//  sub-tiles of 16x16), the last partial round of tiles as 256 x 128 tiles
//  (waves of 64x64); split-K launches: 256 x 128; grouped launches: 128
//  columns by 64, 128, 192 or 256 rows, with loader and compute waves apart
//  (grouped_split_kernel).
//
//  ACC_MFMA8_POW2 (2).  As ACC_MFMA8, for power-of-two scales: they enter
//  the scaled MFMA as E8M0 block scales and every group is accumulated by
//  the matrix core itself, so there is no promotion step on the VALU.
//
// All: the MFMA's first operand is the B (weight) tile and its second the
// A (activation) tile, so each result sub-tile is D^T: every lane holds runs
// of four consecutive output columns of one row and needs one activation
// scale per sub-tile.  Each lane's k positions depend only on its lane
// index, identically for both operands, so whatever order the hardware
// pairs elements in, equal k meet.
//
// Staging: 512 threads (two waves per SIMD).  Each K group of both tiles
// goes global -> LDS with global_load_lds_dwordx4 (no register staging:
// lane i of a wave instruction lands at LDS base + 16*i, so each
// instruction fills 8 rows of 128 B), the group's scales with 4-byte
// global_load_lds (see dma16s, Stager).  Tiles sit in LDS as FP8 codes,
// rows of 128 B whose 16-byte chunks are XOR-swizzled by (row & 7) ^ (row>>3 & 1)
// -- lanes fetch the permuted chunk of their row, so coalescing is unchanged
// and the fragment reads of 16 consecutive rows spread over all banks.
// STAGES groups are in flight; one barrier per group both publishes the
// landed group and frees the stage the next issue overwrites.
//
// Epilogue: the tile goes through a row-major fp32 image in the freed stage
// memory and leaves in whole row segments (bf16, fp32, or -- fused -- the
// bf16 result quantised 1x128 along n, one group per tile row).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int THREADS = 512;
constexpr int WAVES = THREADS / 64;
// Waves 0..3 (one per SIMD) stage the tiles; waves 4..7 write the output.
// All eight compute.  A wave's vmcnt counts its loads and its stores
// alike, so with the roles apart the loaders' waits for the next groups
// never wait for the previous tile's output stores.
constexpr int LOADERS = 4;
constexpr int STORE_THREADS = THREADS - LOADERS * 64;

// Workgroup tile shapes, 8 waves each on a 4 (m) x 2 (n) wave grid.
//  Shape 0: 256 (m) x 128 (n), waves of 64 x 64, three K groups in flight.
//    The f16 path, split-K and the grouped kernels use it.  (A 128 x 256
//    shape for experts of about 128 rows measured no faster on the grouped
//    workloads: the 256-row tile reads each weight tile once per expert.)
//  Shape 1: 256 x 256, waves of 64 x 128, two K groups in flight.  The FP8
//    matrix-core paths of the dense GEMM use it: at the FP8 rate the
//    staging, not the matrix core, bounds the 256 x 128 tile, and the wider
//    tile stages a third fewer bytes and reads a quarter fewer from LDS per
//    FLOP.  Two stages of 66 KB fill the LDS.
template <int SH>
struct Shape;
template <>
struct Shape<0> {
    static constexpr int BM = 256, BN = 128;
    static constexpr int WM = 64, WN = 64;  // wave tile
    static constexpr int STAGES = 3;
    // Wave w runs on SIMD w % 4.  The two waves of a SIMD take one m-slot
    // from the top half of the tile and one from the bottom half, so a tile
    // with at most 128 valid rows (a typical expert) still keeps all four
    // SIMDs' matrix cores busy.
    __device__ static void wave_grid(int wave, int& wm, int& wn) {
        wm = (wave & 1) + 2 * (wave >> 2);
        wn = (wave >> 1) & 1;
    }
};
template <>
struct Shape<1> {
    static constexpr int BM = 256, BN = 256;
    static constexpr int WM = 64, WN = 128;
    static constexpr int STAGES = 2;
    __device__ static void wave_grid(int wave, int& wm, int& wn) { Shape<0>::wave_grid(wave, wm, wn); }
};
//  Shape 5: 128 x 128 with waves of 32 x 64 and two stages (66 KB, which
//    the 128 x 128 fp32 output image also fits): the K-grouped Wgrad, whose
//    experts hold one or two K groups and whose cost is the fp32 output,
//    runs two workgroups per CU with it, so one workgroup's stores overlap
//    the other's loads and MFMAs.
template <>
struct Shape<5> {
    static constexpr int BM = 128, BN = 128;
    static constexpr int WM = 32, WN = 64;
    static constexpr int STAGES = 2;
    // SIMD s holds waves s and s + 4: one m-slot, both n-slots
    __device__ static void wave_grid(int wave, int& wm, int& wn) {
        wm = wave & 3;
        wn = wave >> 2;
    }
};

//  Shape 7: 256 x 224, waves of 64 x 112 (seven 16-column fragments),
//    two stages: the per-column-scale (Wgrad) GEMMs whose 256 x 256 tiles
//    would leave part of the CUs idle for a whole round -- the expert Wgrad
//    2048 x 7168 is 224 wide tiles on 256 CUs, or 256 of these.  Only the
//    tile kind (a 112-column wave slot may straddle a 128-column weight
//    block) and the FP32-scale FP8 mode.
template <>
struct Shape<7> {
    static constexpr int BM = 256, BN = 224;
    static constexpr int WM = 64, WN = 112;
    static constexpr int STAGES = 2;
    __device__ static void wave_grid(int wave, int& wm, int& wn) { Shape<0>::wave_grid(wave, wm, wn); }
};

//  Shape 8: shape 5's tile and waves with 64-column output images: the
//    K-grouped Wgrad that keeps B resident passes its images through its
//    34 KB A ring.
template <>
struct Shape<8> {
    static constexpr int BM = 128, BN = 128;
    static constexpr int WM = 32, WN = 64;
    static constexpr int STAGES = 2;
    __device__ static void wave_grid(int wave, int& wm, int& wn) { Shape<5>::wave_grid(wave, wm, wn); }
};

//  Shapes 10 and 11: the grouped GEMMs' FP8 paths with the roles apart --
//    waves 0..3 only stage, waves 4..7 only compute, each of those owning
//    32 columns of the 128-column tile and every row of the row tile.
//    Shape 10 takes row tiles of 65..128 rows (four stages, three K groups
//    in flight), shape 11 those of 193..256 rows (three stages).
template <>
struct Shape<10> {
    static constexpr int BM = 128, BN = 128;
    static constexpr int WM = 128, WN = 32;
    static constexpr int STAGES = 4;
};
template <>
struct Shape<11> {
    static constexpr int BM = 256, BN = 128;
    static constexpr int WM = 256, WN = 32;
    static constexpr int STAGES = 3;
};
//  Shapes 12 and 13: the same for row tiles of 129..192 rows (three
//    stages) and of at most 64 rows (four stages), so a tile stages and
//    multiplies at most 63 rows past the expert's end.
template <>
struct Shape<12> {
    static constexpr int BM = 192, BN = 128;
    static constexpr int WM = 192, WN = 32;
    static constexpr int STAGES = 3;
};
template <>
struct Shape<13> {
    static constexpr int BM = 64, BN = 128;
    static constexpr int WM = 64, WN = 32;
    static constexpr int STAGES = 4;
};

// LDS map of one stage: A codes [BM][128], B codes [BN][128], sa [BM],
// B scales: per-column [BN] (tile kind) or the BN/128 block scalars.
template <int SH>
struct Lds {
    static constexpr int BM = Shape<SH>::BM, BN = Shape<SH>::BN;
    static constexpr int A = 0;
    static constexpr int B = BM * 128;
    static constexpr int SA = B + BN * 128;
    static constexpr int SB = SA + BM * 4;
    // the per-column scales are staged 64 at a time
    static constexpr int STAGE = SB + (BN + 63) / 64 * 64 * 4;
    static constexpr int BYTES = STAGE * Shape<SH>::STAGES;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct global -> LDS loads.  Issued from inline assembly so that the
// compiler does not treat the in-flight transfer as aliasing every later LDS
// read (it would otherwise wait for all outstanding transfers, including the
// prefetched groups, before the first read of the current group); the
// kernel orders them itself with wait_and_barrier.  The instructions have
// no register results.  M0 holds the wave-uniform LDS base; lane i's data
// lands at M0 + size*i.  M0 is a reserved register the compiler never
// assigns in these kernels, so it is not listed as clobbered.  The SADDR
// form is used: a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane
// byte offset, so the per-lane offsets stay fixed over the K loop and only
// the scalar base advances.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

// The same with the non-temporal hint: for operands that stream through
// once (the grouped GEMMs' expert weights), so they do not displace the
// activation rows that the other column tiles of the expert re-read from L2.
__device__ __forceinline__ void dma16s_nt(uint32_t voff, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

__device__ __forceinline__ void dma4s(uint32_t voff, const void* base, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

// Loader waves wait until at most N of their direct loads are in flight;
// then every wave meets at the barrier.  The memory clobber keeps the
// compiler from moving LDS accesses across it.  `wave` is wave-uniform.
template <int N>
__device__ __forceinline__ void wait_and_barrier(int wave) {
    if (wave < LOADERS)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
    else
        asm volatile("s_barrier" ::: "memory");
}

// Loader wave: wait until at most n (wave-uniform, 0 <= n <= N) of its
// direct loads are in flight, then the barrier.  s_waitcnt takes its count
// as an immediate, so n selects one of the N + 1 forms.
template <int N>
__device__ __forceinline__ void wait_n_and_barrier(int n) {
    if constexpr (N > 0) {
        if (n < N) {
            wait_n_and_barrier<N - 1>(n);
            return;
        }
    }
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Chunk swizzle of a tile row: (row mod 8) ^ bit 3 of the row.  The 16
// rows of a fragment read (16 lanes per LDS cycle, 256 B over the banks)
// fall 8 on even and 8 on odd bank halves, and each half sees 8 distinct
// chunk positions; rows 16 apart share the swizzle, so the fragments of a
// wave differ by constant offsets.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int f8_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

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
    float* qs;  // fused 1x128 quantisation of the output: scales qs[(n/128)*qlds + m]
    int64_t qlds;
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

// ---- staging: issue one K group of both tiles and their scales into a stage ---------------
//
// Per-lane source offsets are computed once per tile (rows past the end are
// clamped to the last row, so every load stays inside the operand); per
// group only the wave-uniform base pointers advance.  Each wave instruction
// moves 8 rows of 128 B: lane i fetches chunk (i%8) ^ swz(row) of row i/8
// and lands at LDS base + 16*i.  Only the LOADERS waves issue.

// GROUPED: the grouped kernels' form -- the weight codes are loaded with
// the non-temporal hint, and a loader issues only the A instructions whose
// 8-row block holds a row of the tile (see na_valid).
template <int SH, int KIND, bool GROUPED = false>
struct Stager {
    static constexpr int BM = Shape<SH>::BM, BN = Shape<SH>::BN;
    static constexpr int NA = BM / 8 / LOADERS, NB = BN / 8 / LOADERS;
    static constexpr int SA_INS = BM / 64, SB_INS = KIND == 1 ? (BN + 63) / 64 : 1;
    static_assert(SA_INS <= LOADERS && SB_INS <= LOADERS, "one instruction per loader for each scale");
    static_assert(KIND == 1 || BN <= 64 * 128, "block scalars of one tile fit one instruction");
    uint32_t va[NA], vb[NB], vsa, vsb;
    // GROUPED: this loader issues only the A instructions whose 8-row block
    // holds a row of the tile, na_valid of them per group (wave-uniform);
    // the compute waves' rows past the end then read stale LDS and are never
    // stored.  Otherwise every instruction is issued.
    int na_valid;

    __device__ __forceinline__ void init(const Tile& T, int wave, int lane) {
        {
            const int64_t rows = T.m_end - T.m0;
            // blocks ins * LOADERS + wave below ceil(rows / 8)
            const int64_t blocks = (rows + 7) >> 3;
            const int64_t n = blocks > wave ? (blocks - wave + LOADERS - 1) / LOADERS : 0;
            na_valid = GROUPED ? (int)(n < NA ? n : NA) : NA;
        }
#pragma unroll
        for (int ins = 0; ins < NA; ins++) {
            const int row = (ins * LOADERS + wave) * 8 + (lane >> 3);
            const int64_t m = T.m0 + row < T.m_end ? T.m0 + row : T.m_end - 1;
            va[ins] = (uint32_t)((m - T.m0) * T.lda) + ((((lane & 7) ^ swz(row))) << 4);
        }
#pragma unroll
        for (int ins = 0; ins < NB; ins++) {
            const int row = (ins * LOADERS + wave) * 8 + (lane >> 3);
            const int64_t n = T.n0 + row < T.n_end ? T.n0 + row : T.n_end - 1;
            vb[ins] = (uint32_t)((n - T.n0) * T.ldb) + ((((lane & 7) ^ swz(row))) << 4);
        }
        const int64_t m = T.m0 + wave * 64 + lane < T.m_end ? T.m0 + wave * 64 + lane : T.m_end - 1;
        vsa = (uint32_t)(m - T.m0) * 4;
        if (KIND == 1) {
            const int64_t n = T.n0 + wave * 64 + lane < T.n_end ? T.n0 + wave * 64 + lane : T.n_end - 1;
            vsb = (uint32_t)(n - T.n0) * 4;
        } else {
            // lane l loads the scalar of the tile's block column l (clamped
            // to the last block column present)
            const int64_t last = (T.n_end - 1 - T.n0) >> 7;
            const int64_t blk = lane < last ? lane : last;
            vsb = (uint32_t)(blk * T.sb_s0 * 4);
        }
    }

    // Group g into the stage at LDS byte offset `stage` of smem.
    __device__ __forceinline__ void issue(const Tile& T, int64_t g, uint8_t* smem, int stage, int wave) const {
        if (wave >= LOADERS) return;
        const uint8_t* a = T.a + T.m0 * T.lda + g * 128;
        const uint8_t* b = T.b + T.n0 * T.ldb + g * 128;
        const uint32_t base = lds_addr(smem + stage);
#pragma unroll
        for (int ins = 0; ins < NA; ins++)
            if (!GROUPED || ins < na_valid) dma16s(va[ins], a, base + Lds<SH>::A + (ins * LOADERS + wave) * 8 * 128);
#pragma unroll
        for (int ins = 0; ins < NB; ins++) {
            if (GROUPED)
                dma16s_nt(vb[ins], b, base + Lds<SH>::B + (ins * LOADERS + wave) * 8 * 128);
            else
                dma16s(vb[ins], b, base + Lds<SH>::B + (ins * LOADERS + wave) * 8 * 128);
        }
        // scales: loader w loads sa rows 64w..64w+63 and the B scales --
        // per-column floats 64w..64w+63 (tile kind) or, block kind (loader
        // 0), the group's BN/128 block scalars (lane l loads block column
        // l; the copies past them land in unused words)
        if (wave < SA_INS) dma4s(vsa, T.sa + g * T.ldsa + T.m0, base + Lds<SH>::SA + wave * 256);
        if (KIND == 1 && wave < SB_INS)
            dma4s(vsb, T.sb + g * T.sb_s0 + T.n0, base + Lds<SH>::SB + wave * 256);
        else if (KIND == 0 && wave == 0)
            dma4s(vsb, T.sb + (T.n0 >> 7) * T.sb_s0 + g * T.sb_s1, base + Lds<SH>::SB);
    }
};

// ==== ACC_F32 path: exact f16 widening, f16 matrix cores =============================
//
// v_mfma_f32_32x32x16_f16: lane l feeds row l%32 of its operand with 8
// values per k-step.  Lane l reads the 16-byte chunk c = 2q + l/32 of its
// row (q = 0..3) and widens it to 16 f16: the first 8 feed k-step 2q, the
// last 8 k-step 2q+1.  lds16 reads a chunk of a swizzled tile row; widen16
// converts its 16 codes exactly (v_cvt_scalef32_pk_f16_fp8, scale 1).

__device__ __forceinline__ uint4 lds16(const uint8_t* tile, int row, int chunk) {
    return *(const uint4*)(tile + f8_off(row, chunk));
}

__device__ __forceinline__ void widen16(const uint4 v, v8h& lo, v8h& hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    v2h h[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        h[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
        h[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo[2 * i] = h[i][0];
        lo[2 * i + 1] = h[i][1];
        hi[2 * i] = h[4 + i][0];
        hi[2 * i + 1] = h[4 + i][1];
    }
}

// Per-column (tile-kind) B scales, as Wgrad uses: acc += (P_g * sa[m]) *
// sb[n], the partials promoted at the end of the group.  The fragments of
// k-chunk q+1 are read from LDS while chunk q is widened and multiplied.
// acc[i][j]: 32x32 sub-tile (m-sub i, n-sub j) of this wave, D^T layout:
// register r of lane l is n = 32j + 8(r/4) + 4(l/32) + r%4, m = 32i + l%32.
template <int SH>
__device__ __forceinline__ void compute_f32_tile(const uint8_t* stage, int wm, int wn, int lane, int m_valid,
                                                 v16f (&acc)[2][2]) {
    const uint8_t* la = stage + Lds<SH>::A;
    const uint8_t* lb = stage + Lds<SH>::B;
    const float* lsa = (const float*)(stage + Lds<SH>::SA);
    const float* lsb = (const float*)(stage + Lds<SH>::SB);
    const int mbase = wm * 64, nbase = wn * 64;
    const int r = lane & 31, h = lane >> 5;
    if (mbase >= m_valid) return;  // this wave's rows are all past the end

    uint4 ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) ra[i] = lds16(la, mbase + 32 * i + r, h);
#pragma unroll
    for (int j = 0; j < 2; j++) rb[j] = lds16(lb, nbase + 32 * j + r, h);
    v16f p[2][2];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint4 na[2], nb[2];
        if (q < 3) {
#pragma unroll
            for (int i = 0; i < 2; i++) na[i] = lds16(la, mbase + 32 * i + r, 2 * (q + 1) + h);
#pragma unroll
            for (int j = 0; j < 2; j++) nb[j] = lds16(lb, nbase + 32 * j + r, 2 * (q + 1) + h);
        }
        v8h a0[2], a1[2], b0[2], b1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) widen16(ra[i], a0[i], a1[i]);
#pragma unroll
        for (int j = 0; j < 2; j++) widen16(rb[j], b0[j], b1[j]);
        const v16f zero = {};
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0[j], a0[i], q == 0 ? zero : p[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1[j], a1[i], p[i][j], 0, 0, 0);
        if (q < 3) {
#pragma unroll
            for (int i = 0; i < 2; i++) ra[i] = na[i];
#pragma unroll
            for (int j = 0; j < 2; j++) rb[j] = nb[j];
        }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const float sam = lsa[mbase + 32 * i + r];
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const v4f sbn = *(const v4f*)(lsb + nbase + 32 * j + 8 * q + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; e++) acc[i][j][4 * q + e] += (p[i][j][4 * q + e] * sam) * sbn[e];
            }
    }
}

// Block-scale kind (Fprop, Dgrad, grouped), software-pipelined: the
// fragments of k-chunk q+1 are read from LDS while chunk q is widened and
// multiplied, and the partials of the previous group are promoted at the
// start of this group, each sub-tile's promotion just before the first MFMA
// that reuses its registers, so the promotion FMAs run beside this group's
// MFMAs.  p and cp carry the previous group's partials and scale factors
// (zero before the first group).
template <int SH>
__device__ __forceinline__ void compute_f32_block(const uint8_t* stage, int wm, int wn, int lane,
                                                  v16f (&acc)[2][2], v16f (&p)[2][2], float (&cp)[2]) {
    const uint8_t* la = stage + Lds<SH>::A;
    const uint8_t* lb = stage + Lds<SH>::B;
    const float* lsa = (const float*)(stage + Lds<SH>::SA);
    const float* lsb = (const float*)(stage + Lds<SH>::SB);
    const int mbase = wm * 64, nbase = wn * 64;
    const int r = lane & 31, h = lane >> 5;

    uint4 ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) ra[i] = lds16(la, mbase + 32 * i + r, h);
#pragma unroll
    for (int j = 0; j < 2; j++) rb[j] = lds16(lb, nbase + 32 * j + r, h);
    const float sbk = lsb[nbase >> 7];
    float cn[2];
#pragma unroll
    for (int i = 0; i < 2; i++) cn[i] = lsa[mbase + 32 * i + r] * sbk;

#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint4 na[2], nb[2];
        if (q < 3) {
#pragma unroll
            for (int i = 0; i < 2; i++) na[i] = lds16(la, mbase + 32 * i + r, 2 * (q + 1) + h);
#pragma unroll
            for (int j = 0; j < 2; j++) nb[j] = lds16(lb, nbase + 32 * j + r, 2 * (q + 1) + h);
        }
        v8h a0[2], a1[2], b0[2], b1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) widen16(ra[i], a0[i], a1[i]);
#pragma unroll
        for (int j = 0; j < 2; j++) widen16(rb[j], b0[j], b1[j]);
        if (q == 0) {
            const v16f zero = {};
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    acc[i][j] += p[i][j] * cp[i];
                    p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0[j], a0[i], zero, 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0[j], a0[i], p[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1[j], a1[i], p[i][j], 0, 0, 0);
        if (q < 3) {
#pragma unroll
            for (int i = 0; i < 2; i++) ra[i] = na[i];
#pragma unroll
            for (int j = 0; j < 2; j++) rb[j] = nb[j];
        }
    }
    cp[0] = cn[0];
    cp[1] = cn[1];
}

// LDS addresses of one K group's operands (within one stage, or in
// separate regions where a kernel keeps an operand resident).
struct StagePtrs {
    const uint8_t* a;  // A codes [BM][128], rows swizzled as f8_off
    const uint8_t* b;  // B codes [BN][128]
    const float* sa;   // A row scales [BM]
    const float* sb;   // B scales: per column [BN] (tile kind) or the block scalars
};

template <int SH>
__device__ __forceinline__ StagePtrs stage_ptrs(const uint8_t* stage) {
    return StagePtrs{stage + Lds<SH>::A, stage + Lds<SH>::B, (const float*)(stage + Lds<SH>::SA),
                     (const float*)(stage + Lds<SH>::SB)};
}

// ==== ACC_MFMA8 path: FP8 matrix cores, one MFMA per K group =============================
//
// Lane l feeds bytes [32(l/16), 32(l/16)+32) of its row: chunks 2(l/16) and
// 2(l/16)+1.

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

// Sub-tiles of one wave: MI (m) x NJ (n) of 16 x 16.
template <int SH>
struct Sub {
    static constexpr int MI = Shape<SH>::WM / 16, NJ = Shape<SH>::WN / 16;
};

// The two waves of a SIMD (w and w + 4) leave each barrier together and
// would run their MFMA blocks and their promotion FMAs in step; the second
// one starts the group's MFMA work about 64 cycles later, so that its MFMAs
// overlap the first one's FMAs.  On the dense Fprop with FP32 scales: 2-3%
// faster on average over six paired runs (run-to-run spread is about 2%).
// The per-column (Wgrad) loop, which issues a fragment's MFMAs before their
// promotion, uses it too: with it that loop ran 4-6% faster on the expert
// Wgrad in three paired runs.
__device__ __forceinline__ void offset_second_wave() {
    if (threadIdx.x >= THREADS / 2) __builtin_amdgcn_s_sleep(1);
}

// acc[i][j]: 16x16 sub-tile (m-sub i, n-sub j), D^T layout: register e of
// lane l is n = 16j + 4(l/16) + e, m = 16i + l%16.  The fragments of the
// wave's shorter side stay in registers while those of the longer side
// stream past them.  A wave's WN <= 128 columns lie in one 128-column block.
template <int SH, int KIND>
__device__ __forceinline__ void compute_mfma8(const StagePtrs& sp, int wm, int wn, int lane, int m_valid,
                                              v4f (&acc)[Sub<SH>::MI][Sub<SH>::NJ]) {
    constexpr int MI = Sub<SH>::MI, NJ = Sub<SH>::NJ;
    const uint8_t* la = sp.a;
    const uint8_t* lb = sp.b;
    const float* lsa = sp.sa;
    const float* lsb = sp.sb;
    const int mbase = wm * Shape<SH>::WM, nbase = wn * Shape<SH>::WN;
    const int c0 = 2 * (lane >> 4);
    if (mbase >= m_valid) return;
    const float sbk = KIND == 0 ? lsb[nbase >> 7] : 0.f;

    if constexpr (MI < NJ) {
        // A resident: rows past m_valid are read (stale LDS) but never stored
        v8i af[MI];
        float c[MI];
#pragma unroll
        for (int i = 0; i < MI; i++) {
            const int mrow = mbase + 16 * i + (lane & 15);
            af[i] = f8_frag(la, mrow, c0);
            c[i] = KIND == 0 ? lsa[mrow] * sbk : lsa[mrow];
        }
        if constexpr (KIND == 0) {
            offset_second_wave();
            // two B fragments per step: eight MFMAs are in flight before
            // their partials are promoted (7% faster than one; the tile
            // kind's extra scale registers do not leave room for it)
#pragma unroll
            for (int j = 0; j < NJ; j += 2) {
                const v8i b0 = f8_frag(lb, nbase + 16 * j + (lane & 15), c0);
                const v8i b1 = f8_frag(lb, nbase + 16 * (j + 1) + (lane & 15), c0);
                v4f p0[MI], p1[MI];
#pragma unroll
                for (int i = 0; i < MI; i++) p0[i] = mfma8_group(b0, af[i]);
#pragma unroll
                for (int i = 0; i < MI; i++) p1[i] = mfma8_group(b1, af[i]);
#pragma unroll
                for (int i = 0; i < MI; i++) {
                    acc[i][j] += p0[i] * c[i];
                    acc[i][j + 1] += p1[i] * c[i];
                }
            }
        } else {
            // per-column scales: the MI MFMAs of a fragment first, then their
            // promotion (two multiplies per output), so one wave's VALU phase
            // can run beside the other wave's MFMA phase on the SIMD
            offset_second_wave();
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const v8i bf = f8_frag(lb, nbase + 16 * j + (lane & 15), c0);
                const v4f sbn = *(const v4f*)(lsb + nbase + 16 * j + 4 * (lane >> 4));
                v4f p[MI];
#pragma unroll
                for (int i = 0; i < MI; i++) p[i] = mfma8_group(bf, af[i]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < MI; i++) acc[i][j] += (p[i] * c[i]) * sbn;
            }
        }
    } else {
        v8i bf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) bf[j] = f8_frag(lb, nbase + 16 * j + (lane & 15), c0);
        v4f sbn[NJ];
        if (KIND == 1) {
#pragma unroll
            for (int j = 0; j < NJ; j++) sbn[j] = *(const v4f*)(lsb + nbase + 16 * j + 4 * (lane >> 4));
        }
#pragma unroll
        for (int i = 0; i < MI; i++) {
            if (mbase + 16 * i >= m_valid) break;  // wave-uniform
            const int mrow = mbase + 16 * i + (lane & 15);
            const v8i af = f8_frag(la, mrow, c0);
            const float sam = lsa[mrow];
            const float c = KIND == 0 ? sam * sbk : sam;
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const v4f p = mfma8_group(bf[j], af);
                if (KIND == 0)
                    acc[i][j] += p * c;
                else
                    acc[i][j] += (p * c) * sbn[j];
            }
        }
    }
}

// ==== ACC_MFMA8_POW2 path: power-of-two scales inside the FP8 matrix cores ====================
//
// With every scale a power of two, 2^k is the E8M0 byte k + 127 -- the
// exponent field of the fp32 scale.  The scaled MFMA multiplies lane l's
// 32-element K block of its row by 2^(byte - 127) for each operand, so the
// whole dequantised group dec(a)*sa * dec(b)*SB is summed by the matrix
// core straight into the fp32 accumulator: no promotion on the VALU.  The
// scale bytes are per (row, K block); a 128-element group's four blocks of a
// row share its 1x128 or 128x128 scale.
__device__ __forceinline__ int e8m0(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

template <int SH, int KIND>
__device__ __forceinline__ void compute_mfma8_pow2(const StagePtrs& sp, int wm, int wn, int lane, int m_valid,
                                                   v4f (&acc)[Sub<SH>::MI][Sub<SH>::NJ]) {
    constexpr int MI = Sub<SH>::MI, NJ = Sub<SH>::NJ;
    const uint8_t* la = sp.a;
    const uint8_t* lb = sp.b;
    const float* lsa = sp.sa;
    const float* lsb = sp.sb;
    const int mbase = wm * Shape<SH>::WM, nbase = wn * Shape<SH>::WN;
    const int c0 = 2 * (lane >> 4);
    if (mbase >= m_valid) return;

    if constexpr (MI < NJ) {
        v8i af[MI];
        int sab[MI];
#pragma unroll
        for (int i = 0; i < MI; i++) {
            const int mrow = mbase + 16 * i + (lane & 15);
            af[i] = f8_frag(la, mrow, c0);
            sab[i] = e8m0(lsa[mrow]);
        }
        if constexpr (KIND == 0) {
            // Block kind: the next step's B pair is read from LDS while this
            // pair multiplies, and the one block scale is read once.
            const int col = nbase + (lane & 15);
            const int sbk = e8m0(lsb[nbase >> 7]);
            v8i b0 = f8_frag(lb, col, c0);
            v8i b1 = f8_frag(lb, col + 16, c0);
#pragma unroll
            for (int j = 0; j < NJ; j += 2) {
                v8i nb0, nb1;
                if (j + 2 < NJ) {
                    nb0 = f8_frag(lb, col + 16 * (j + 2), c0);
                    nb1 = f8_frag(lb, col + 16 * (j + 3), c0);
                    // keep the reads ahead of this pair's MFMAs (the scheduler
                    // would otherwise sink them into the registers the MFMAs free)
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < MI; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, af[i], acc[i][j], 0, 0, 0, sbk, 0,
                                                                             sab[i]);
#pragma unroll
                for (int i = 0; i < MI; i++)
                    acc[i][j + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, af[i], acc[i][j + 1], 0, 0, 0,
                                                                                     sbk, 0, sab[i]);
                if (j + 2 < NJ) {
                    b0 = nb0;
                    b1 = nb1;
                }
            }
        } else {
            // per-column scales: one read per fragment (the registers for a
            // prefetched pair and its scales are not free here)
#pragma unroll
            for (int j = 0; j < NJ; j += 2) {
                const v8i b0 = f8_frag(lb, nbase + 16 * j + (lane & 15), c0);
                const v8i b1 = f8_frag(lb, nbase + 16 * (j + 1) + (lane & 15), c0);
                const int s0 = e8m0(lsb[nbase + 16 * j + (lane & 15)]);
                const int s1 = e8m0(lsb[nbase + 16 * (j + 1) + (lane & 15)]);
#pragma unroll
                for (int i = 0; i < MI; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, af[i], acc[i][j], 0, 0, 0, s0, 0,
                                                                             sab[i]);
#pragma unroll
                for (int i = 0; i < MI; i++)
                    acc[i][j + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, af[i], acc[i][j + 1], 0, 0, 0,
                                                                                     s1, 0, sab[i]);
            }
        }
        return;
    }
    v8i bf[NJ];
    int sbb[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        bf[j] = f8_frag(lb, nbase + 16 * j + (lane & 15), c0);
        sbb[j] = e8m0(KIND == 0 ? lsb[nbase >> 7] : lsb[nbase + 16 * j + (lane & 15)]);
    }
#pragma unroll
    for (int i = 0; i < MI; i++) {
        if (mbase + 16 * i >= m_valid) break;  // wave-uniform
        const int mrow = mbase + 16 * i + (lane & 15);
        const v8i af = f8_frag(la, mrow, c0);
        const int sab = e8m0(lsa[mrow]);
#pragma unroll
        for (int j = 0; j < NJ; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, sbb[j], 0, sab);
    }
}

// ==== epilogue ===========================================================================

// Store four consecutive columns n..n+3 of row m (masked at the edges).
// Four consecutive columns n..n+3 of row m, all inside the output.
template <int OUT>
__device__ __forceinline__ void store4_full(void* d, int64_t ldd, int64_t m, int64_t n, float v0, float v1,
                                            float v2, float v3) {
    if (OUT) {
        *(float4*)((float*)d + m * ldd + n) = make_float4(v0, v1, v2, v3);
    } else {
        const uint32_t b0 = f32_to_bf16_bits(v0), b1 = f32_to_bf16_bits(v1);
        const uint32_t b2 = f32_to_bf16_bits(v2), b3 = f32_to_bf16_bits(v3);
        *(uint2*)((uint16_t*)d + m * ldd + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
}

template <int OUT>
__device__ __forceinline__ void store4(void* d, int64_t ldd, int64_t m, int64_t n, int64_t n_end, float v0,
                                       float v1, float v2, float v3) {
    if (OUT) {
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

// The tile leaves through LDS, 128 columns at a time: the waves holding
// those columns write their accumulators into a row-major fp32 image (row
// stride 128 + 4 floats, which spreads consecutive rows over the banks), then
// each row of the image is stored with 32 lanes writing 16 contiguous bytes
// each (fp32) or 8 (bf16).  Written
// straight from the MFMA layout, a store instruction would touch 32 rows with
// 32 bytes each; through LDS it writes whole 512- or 256-byte row segments,
// which matters where the output is large next to the work (fp32 gradients
// summed over few tokens).  The stages are free: every wave has left the K
// loop (wait_and_barrier<0>) before this runs.
template <int SH>
struct Epi {
    static constexpr int W = SH == 7 ? 112 : SH == 8 ? 64 : 128;  // columns per image
    static constexpr int LD = W + 4;
    static_assert(Shape<SH>::BM * LD * 4 <= Lds<SH>::BYTES, "the image fits in the stages");
    static_assert(Shape<SH>::BN % W == 0 && W % Shape<SH>::WN == 0, "waves' columns tile the images");
};

template <int SH>
__device__ __forceinline__ void put4(float* ep, int row, int col, float v0, float v1, float v2, float v3) {
    *(float4*)&ep[row * Epi<SH>::LD + col] = make_float4(v0, v1, v2, v3);
}

// OUT: 0 bf16, 1 fp32, 2 / 3 the bf16 result quantised in 1x128 groups
// along n with FP32 / power-of-two scales (the image's 128 columns, starting
// at output column n0, are one group of every row), codes to d, scales to
// T.qs.
// ALL: every wave stores (kernels that run one tile per workgroup); else
// the loader waves do not, so that their vmcnt waits for a following
// tile's groups never count this tile's stores.
template <int SH, int OUT, bool ALL = false>
__device__ __forceinline__ void write_tile_image(const float* ep, const Tile& T, int64_t n0, void* d,
                                                 int64_t ldd) {
    constexpr int BM = Shape<SH>::BM, W = Epi<SH>::W;
    constexpr int LPR = W / 4;                                  // lanes per row
    constexpr int RPI = (ALL ? THREADS : STORE_THREADS) / LPR;  // rows per pass
    const int t = (int)threadIdx.x - (ALL ? 0 : LOADERS * 64);
    // (with 112-column images, the threads past a whole number of rows
    // stay idle too)
    if (t < 0 || t >= RPI * LPR) return;
    const int col = (t % LPR) * 4;
    const int64_t n = n0 + col;
    if constexpr (OUT <= 1) {
        // Images whose columns all lie inside the output store whole
        // 16- / 8-byte runs with no per-lane edge test (kept apart so the
        // compiler does not fold the edge path's element stores into them).
        if (n0 + W <= T.n_end) {
#pragma unroll 4
            for (int r = t / LPR; r < BM; r += RPI) {
                const int64_t m = T.m0 + r;
                if (m >= T.m_end) break;
                const float4 v = *(const float4*)&ep[r * Epi<SH>::LD + col];
                store4_full<OUT>(d, ldd, m, n, v.x, v.y, v.z, v.w);
            }
        } else {
            for (int r = t / LPR; r < BM; r += RPI) {
                const int64_t m = T.m0 + r;
                if (m >= T.m_end || n >= T.n_end) continue;
                const float4 v = *(const float4*)&ep[r * Epi<SH>::LD + col];
                store4<OUT>(d, ldd, m, n, T.n_end, v.x, v.y, v.z, v.w);
            }
        }
    } else {
        static_assert(W == 128 && LPR == 32, "one 1x128 group per image row, 32 lanes per row");
        // Every lane runs every pass (the 32-lane reductions need them all);
        // only the stores are masked.
        for (int r = t / LPR; r < BM; r += RPI) {
            const int64_t m = T.m0 + r;
            const float4 v = *(const float4*)&ep[r * Epi<SH>::LD + col];
            const uint32_t b0 = f32_to_bf16_bits(v.x), b1 = f32_to_bf16_bits(v.y);
            const uint32_t b2 = f32_to_bf16_bits(v.z), b3 = f32_to_bf16_bits(v.w);
            uint32_t am = max(max(b0 & 0x7FFFu, b1 & 0x7FFFu), max(b2 & 0x7FFFu, b3 & 0x7FFFu)) << 16;
            am = row16_max(am);
            am = max(am, (uint32_t)__shfl_xor((int)am, 16));
            const GroupScale gs = group_scale(am, OUT == 3);
            const uint32_t codes = pack4(bf16_lo(b0) * gs.inv, bf16_lo(b1) * gs.inv, bf16_lo(b2) * gs.inv,
                                         bf16_lo(b3) * gs.inv);
            if (m < T.m_end && n < T.n_end) {
                *(uint32_t*)((uint8_t*)d + m * ldd + n) = codes;
                if (col == 0) T.qs[(n0 >> 7) * T.qlds + m] = gs.s;
            }
        }
    }
}

template <int SH, int OUT, bool ALL = false>
__device__ __forceinline__ void store_f32(const v16f (&acc)[2][2], const Tile& T, int wm, int wn, int lane,
                                          void* d, int64_t ldd, uint8_t* smem) {
    float* ep = (float*)smem;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 4; q++)
                put4<SH>(ep, wm * 64 + 32 * i + (lane & 31), wn * 64 + 32 * j + 8 * q + 4 * (lane >> 5),
                         acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    static_assert(Shape<SH>::BN == Epi<SH>::W, "one image");
    __syncthreads();
    write_tile_image<SH, OUT, ALL>(ep, T, T.n0, d, ldd);
    __syncthreads();  // the stages may be refilled by a following tile
}

template <int SH, int OUT, bool ALL = false>
__device__ __forceinline__ void store_mfma8(const v4f (&acc)[Sub<SH>::MI][Sub<SH>::NJ], const Tile& T, int wm,
                                            int wn, int lane, void* d, int64_t ldd, uint8_t* smem) {
    constexpr int W = Epi<SH>::W, WM = Shape<SH>::WM, WN = Shape<SH>::WN;
    float* ep = (float*)smem;
#pragma unroll
    for (int h = 0; h < Shape<SH>::BN / W; h++) {
        if (T.n0 + h * W >= T.n_end) break;  // workgroup-uniform: columns past the end
        if (wn * WN / W == h) {
#pragma unroll
            for (int i = 0; i < Sub<SH>::MI; i++)
#pragma unroll
                for (int j = 0; j < Sub<SH>::NJ; j++)
                    put4<SH>(ep, wm * WM + 16 * i + (lane & 15), wn * WN % W + 16 * j + 4 * (lane >> 4),
                             acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
        __syncthreads();
        write_tile_image<SH, OUT, ALL>(ep, T, T.n0 + h * W, d, ldd);
        __syncthreads();
    }
}

// ==== one tile: pipelined K loop, then the store ==============================================

// ALL_STORE: every wave writes the output (a kernel that runs one tile per
// workgroup; see write_tile_image).
template <int ACC, int SH, int KIND, int OUT, bool ALL_STORE = false>
__device__ __forceinline__ void run_tile(const Tile& T, int64_t g0, int64_t g1, void* d, int64_t ldd,
                                         uint8_t* smem) {
    constexpr int S = Shape<SH>::STAGES;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    int wm, wn;
    Shape<SH>::wave_grid(wave, wm, wn);
    const int m_valid = (int)(T.m_end - T.m0 < Shape<SH>::BM ? T.m_end - T.m0 : Shape<SH>::BM);

    static_assert(ACC != 0 || SH == 0, "the f16 path runs on 64 x 64 wave tiles");
    constexpr int MI = Sub<SH>::MI, NJ = Sub<SH>::NJ;
    // ACC 0: 32x32 sub-tiles; ACC 1, 2: 16x16 sub-tiles
    typedef typename std::conditional<ACC == 0, v16f[2][2], v4f[MI][NJ]>::type AccT;
    AccT acc;
    if constexpr (ACC == 0) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < NJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // pipelined block-kind f16 path: previous group's partials and factors
    v16f pp[2][2];
    float cp[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) pp[i][j][r] = 0.f;

    Stager<SH, KIND> stg;
    stg.init(T, wave, lane);
    // prologue: groups g0 .. g0+S-2
#pragma unroll
    for (int s = 0; s < S - 1; s++)
        if (g0 + s < g1) stg.issue(T, g0 + s, smem, s * Lds<SH>::STAGE, wave);

    // Tile loads per group per loader wave; the scale loads come on top, so
    // waiting for k * PER outstanding (k groups issued after this one) is
    // conservative.  With two stages the following group is issued only
    // after the wait.
    constexpr int PER = (Shape<SH>::BM + Shape<SH>::BN) / 8 / LOADERS;
    static_assert((S == 4 && PER == 8) || (S == 3 && PER == 12) || S == 2, "wait counts cover this pipeline");
    // One group: wait until it has landed (at most the S - 2 following
    // groups still in flight) for every wave and every wave is done with the stage
    // of the previous group, refill that stage, compute.  The stage index SS
    // is a compile-time constant, so LDS addresses fold into immediates.
    auto step = [&](auto ss, int64_t g) {
        constexpr int SS = decltype(ss)::value;
        if (S == 4 && g + 2 < g1)
            wait_and_barrier<2 * PER>(wave);
        else if (S >= 3 && g + 1 < g1)
            wait_and_barrier<PER>(wave);
        else
            wait_and_barrier<0>(wave);
        if (g + S - 1 < g1) stg.issue(T, g + S - 1, smem, ((SS + S - 1) % S) * Lds<SH>::STAGE, wave);
        const uint8_t* stage = smem + SS * Lds<SH>::STAGE;
        if constexpr (ACC == 0 && KIND == 0) {
            if (wm * 64 < m_valid) compute_f32_block<SH>(stage, wm, wn, lane, acc, pp, cp);
        } else if constexpr (ACC == 0) {
            compute_f32_tile<SH>(stage, wm, wn, lane, m_valid, acc);
        } else {
            if constexpr (ACC == 1)
                compute_mfma8<SH, KIND>(stage_ptrs<SH>(stage), wm, wn, lane, m_valid, acc);
            else
                compute_mfma8_pow2<SH, KIND>(stage_ptrs<SH>(stage), wm, wn, lane, m_valid, acc);
        }
    };
    for (int64_t g = g0; g < g1; g += S) {
        step(std::integral_constant<int, 0>(), g);
        if (g + 1 < g1) step(std::integral_constant<int, 1>(), g + 1);
        if constexpr (S >= 3)
            if (g + 2 < g1) step(std::integral_constant<int, 2>(), g + 2);
        if constexpr (S == 4)
            if (g + 3 < g1) step(std::integral_constant<int, 3>(), g + 3);
    }
    if constexpr (ACC == 0 && KIND == 0) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) acc[i][j] += pp[i][j] * cp[i];
    }
    wait_and_barrier<0>(wave);  // the LDS stages may be reused by a following tile

    if constexpr (ACC == 0)
        store_f32<SH, OUT, ALL_STORE>(acc, T, wm, wn, lane, d, ldd, smem);
    else
        store_mfma8<SH, OUT, ALL_STORE>(acc, T, wm, wn, lane, d, ldd, smem);
}

// ==== kernels ==========================================================================

template <int ACC, int SH, int KIND, int OUT, bool SPLIT>
__global__ __launch_bounds__(THREADS) void gemm_kernel(GemmArgs p, int64_t tiles_m, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Lds<SH>::BYTES];
    const int64_t ntiles = tiles_m * tiles_n;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t split = SPLIT ? wid / ntiles : 0;
    int64_t tm, tn;
    tile_coords(wid % ntiles, tiles_m, tiles_n, tm, tn);

    Tile T;
    T.m0 = tm * Shape<SH>::BM;
    T.m_end = p.M;
    T.n0 = tn * Shape<SH>::BN;
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
    T.qs = p.qs;
    T.qlds = p.qlds;

    const int64_t groups = p.K / 128;
    if (SPLIT) {
        const int64_t per = (groups + p.splits - 1) / p.splits;
        const int64_t g0 = split * per;
        const int64_t g1 = g0 + per < groups ? g0 + per : groups;
        run_tile<ACC, SH, KIND, 1, true>(T, g0, g1, p.ws + split * p.M * p.ws_ld, p.ws_ld, smem);
    } else {
        run_tile<ACC, SH, KIND, OUT, true>(T, 0, groups, p.d, p.ldd, smem);
    }
}

// FP8 dense paths: one launch, two tile shapes.  Output columns [0, n1)
// (n1 a multiple of 256, possibly past N) run on 256 x 256 tiles
// (workgroups 0 .. wide-1), the rest on 256 x 128
// tiles (the following workgroups): a last, partial round of wide tiles
// becomes a full round of narrow ones.  Each region is XCD-remapped on its
// own, so both spread over all XCDs in dispatch order.
template <int ACC, int KIND, int OUT>
__global__ __launch_bounds__(THREADS) void gemm_wide_kernel(GemmArgs p, int64_t n1) {
    constexpr int LDS_BYTES = Lds<0>::BYTES > Lds<1>::BYTES ? Lds<0>::BYTES : Lds<1>::BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
    static_assert(Shape<0>::BM == Shape<1>::BM, "both regions share the m tiling");
    const int64_t tiles_m = (p.M + Shape<1>::BM - 1) / Shape<1>::BM;
    const int64_t wide = tiles_m * (n1 / Shape<1>::BN);
    Tile T;
    T.m_end = p.M;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b;
    T.ldb = p.ldb;
    T.sb = p.sb;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = p.sb_s1;
    T.qs = p.qs;
    T.qlds = p.qlds;
    const int64_t groups = p.K / 128;
    int64_t tm, tn;
    if ((int64_t)blockIdx.x < wide) {
        tile_coords(xcd_remap(blockIdx.x, wide), tiles_m, n1 / Shape<1>::BN, tm, tn);
        T.m0 = tm * Shape<1>::BM;
        T.n0 = tn * Shape<1>::BN;
        T.n_end = n1 < p.N ? n1 : p.N;
        run_tile<ACC, 1, KIND, OUT, true>(T, 0, groups, p.d, p.ldd, smem);
    } else {
        // only launched when n1 < N
        const int64_t tiles_n = (p.N - n1 + Shape<0>::BN - 1) / Shape<0>::BN;
        tile_coords(xcd_remap(blockIdx.x - wide, gridDim.x - wide), tiles_m, tiles_n, tm, tn);
        T.m0 = tm * Shape<0>::BM;
        T.n0 = n1 + tn * Shape<0>::BN;
        T.n_end = p.N;
        run_tile<ACC, 0, KIND, OUT, true>(T, 0, groups, p.d, p.ldd, smem);
    }
}

// Grouped, exact mode: workgroup (expert e, n-tile) walks the expert's
// m-tiles.  (The FP8 modes run grouped_split_kernel below.)
template <int ACC, int KIND, int OUT>
__global__ __launch_bounds__(THREADS) void grouped_kernel(GemmArgs p, int64_t tiles_n) {
    static_assert(ACC == 0, "the exact mode");
    __shared__ __attribute__((aligned(16))) uint8_t smem[Lds<0>::BYTES];
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t e = wid / tiles_n;
    const int64_t tn = wid % tiles_n;
    const int64_t r0 = p.offsets[e], r1 = p.offsets[e + 1];

    Tile T;
    T.m_end = r1;
    T.n0 = tn * Shape<0>::BN;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b + e * p.b_estride;
    T.ldb = p.ldb;
    T.sb = p.sb + e * p.sb_estride;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = p.sb_s1;
    for (int64_t m0 = r0; m0 < r1; m0 += Shape<0>::BM) {
        T.m0 = m0;
        run_tile<ACC, 0, KIND, OUT>(T, 0, p.K / 128, p.d, p.ldd, smem);
    }
}

// ==== grouped GEMMs with the roles apart ===================================================
//
// The FP8 paths of the grouped GEMMs stream every weight tile once and are
// bound by that staging, not by the matrix cores.  Waves 0..3 only issue
// the direct loads (the weight codes with the non-temporal hint) and waves
// 4..7 only compute, so a loader's issue of the next groups never waits
// behind its own MFMA and promotion work.  Compute wave c (on SIMD c) owns
// columns 32c..32c+31: its two B fragments stay in registers while the A
// fragments of the tile's 16-row blocks stream past them.  A row tile is
// the smallest of 64, 128, 192 or 256 rows that holds the expert's
// remaining rows, so an expert with few rows stages and multiplies few.

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
typedef __attribute__((address_space(3))) const float lds_f32;

// The fragment of rows 16i + lane % 16 from per-lane LDS byte addresses of
// the two chunks in row lane % 16 (rows 16 apart share the swizzle, so row
// block i is at +2048 i, an immediate offset).
__device__ __forceinline__ v8i f8_frag_at(uint32_t lo, uint32_t hi, int i) {
    const u32x4_t x = *(lds_u4*)(uintptr_t)(lo + 2048 * i);
    const u32x4_t y = *(lds_u4*)(uintptr_t)(hi + 2048 * i);
    v8i r;
    r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
    r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
    return r;
}

// `stage`: LDS byte address of the stage, opaque to the compiler.  The
// stage offsets of the later stages do not fit a DS instruction's 16-bit
// offset; folded into every read they made the compiler keep an address
// register per row block and spill them.  From one per-lane base per
// operand, every read of a step takes an immediate offset.
template <int ACC, int SH, int KIND>
__device__ __forceinline__ void compute_cols(uint32_t stage, int c, int lane, v4f (&acc)[Shape<SH>::BM / 16][2]) {
    constexpr int MI = Shape<SH>::BM / 16;
    static_assert(Shape<SH>::BN == 128, "one block column per tile");
    const int nbase = 32 * c, c0 = 2 * (lane >> 4), l16 = lane & 15;
    const uint32_t alo = stage + Lds<SH>::A + f8_off(l16, c0), ahi = stage + Lds<SH>::A + f8_off(l16, c0 + 1);
    const uint32_t bb = stage + Lds<SH>::B + 128 * nbase;
    const v8i b0 = f8_frag_at(bb + f8_off(l16, c0), bb + f8_off(l16, c0 + 1), 0);
    const v8i b1 = f8_frag_at(bb + f8_off(l16, c0), bb + f8_off(l16, c0 + 1), 1);
    lds_f32* sal = (lds_f32*)(uintptr_t)(stage + Lds<SH>::SA + 4 * l16);  // row scales, +16 per row block
    lds_f32* sb = (lds_f32*)(uintptr_t)(stage + Lds<SH>::SB);  // block scalar, or per-column scales
    // Every row block of the tile (rows past m_valid come from the stage's
    // clamped rows and are never stored; a data-dependent exit made the
    // compiler copy the accumulators at every exit and spill), in pairs,
    // software-pipelined: the next pair's A fragments and scales are read
    // from LDS before this pair's MFMAs, and the previous pair's partials
    // are promoted while this pair's MFMAs run.
    v8i a[2];
    float sv[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        a[h] = f8_frag_at(alo, ahi, h);
        sv[h] = sal[16 * h];
    }
    if constexpr (ACC == 2) {
        const int s0 = e8m0(KIND == 0 ? sb[0] : sb[nbase + (lane & 15)]);
        const int s1 = e8m0(KIND == 0 ? sb[0] : sb[nbase + 16 + (lane & 15)]);
#pragma unroll
        for (int i = 0; i < MI; i += 2) {
            v8i na[2];
            float ns[2];
            if (i + 2 < MI) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    na[h] = f8_frag_at(alo, ahi, i + 2 + h);
                    ns[h] = sal[16 * (i + 2 + h)];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int sab = e8m0(sv[h]);
                acc[i + h][0] =
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, a[h], acc[i + h][0], 0, 0, 0, s0, 0, sab);
                acc[i + h][1] =
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, a[h], acc[i + h][1], 0, 0, 0, s1, 0, sab);
            }
            if (i + 2 < MI) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    a[h] = na[h];
                    sv[h] = ns[h];
                }
            }
        }
    } else {
        const float sbk = KIND == 0 ? sb[0] : 1.f;
        v4f sbn0 = {1.f, 1.f, 1.f, 1.f}, sbn1 = sbn0;
        if (KIND == 1) {
            sbn0 = *(__attribute__((address_space(3))) const v4f*)(sb + nbase + 4 * (lane >> 4));
            sbn1 = *(__attribute__((address_space(3))) const v4f*)(sb + nbase + 16 + 4 * (lane >> 4));
        }
        v4f pp[2][2];
        float pc[2];
        auto promote = [&](int i) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                if (KIND == 0) {
                    acc[i + h][0] += pp[h][0] * pc[h];
                    acc[i + h][1] += pp[h][1] * pc[h];
                } else {
                    acc[i + h][0] += (pp[h][0] * pc[h]) * sbn0;
                    acc[i + h][1] += (pp[h][1] * pc[h]) * sbn1;
                }
            }
        };
#pragma unroll
        for (int i = 0; i < MI; i += 2) {
            v8i na[2];
            float ns[2];
            if (i + 2 < MI) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    na[h] = f8_frag_at(alo, ahi, i + 2 + h);
                    ns[h] = sal[16 * (i + 2 + h)];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            v4f p[2][2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                p[h][0] = mfma8_group(b0, a[h]);
                p[h][1] = mfma8_group(b1, a[h]);
            }
            if (i > 0) promote(i - 2);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                pp[h][0] = p[h][0];
                pp[h][1] = p[h][1];
                pc[h] = KIND == 0 ? sv[h] * sbk : sv[h];
            }
            if (i + 2 < MI) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    a[h] = na[h];
                    sv[h] = ns[h];
                }
            }
        }
        promote(MI - 2);
    }
}

template <int ACC, int SH, int KIND, int OUT>
__device__ __forceinline__ void run_tile_split(const Tile& T, int64_t g1, void* d, int64_t ldd, uint8_t* smem) {
    static_assert(ACC != 0 && OUT <= 1, "FP8 paths, bf16 or fp32 output");
    constexpr int S = Shape<SH>::STAGES, MI = Shape<SH>::BM / 16;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    float* ep = (float*)smem;

    // The two roles run separate loops that meet at the same barriers (one
    // per group and one after the last): s_barrier waits for every wave of
    // the workgroup whichever barrier instruction each one is at.  Kept
    // apart, the compute loop's accumulators never merge with a path that
    // leaves them untouched (such merges cost a copy of every accumulator).
    if (wave < LOADERS) {
        Stager<SH, KIND, true> stg;
        stg.init(T, wave, lane);
#pragma unroll
        for (int s = 0; s < S - 1; s++)
            if (s < g1) stg.issue(T, s, smem, s * Lds<SH>::STAGE, wave);
        // as in run_tile: wait until group g has landed (the S - 2 following
        // groups may still be in flight), meet the compute waves at the
        // barrier, refill the stage of group g - 1.  This loader's tile
        // loads per group: its valid A instructions and its B ones; its
        // scale loads come on top, so waiting for k * per outstanding is
        // conservative.
        constexpr int PER = (Shape<SH>::BM + Shape<SH>::BN) / 8 / LOADERS;
        static_assert((S == 4 || S == 3) && (S - 2) * PER <= 63, "wait counts cover this pipeline");
        const int per = stg.na_valid + Stager<SH, KIND, true>::NB;
        auto step = [&](auto ss, int64_t g) {
            constexpr int SS = decltype(ss)::value;
            if (S == 4 && g + 2 < g1)
                wait_n_and_barrier<2 * PER>(2 * per);
            else if (S >= 3 && g + 1 < g1)
                wait_n_and_barrier<PER>(per);
            else
                asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            if (g + S - 1 < g1) stg.issue(T, g + S - 1, smem, ((SS + S - 1) % S) * Lds<SH>::STAGE, wave);
        };
        for (int64_t g = 0; g < g1; g += S) {
            step(std::integral_constant<int, 0>(), g);
            if (g + 1 < g1) step(std::integral_constant<int, 1>(), g + 1);
            if (g + 2 < g1) step(std::integral_constant<int, 2>(), g + 2);
            if constexpr (S == 4)
                if (g + 3 < g1) step(std::integral_constant<int, 3>(), g + 3);
        }
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // every group used
    } else {
        const int c = wave - LOADERS;
        v4f acc[MI][2];
#pragma unroll
        for (int i = 0; i < MI; i++) acc[i][0] = acc[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
        auto step = [&](auto ss) {
            constexpr int SS = decltype(ss)::value;
            asm volatile("s_barrier" ::: "memory");
            uint32_t stage = lds_addr(smem) + SS * Lds<SH>::STAGE;
            asm volatile("" : "+s"(stage));
            compute_cols<ACC, SH, KIND>(stage, c, lane, acc);
        };
        for (int64_t g = 0; g < g1; g += S) {
            step(std::integral_constant<int, 0>());
            if (g + 1 < g1) step(std::integral_constant<int, 1>());
            if (g + 2 < g1) step(std::integral_constant<int, 2>());
            if constexpr (S == 4)
                if (g + 3 < g1) step(std::integral_constant<int, 3>());
        }
        asm volatile("s_barrier" ::: "memory");  // the stages hold the output image next
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                put4<SH>(ep, 16 * i + (lane & 15), 32 * c + 16 * j + 4 * (lane >> 4), acc[i][j][0], acc[i][j][1],
                         acc[i][j][2], acc[i][j][3]);
    }
    __syncthreads();
    write_tile_image<SH, OUT, true>(ep, T, T.n0, d, ldd);
    __syncthreads();  // a following row tile refills the stages
}

// Grouped, FP8 paths: workgroup (expert e, n-tile) walks the expert's rows
// in 256-row tiles, a last tile of fewer rows on the smallest shape that
// holds them.
template <int ACC, int KIND, int OUT>
__global__ __launch_bounds__(THREADS) void grouped_split_kernel(GemmArgs p, int64_t tiles_n) {
    constexpr int LDS_BYTES = Lds<11>::BYTES;
    static_assert(Lds<10>::BYTES <= LDS_BYTES && Lds<12>::BYTES <= LDS_BYTES && Lds<13>::BYTES <= LDS_BYTES,
                  "every row-tile shape fits");
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t e = wid / tiles_n;
    const int64_t tn = wid % tiles_n;
    const int64_t r0 = p.offsets[e], r1 = p.offsets[e + 1];

    Tile T;
    T.m_end = r1;
    T.n0 = tn * 128;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b + e * p.b_estride;
    T.ldb = p.ldb;
    T.sb = p.sb + e * p.sb_estride;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = p.sb_s1;
    for (int64_t m0 = r0; m0 < r1; m0 += Shape<11>::BM) {
        T.m0 = m0;
        const int64_t rows = r1 - m0;
        if (rows <= Shape<13>::BM)
            run_tile_split<ACC, 13, KIND, OUT>(T, p.K / 128, p.d, p.ldd, smem);
        else if (rows <= Shape<10>::BM)
            run_tile_split<ACC, 10, KIND, OUT>(T, p.K / 128, p.d, p.ldd, smem);
        else if (rows <= Shape<12>::BM)
            run_tile_split<ACC, 12, KIND, OUT>(T, p.K / 128, p.d, p.ldd, smem);
        else
            run_tile_split<ACC, 11, KIND, OUT>(T, p.K / 128, p.d, p.ldd, smem);
    }
}

// K-grouped (MoE Wgrad over each expert's tokens): workgroup (expert e,
// output tile) sums the expert's K groups, which sit consecutively on the
// padded token axis starting at group sum_{e'<e} ceil(n_e'/128).  An expert
// without tokens writes zeros.
__device__ __forceinline__ int64_t expert_first_group(const int32_t* __restrict__ offsets, int64_t e) {
    __shared__ int64_t wsum[WAVES];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t acc = 0;
    for (int64_t i = t; i < e; i += THREADS) acc += ((int64_t)offsets[i + 1] - offsets[i] + 127) / 128;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
    if (lane == 0) wsum[wave] = acc;
    __syncthreads();
    int64_t total = 0;
#pragma unroll
    for (int w = 0; w < WAVES; w++) total += wsum[w];
    __syncthreads();
    return total;
}

// Each workgroup takes a strip of KSTRIP n-tiles of one (expert, m-tile):
// experts hold few tokens, so a tile's K loop is short and the expert's
// group range (two dependent reads of the offsets) is looked up once per
// strip rather than once per tile.
constexpr int KSTRIP = 8;

template <int ACC, int OUT>
__global__ __launch_bounds__(THREADS) void kgrouped_kernel(GemmArgs p, int64_t tiles_m, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Lds<0>::BYTES];
    const int64_t strips = (tiles_n + KSTRIP - 1) / KSTRIP;
    const int64_t per = tiles_m * strips;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t e = wid / per;
    const int64_t tm = (wid % per) % tiles_m, strip = (wid % per) / tiles_m;
    const int64_t g0 = expert_first_group(p.offsets, e);
    const int64_t g1 = g0 + ((int64_t)p.offsets[e + 1] - p.offsets[e] + 127) / 128;

    Tile T;
    T.m0 = tm * Shape<0>::BM;
    T.m_end = p.M;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b;
    T.ldb = p.ldb;
    T.sb = p.sb;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = 0;
    void* d = (uint8_t*)p.d + e * p.d_estride * (OUT ? 4 : 2);
    const int64_t tn_end = (strip + 1) * KSTRIP < tiles_n ? (strip + 1) * KSTRIP : tiles_n;
    for (int64_t tn = strip * KSTRIP; tn < tn_end; tn++) {
        T.n0 = tn * Shape<0>::BN;
        run_tile<ACC, 0, 1, OUT>(T, g0, g1, d, p.ldd, smem);
    }
}

// K-grouped Wgrad, experts of at most two K groups: the workgroup's B tile
// (its column tile of every group of the expert) is staged once and stays
// in LDS while the strip's row tiles stage only their A groups; a tile's
// fp32 output goes out through the A ring in two 64-column images.  Other
// experts run each tile through the two-stage pipeline of shape 5.  LDS:
// B groups [2][codes 16 KB + 128
// column scales], then the A ring [2][codes 16 KB + 128 row scales, padded
// so that the ring holds a 128 x 64 fp32 image].
constexpr int KG3_BGROUP = 128 * 128 + 128 * 4;
constexpr int KG3_ASTAGE = 128 * 128 + 128 * 4 + 512;
constexpr int KG3_A = 2 * KG3_BGROUP;
constexpr int KG3_BYTES = KG3_A + 2 * KG3_ASTAGE;
static_assert(128 * Epi<8>::LD * 4 <= 2 * KG3_ASTAGE && Lds<5>::BYTES <= KG3_BYTES, "the K-grouped LDS map");

__device__ __forceinline__ void kg3_issue_a(const Stager<5, 1>& stg, const Tile& T, int64_t g, uint8_t* dst,
                                            int wave) {
    const uint8_t* a = T.a + T.m0 * T.lda + g * 128;
    const uint32_t base = lds_addr(dst);
#pragma unroll
    for (int ins = 0; ins < Stager<5, 1>::NA; ins++) dma16s(stg.va[ins], a, base + (ins * LOADERS + wave) * 8 * 128);
    if (wave < Stager<5, 1>::SA_INS) dma4s(stg.vsa, T.sa + g * T.ldsa + T.m0, base + 128 * 128 + wave * 256);
}

__device__ __forceinline__ void kg3_issue_b(const Stager<5, 1>& stg, const Tile& T, int64_t g, uint8_t* dst,
                                            int wave) {
    const uint8_t* b = T.b + T.n0 * T.ldb + g * 128;
    const uint32_t base = lds_addr(dst);
#pragma unroll
    for (int ins = 0; ins < Stager<5, 1>::NB; ins++) dma16s(stg.vb[ins], b, base + (ins * LOADERS + wave) * 8 * 128);
    if (wave < Stager<5, 1>::SB_INS) dma4s(stg.vsb, T.sb + g * T.sb_s0 + T.n0, base + 128 * 128 + wave * 256);
}

template <int ACC, int OUT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void kgrouped3_kernel(
    GemmArgs p, int64_t tiles_m, int64_t tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[KG3_BYTES];
    const int64_t strips = (tiles_m + KSTRIP - 1) / KSTRIP;
    const int64_t per = tiles_n * strips;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t e = wid / per;
    const int64_t tn = (wid % per) % tiles_n, strip = (wid % per) / tiles_n;
    const int64_t g0 = expert_first_group(p.offsets, e);
    const int64_t ng = ((int64_t)p.offsets[e + 1] - p.offsets[e] + 127) / 128;

    Tile T;
    T.n0 = tn * 128;
    T.m_end = p.M;
    T.n_end = p.N;
    T.a = p.a;
    T.lda = p.lda;
    T.sa = p.sa;
    T.ldsa = p.ldsa;
    T.b = p.b;
    T.ldb = p.ldb;
    T.sb = p.sb;
    T.sb_s0 = p.sb_s0;
    T.sb_s1 = 0;
    void* d = (uint8_t*)p.d + e * p.d_estride * (OUT ? 4 : 2);
    const int64_t tm0 = strip * KSTRIP, tm1 = tm0 + KSTRIP < tiles_m ? tm0 + KSTRIP : tiles_m;
    if (ng == 0 || ng > 2) {
        for (int64_t tm = tm0; tm < tm1; tm++) {
            T.m0 = tm * 128;
            run_tile<ACC, 5, 1, OUT>(T, g0, g0 + ng, d, p.ldd, smem);
        }
        return;
    }
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    int wm, wn;
    Shape<8>::wave_grid(wave, wm, wn);
    Stager<5, 1> stg;
    T.m0 = tm0 * 128;
    stg.init(T, wave, lane);
    if (wave < LOADERS)
        for (int k = 0; k < ng; k++) kg3_issue_b(stg, T, g0 + k, smem + k * KG3_BGROUP, wave);
    for (int64_t tm = tm0; tm < tm1; tm++) {
        T.m0 = tm * 128;
        if (tm != tm0) stg.init(T, wave, lane);
        if (wave < LOADERS)
            for (int k = 0; k < ng; k++) kg3_issue_a(stg, T, g0 + k, smem + KG3_A + k * KG3_ASTAGE, wave);
        wait_and_barrier<0>(wave);  // this tile's A groups (and, the first time, B) have landed
        const int m_valid = (int)(T.m_end - T.m0 < 128 ? T.m_end - T.m0 : 128);
        v4f acc[Sub<8>::MI][Sub<8>::NJ];
#pragma unroll
        for (int i = 0; i < Sub<8>::MI; i++)
#pragma unroll
            for (int j = 0; j < Sub<8>::NJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < ng; k++) {
            const uint8_t* as = smem + KG3_A + k * KG3_ASTAGE;
            const uint8_t* bg = smem + k * KG3_BGROUP;
            const StagePtrs sp{as, bg, (const float*)(as + 128 * 128), (const float*)(bg + 128 * 128)};
            if constexpr (ACC == 1)
                compute_mfma8<8, 1>(sp, wm, wn, lane, m_valid, acc);
            else
                compute_mfma8_pow2<8, 1>(sp, wm, wn, lane, m_valid, acc);
        }
        __syncthreads();  // every wave is done with the A ring, which the images reuse
        store_mfma8<8, OUT>(acc, T, wm, wn, lane, d, p.ldd, smem + KG3_A);
    }
}

// Sum split-K partials in split order and convert.
template <int OUT>
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
    if (n + 4 <= N)
        store4_full<OUT>(d, ldd, m, n, s.x, s.y, s.z, s.w);
    else
        store4<OUT>(d, ldd, m, n, N, s.x, s.y, s.z, s.w);
}

// ==== host side ==========================================================================

int gemm_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + Shape<0>::BM - 1) / Shape<0>::BM) * ((N + Shape<0>::BN - 1) / Shape<0>::BN);
    const int64_t groups = K / 128;
    if (tiles == 0 || groups < 16 || tiles >= 128) return 1;
    int64_t s = 256 / tiles;         // about one workgroup per CU
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

template <int ACC, int SH, int KIND, int OUT, bool SPLIT>
static void launch_shape(const GemmArgs& g, hipStream_t st) {
    const int64_t tiles_m = (g.M + Shape<SH>::BM - 1) / Shape<SH>::BM;
    const int64_t tiles_n = (g.N + Shape<SH>::BN - 1) / Shape<SH>::BN;
    const int64_t wgs = tiles_m * tiles_n * (SPLIT ? g.splits : 1);
    hipLaunchKernelGGL((gemm_kernel<ACC, SH, KIND, OUT, SPLIT>), dim3((unsigned)wgs), dim3(THREADS), 0, st, g,
                       tiles_m, tiles_n);
}

// Compute units of the current device (one workgroup of either shape fills
// a CU's LDS, so this is also the number of tiles in flight).
static int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// The FP8 paths run the first n1 output columns on 256 x 256 tiles and the
// rest on 256 x 128 tiles.  n1 (a multiple of 256; n1 >= N puts every
// column on wide tiles) minimises the rounds of
// workgroups, counting a round of the narrow tiles as 0.65 of a round of
// the wide ones (their measured time per tile): 4096 x 18432, 4.5 rounds
// of wide tiles, becomes 4 rounds of wide tiles and one of narrow ones.
int64_t wide_columns(int64_t M, int64_t N, int cus, double* cost_out) {
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    int64_t best_n1 = 256 * tn;  // every column on wide tiles
    double best = (double)((tm * tn + cus - 1) / cus);
    for (int64_t n1t = 0; n1t < tn; n1t++) {
        const int64_t t1 = tm * n1t, t0 = tm * ((N - 256 * n1t + 127) / 128);
        const double cost = (double)((t1 + cus - 1) / cus) + 0.65 * (double)((t0 + cus - 1) / cus);
        if (cost < best - 1e-9) {
            best = cost;
            best_n1 = 256 * n1t;
        }
    }
    if (cost_out) *cost_out = best;
    return best_n1;
}

// Rounds of 256 x 224 tiles, in the wide tile's rounds (a 256 x 224 tile is
// 7/8 of a wide tile's work).
static double cols224_cost(int64_t M, int64_t N, int cus) {
    const int64_t tiles = ((M + 255) / 256) * ((N + 223) / 224);
    return 0.875 * (double)((tiles + cus - 1) / cus);
}

// Split-K and the f16 path use shape 0; the FP8 paths gemm_wide_kernel,
// shape 1 on the first wide_columns() columns and shape 0 on the rest.
template <int ACC, int KIND, int OUT, bool SPLIT>
static void launch_dense(const GemmArgs& g, hipStream_t st) {
    if constexpr (ACC == 0 || SPLIT) {
        launch_shape<ACC, 0, KIND, OUT, SPLIT>(g, st);
    } else {
        const int cus = device_cus();
        double wide_cost = 0.0;
        const int64_t n1 = wide_columns(g.M, g.N, cus, &wide_cost);
        if constexpr (ACC == 1 && KIND == 1 && OUT <= 1) {
            // per-column scales, FP32-scale mode: 256 x 224 tiles where
            // their rounds come out fuller (2048 x 7168: one full round)
            if (cols224_cost(g.M, g.N, cus) < wide_cost - 0.05) {
                launch_shape<1, 7, 1, OUT, false>(g, st);
                return;
            }
        }
        const int64_t tiles_m = (g.M + Shape<1>::BM - 1) / Shape<1>::BM;
        const int64_t narrow_n = n1 < g.N ? (g.N - n1 + Shape<0>::BN - 1) / Shape<0>::BN : 0;
        const int64_t wgs = tiles_m * (n1 / Shape<1>::BN) + tiles_m * narrow_n;
        hipLaunchKernelGGL((gemm_wide_kernel<ACC, KIND, OUT>), dim3((unsigned)wgs), dim3(THREADS), 0, st, g, n1);
    }
}

template <int ACC>
static hipError_t launch_gemm_acc(const GemmArgs& g, hipStream_t st) {
    if (g.splits > 1 && !g.out_quant) {
        if (g.bscale_kind == 0)
            launch_dense<ACC, 0, 1, true>(g, st);
        else
            launch_dense<ACC, 1, 1, true>(g, st);
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
    if (g.out_quant) {
        if (g.bscale_kind == 0) {
            if (g.out_quant == 1)
                launch_dense<ACC, 0, 2, false>(g, st);
            else
                launch_dense<ACC, 0, 3, false>(g, st);
        } else {
            if (g.out_quant == 1)
                launch_dense<ACC, 1, 2, false>(g, st);
            else
                launch_dense<ACC, 1, 3, false>(g, st);
        }
        return hipGetLastError();
    }
    if (g.bscale_kind == 0) {
        if (g.out_f32)
            launch_dense<ACC, 0, 1, false>(g, st);
        else
            launch_dense<ACC, 0, 0, false>(g, st);
    } else {
        if (g.out_f32)
            launch_dense<ACC, 1, 1, false>(g, st);
        else
            launch_dense<ACC, 1, 0, false>(g, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    if (g.accum == 0) return launch_gemm_acc<0>(g, st);
    return g.accum == 1 ? launch_gemm_acc<1>(g, st) : launch_gemm_acc<2>(g, st);
}

template <int ACC>
static hipError_t launch_grouped_acc(const GemmArgs& g, hipStream_t st) {
    const int64_t tiles_n = (g.N + Shape<0>::BN - 1) / Shape<0>::BN;
    const dim3 grid((unsigned)(tiles_n * g.G));
    if constexpr (ACC != 0) {
        if (g.bscale_kind == 0) {
            if (g.out_f32)
                hipLaunchKernelGGL((grouped_split_kernel<ACC, 0, 1>), grid, dim3(THREADS), 0, st, g, tiles_n);
            else
                hipLaunchKernelGGL((grouped_split_kernel<ACC, 0, 0>), grid, dim3(THREADS), 0, st, g, tiles_n);
        } else {
            if (g.out_f32)
                hipLaunchKernelGGL((grouped_split_kernel<ACC, 1, 1>), grid, dim3(THREADS), 0, st, g, tiles_n);
            else
                hipLaunchKernelGGL((grouped_split_kernel<ACC, 1, 0>), grid, dim3(THREADS), 0, st, g, tiles_n);
        }
        return hipGetLastError();
    }
    else {
        if (g.bscale_kind == 0) {
            if (g.out_f32)
                hipLaunchKernelGGL((grouped_kernel<ACC, 0, 1>), grid, dim3(THREADS), 0, st, g, tiles_n);
            else
                hipLaunchKernelGGL((grouped_kernel<ACC, 0, 0>), grid, dim3(THREADS), 0, st, g, tiles_n);
        } else {
            if (g.out_f32)
                hipLaunchKernelGGL((grouped_kernel<ACC, 1, 1>), grid, dim3(THREADS), 0, st, g, tiles_n);
            else
                hipLaunchKernelGGL((grouped_kernel<ACC, 1, 0>), grid, dim3(THREADS), 0, st, g, tiles_n);
        }
        return hipGetLastError();
    }
}

template <int ACC>
static hipError_t launch_kgrouped_acc(const GemmArgs& g, hipStream_t st) {
    if constexpr (ACC != 0) {
        const int64_t tiles_m = (g.M + 127) / 128, tiles_n = (g.N + 127) / 128;
        const dim3 grid((unsigned)(tiles_n * ((tiles_m + KSTRIP - 1) / KSTRIP) * g.G));
        if (g.out_f32)
            hipLaunchKernelGGL((kgrouped3_kernel<ACC, 1>), grid, dim3(THREADS), 0, st, g, tiles_m, tiles_n);
        else
            hipLaunchKernelGGL((kgrouped3_kernel<ACC, 0>), grid, dim3(THREADS), 0, st, g, tiles_m, tiles_n);
        return hipGetLastError();
    }
    const int64_t tiles_m = (g.M + Shape<0>::BM - 1) / Shape<0>::BM;
    const int64_t tiles_n = (g.N + Shape<0>::BN - 1) / Shape<0>::BN;
    const dim3 grid((unsigned)(tiles_m * ((tiles_n + KSTRIP - 1) / KSTRIP) * g.G));
    if (g.out_f32)
        hipLaunchKernelGGL((kgrouped_kernel<ACC, 1>), grid, dim3(THREADS), 0, st, g, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((kgrouped_kernel<ACC, 0>), grid, dim3(THREADS), 0, st, g, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_kgrouped_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.G == 0 || g.M == 0 || g.N == 0) return hipSuccess;
    if (g.accum == 0) return launch_kgrouped_acc<0>(g, st);
    return g.accum == 1 ? launch_kgrouped_acc<1>(g, st) : launch_kgrouped_acc<2>(g, st);
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.G == 0 || g.N == 0) return hipSuccess;
    if (g.accum == 0) return launch_grouped_acc<0>(g, st);
    return g.accum == 1 ? launch_grouped_acc<1>(g, st) : launch_grouped_acc<2>(g, st);
}

}  // namespace fp8bs
