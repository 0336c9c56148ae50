// quant.hip -- online fine-grained quantisation kernels for gfx950.
//
// The quantisers are HBM-bound: each element is read once as bf16 (2 B) and
// written once as an E4M3 code (1 B), plus 4 B of scale per group.  Every
// kernel keeps its loads 16 B per lane and fully coalesced, finds the group
// max with packed 16-bit maxima and DPP reductions inside a 16-lane row,
// and rounds with e4m3_code (see device.h).
#include "device.h"
#include "kernels.h"

namespace fp8bs {

// Streaming accesses: every input byte is read once and every code written
// once, so loads and the row-contiguous code stores are non-temporal (they
// do not displace other data in the caches; measured 5-10% faster on the
// quantisers).  The transposed copy's 8-byte column stores stay ordinary
// stores: they fill each 128-byte line from several lanes and instructions,
// which the caches merge.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void st_stream8(void* p, uint2 v) {
    __builtin_nontemporal_store((u32x2){v.x, v.y}, (u32x2*)p);
}

// ---- plain cast ------------------------------------------------------------------

__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ x, int64_t n,
                                                   uint8_t* __restrict__ q) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        const float4 v = *(const float4*)(x + i);
        *(uint32_t*)(q + i) = pack4(v.x, v.y, v.z, v.w);
    } else {
        for (int64_t j = i; j < n; j++) q[j] = (uint8_t)e4m3_code(x[j]);
    }
}

hipError_t launch_cast(const float* x, int64_t n, uint8_t* q, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, q);
    return hipGetLastError();
}

// ---- power-of-two scale check ---------------------------------------------------------
//
// Writes 1 to *flag, then any thread that meets an entry which is not a
// positive normal power of two (sign 0, exponent field 1..254, mantissa 0)
// writes 0: every writer stores the same value.

__global__ void pow2_flag_init_kernel(int32_t* __restrict__ flag) { *flag = 1; }

__global__ __launch_bounds__(256) void pow2_check_kernel(const float* __restrict__ s, int64_t rows, int64_t cols,
                                                         int64_t ld_r, int64_t ld_c, int32_t* __restrict__ flag) {
    const int64_t n = rows * cols;
    bool ok = true;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cols, c = i % cols;
        const uint32_t b = __float_as_uint(s[r * ld_r + c * ld_c]);
        const uint32_t e = (b >> 23) & 0xFFu;
        ok = ok && (b & 0x807FFFFFu) == 0 && e != 0 && e != 0xFF;
    }
    if (!ok) *flag = 0;
}

hipError_t launch_scales_pow2_check(const float* s, int64_t rows, int64_t cols, int64_t ld_r, int64_t ld_c,
                                    int32_t* flag, hipStream_t st) {
    hipLaunchKernelGGL(pow2_flag_init_kernel, dim3(1), dim3(1), 0, st, flag);
    const int64_t n = rows * cols;
    if (n == 0) return hipGetLastError();
    const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(pow2_check_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s, rows, cols, ld_r, ld_c, flag);
    return hipGetLastError();
}

// ---- 1x128 groups along rows ---------------------------------------------------------
//
// A workgroup covers 4*RPW rows x 512 columns: each wave takes RPW rows,
// each 16-lane DPP row one 128-element group (8 bf16 = 16 B per lane).  The
// RPW row loads are issued before any reduction so 16*RPW B per lane are in
// flight.

template <bool POW2, int RPW>
__device__ __forceinline__ void row_tile_load(const uint16_t* __restrict__ x, int64_t rows, int64_t ldx,
                                              int64_t r0, int64_t col, bool colok, uint4 (&v)[RPW]) {
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        const int64_t r = r0 + i;
        v[i] = (colok && r < rows) ? ld_stream16(x + r * ldx + col) : make_uint4(0, 0, 0, 0);
    }
}

template <bool POW2, int RPW>
__device__ __forceinline__ void row_tile_store(const uint4 (&v)[RPW], int64_t rows, int64_t r0, int64_t col,
                                               bool colok, int lane, uint8_t* __restrict__ q, int64_t ldq,
                                               float* __restrict__ s, int64_t lds) {
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        const uint32_t am = row16_max(absmax8(v[i]));
        const GroupScale gs = group_scale(am, POW2);
        const int64_t r = r0 + i;
        if (colok && r < rows) {
            st_stream8(q + r * ldq + col, quant8(v[i], gs.inv));
            if ((lane & 15) == 0) s[(col >> 7) * lds + r] = gs.s;
        }
    }
}

template <bool POW2, int RPW>
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s, int64_t lds,
                                                        int64_t col_tiles) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile_c = blockIdx.x % col_tiles;
    const int64_t tile_r = blockIdx.x / col_tiles;
    const int64_t col = tile_c * 512 + lane * 8;
    const bool colok = col < cols;
    const int64_t r0 = (tile_r * 4 + wave) * RPW;
    uint4 v[RPW];
    row_tile_load<POW2, RPW>(x, rows, ldx, r0, col, colok, v);
    row_tile_store<POW2, RPW>(v, rows, r0, col, colok, lane, q, ldq, s, lds);
}

// ---- 128x1 groups down columns, codes written transposed -------------------------------
//
// A workgroup covers one 128-row group x 64 columns.  Load: wave w, lane
// L reads rows 32w + 16it + 2p + {0,1} (p = L%8, it = 0..1) of the 8-column
// chunk L/8, packs the two rows' values of each column into one dword and
// stores it to LDS at column-major position (column c, row pair rp) with the
// 16-byte chunk index of rp XOR-swizzled by 2*(c/8): the 32 lanes of each
// half-wave then hit 32 different banks.  Process: each 16-lane DPP row
// reads one column (lane l: rows 8l..8l+7, one 16 B LDS read), reduces the
// column's amax, and writes 8 codes, so the 16 lanes store the group's 128
// codes as one contiguous 128 B run of the transposed output.

__device__ __forceinline__ uint32_t col_lds_index(int c, int rp) {
    const int chunk = (rp >> 2) ^ ((c >> 3) << 1);
    return (uint32_t)(c * 64 + chunk * 4 + (rp & 3));
}

__device__ __forceinline__ uint4 load_chunk_masked(const uint16_t* __restrict__ p, int64_t col,
                                                   int64_t cols) {
    if (col + 8 <= cols) return ld_stream16(p);
    uint32_t w[4] = {0, 0, 0, 0};
    for (int i = 0; i < 8; i++)
        if (col + i < cols) w[i >> 1] |= (uint32_t)p[i] << (16 * (i & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One 128x1 group per column for 64 columns: source rows xr[i*ldx], i < nrows
// (rows nrows..127 read as zero: they add nothing to the amax and encode to
// zero codes), codes to qg[col*ldq + i], scale to sg[col].
// Loads of one 128-row group x 64 columns: lane (chunk, p) of wave w holds
// the 8-column chunk of rows w*32 + 16*it + 2p and the row after it.
struct ColLoads {
    uint4 lo[2], hi[2];
};

__device__ __forceinline__ void col_group_load(const uint16_t* __restrict__ xr, int nrows, int64_t cols, int64_t ldx,
                                               int64_t c0, ColLoads& L) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = lane >> 3, p = lane & 7;
    const int64_t col = c0 + chunk * 8;
    const bool ok = col < cols;
#pragma unroll
    for (int it = 0; it < 2; it++) {
        const int r = wave * 32 + it * 16 + 2 * p;
        const uint16_t* src = xr + r * ldx + col;
        L.lo[it] = ok && r < nrows ? load_chunk_masked(src, col, cols) : make_uint4(0, 0, 0, 0);
        L.hi[it] = ok && r + 1 < nrows ? load_chunk_masked(src + ldx, col, cols) : make_uint4(0, 0, 0, 0);
    }
}

// The loaded group through the LDS tile (paired-row dwords, column-major),
// then each DPP row quantises one column's 128 values and stores them as
// one 128 B run.
template <bool POW2>
__device__ __forceinline__ void col_group_finish(const ColLoads& L, int64_t cols, int64_t c0,
                                                 uint8_t* __restrict__ qg, int64_t ldq, float* __restrict__ sg,
                                                 uint32_t* tile) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    {
        const int chunk = lane >> 3, p = lane & 7;
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int rp = wave * 16 + it * 8 + p;
            const uint32_t a[4] = {L.lo[it].x, L.lo[it].y, L.lo[it].z, L.lo[it].w};
            const uint32_t b[4] = {L.hi[it].x, L.hi[it].y, L.hi[it].z, L.hi[it].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int c = chunk * 8 + 2 * j;
                tile[col_lds_index(c, rp)] = perm(b[j], a[j], 0x05040100u);      // col c
                tile[col_lds_index(c + 1, rp)] = perm(b[j], a[j], 0x07060302u);  // col c+1
            }
        }
    }
    __syncthreads();

    const int l = lane & 15;
#pragma unroll
    for (int it = 0; it < 4; it++) {
        const int c = wave * 16 + it * 4 + (lane >> 4);
        const uint4 v = *(const uint4*)&tile[col_lds_index(c, 4 * l)];
        const uint32_t am = row16_max(absmax8(v));
        const GroupScale gs = group_scale(am, POW2);
        const int64_t col = c0 + c;
        if (col < cols) {
            st_stream8(qg + col * ldq + 8 * l, quant8(v, gs.inv));
            if (l == 0) sg[col] = gs.s;
        }
    }
}

template <bool POW2>
__device__ __forceinline__ void col_group_tile(const uint16_t* __restrict__ xr, int nrows, int64_t cols,
                                               int64_t ldx, int64_t c0, uint8_t* __restrict__ qg, int64_t ldq,
                                               float* __restrict__ sg, uint32_t* tile) {
    ColLoads L;
    col_group_load(xr, nrows, cols, ldx, c0, L);
    col_group_finish<POW2>(L, cols, c0, qg, ldq, sg, tile);
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_col_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s, int64_t lds,
                                                        int64_t col_tiles) {
    __shared__ uint32_t tile[64 * 64];
    // Consecutive workgroups take consecutive row groups of one column tile,
    // so the transposed code runs they write continue one another in each
    // output row (14% faster than walking the column tiles of a row group
    // first, on X[8192 x 7168]).
    const int64_t gt = gridDim.x / col_tiles;
    const int64_t g = blockIdx.x % gt;
    const int64_t c0 = (blockIdx.x / gt) * 64;
    col_group_tile<POW2>(x + g * 128 * ldx, 128, cols, ldx, c0, q + g * 128, ldq, s + g * lds, tile);
}

// ---- 128x1 groups restarted at every expert boundary ------------------------------------------
//
// Tokens of G experts lie back to back (expert e: rows offsets[e] ..
// offsets[e+1]-1).  Every expert is cut into 128-token groups from its first
// token, the last one possibly partial, and the groups are numbered
// consecutively on a padded token axis (expert e starts at 128 * the number of
// groups before it).  Each group is quantised like quant_col_kernel with
// the rows past the expert's end read as zero -- its padding codes come out
// zero.
//
// Workgroup (expert e, 64 columns) quantises the expert's groups in turn.
// Its first group's loads depend only on offsets[e] and are issued first;
// the expert's place on the padded axis (the groups of the experts before
// it), which only the stores need, is summed while they are in flight.
// Consecutive workgroups take consecutive experts of one column tile, whose
// groups follow one another on the padded axis.
template <bool POW2>
__global__ __launch_bounds__(256) void quant_grouped_col_kernel(const uint16_t* __restrict__ x, int64_t cols,
                                                                int64_t ldx, int G,
                                                                const int32_t* __restrict__ offsets,
                                                                uint8_t* __restrict__ q, int64_t ldq,
                                                                float* __restrict__ s, int64_t lds) {
    __shared__ uint32_t tile[64 * 64];
    __shared__ int64_t wsum[4];
    const int e = (int)(blockIdx.x % (unsigned)G);
    const int64_t c0 = (int64_t)(blockIdx.x / (unsigned)G) * 64;
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    const int64_t ng = (r1 - r0 + 127) / 128;
    if (ng <= 0) return;  // an expert without tokens has no groups
    ColLoads L;
    col_group_load(x + r0 * ldx, (int)(r1 - r0 < 128 ? r1 - r0 : 128), cols, ldx, c0, L);

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t before = 0;
    for (int i = t; i < e; i += 256) before += ((int64_t)offsets[i + 1] - offsets[i] + 127) / 128;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) before += __shfl_xor(before, d);
    if (lane == 0) wsum[wave] = before;
    __syncthreads();
    const int64_t first = wsum[0] + wsum[1] + wsum[2] + wsum[3];

    for (int64_t j = 0; j < ng; j++) {
        if (j > 0) {
            __syncthreads();  // the previous group's tile has been read
            const int64_t rj = r0 + 128 * j;
            col_group_load(x + rj * ldx, (int)(r1 - rj < 128 ? r1 - rj : 128), cols, ldx, c0, L);
        }
        col_group_finish<POW2>(L, cols, c0, q + (first + j) * 128, ldq, s + (first + j) * lds, tile);
    }
}

// ---- 128x128 blocks ----------------------------------------------------------------------
//
// The 256 threads of a workgroup quantise a block.  Thread t owns the 8x8 sub-block at rows
// 8(t/16).., columns 8(t%16)..; each load instruction reads 4 full 256 B
// row segments.  The block amax is a thread max, a wave max, then a max over
// the 4 waves through LDS.  The optional transposed copy is an in-register
// 8x8 byte transpose, each thread storing 8 columns x 8 rows.

// One block's worth for one thread: 8 rows x 8 columns.
__device__ __forceinline__ void block_load(const uint16_t* __restrict__ w, int64_t rows, int64_t ldw,
                                           int64_t r0, int64_t c0, uint4 (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; i++)
        v[i] = (r0 + i < rows) ? ld_stream16(w + (r0 + i) * ldw + c0) : make_uint4(0, 0, 0, 0);
}

// Quantise and store one block given every thread's 8x8 values; wmax is a
// 4-entry LDS array for the per-wave maxima.
template <bool POW2>
__device__ __forceinline__ void block_finish(const uint4 (&v)[8], uint32_t* wmax, int64_t rows, int64_t bi,
                                             int64_t bj, int64_t r0, int64_t c0, uint8_t* __restrict__ q,
                                             int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt,
                                             float* __restrict__ s, int64_t lds) {
    const int t = threadIdx.x;
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) am = max(am, absmax8(v[i]));
    am = wave_max(am);
    if ((t & 63) == 0) wmax[t >> 6] = am;
    __syncthreads();
    am = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const GroupScale gs = group_scale(am, POW2);
    if (t == 0) s[bi * lds + bj] = gs.s;

    uint2 c[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        c[i] = quant8(v[i], gs.inv);
        if (r0 + i < rows) st_stream8(q + (r0 + i) * ldq + c0, c[i]);
    }
    if (qt != nullptr) {
        uint32_t lo[8], hi[8];
        transpose4x4(c[0].x, c[1].x, c[2].x, c[3].x, lo[0], lo[1], lo[2], lo[3]);
        transpose4x4(c[4].x, c[5].x, c[6].x, c[7].x, hi[0], hi[1], hi[2], hi[3]);
        transpose4x4(c[0].y, c[1].y, c[2].y, c[3].y, lo[4], lo[5], lo[6], lo[7]);
        transpose4x4(c[4].y, c[5].y, c[6].y, c[7].y, hi[4], hi[5], hi[6], hi[7]);
        const bool full = r0 + 8 <= rows;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            uint8_t* dst = qt + (c0 + j) * ldqt + r0;
            if (full) {
                *(uint2*)dst = make_uint2(lo[j], hi[j]);
            } else {
                for (int i = 0; i < 8; i++)
                    if (r0 + i < rows) dst[i] = (uint8_t)((i < 4 ? lo[j] >> (8 * i) : hi[j] >> (8 * (i - 4))) & 0xFF);
            }
        }
    }
}

// A workgroup takes two blocks side by side (the second absent past the last
// block column), issuing both blocks' loads before quantising the first:
// its rows are read as 512 B runs.  On W[32x4096x7168] 502 -> 474 us
// against one block per workgroup; four blocks per workgroup left too few
// workgroups for W[18432x7168] (70 -> 75 us).
template <bool POW2>
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                          int64_t ldw, uint8_t* __restrict__ q,
                                                          int64_t ldq, uint8_t* __restrict__ qt,
                                                          int64_t ldqt, float* __restrict__ s,
                                                          int64_t lds, int64_t col_blocks) {
    __shared__ uint32_t wmax[8];
    const int t = threadIdx.x;
    const int64_t pairs = (col_blocks + 1) / 2;
    const int64_t bi = blockIdx.x / pairs, bj = 2 * (blockIdx.x % pairs);
    const bool second = bj + 1 < col_blocks;  // workgroup-uniform
    const int64_t r0 = bi * 128 + 8 * (t >> 4);
    const int64_t c0 = bj * 128 + 8 * (t & 15);
    uint4 v[8], v1[8];
    block_load(w, rows, ldw, r0, c0, v);
    if (second) block_load(w, rows, ldw, r0, c0 + 128, v1);
    block_finish<POW2>(v, wmax, rows, bi, bj, r0, c0, q, ldq, qt, ldqt, s, lds);
    if (second) block_finish<POW2>(v1, wmax + 4, rows, bi, bj + 1, r0, c0 + 128, q, ldq, qt, ldqt, s, lds);
}

// ---- both orientations from one read -------------------------------------------------------
//
// The backward pass needs dY in 1x128 groups (Dgrad) and in 128x1 groups
// (Wgrad).  A workgroup covers one 128 x 128 tile of x, read once.  Pass p,
// wave w, 16-lane DPP row d: lanes read rows r = 32p + 8w + 2d and r + 1 (16 B
// of bf16 each), quantise both as 1x128 groups (each row of the tile is one
// group), and store the two rows' values of every column packed in one
// dword of a column-major LDS tile (row pair r/2; the 16-byte chunk index
// XOR-swizzled by c/8, so the 64 lanes of a store hit distinct banks).  After
// the barrier each DPP row quantises one column at a time as a 128x1 group,
// as quant_col_kernel does.

__device__ __forceinline__ uint32_t dual_lds_index(int c, int rp) {
    return (uint32_t)(c * 64 + ((((rp >> 2) ^ (c >> 3)) & 15) << 2) + (rp & 3));
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_dual_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                         uint8_t* __restrict__ qr, int64_t ldqr,
                                                         float* __restrict__ sr, int64_t ldsr,
                                                         uint8_t* __restrict__ qc, int64_t ldqc,
                                                         float* __restrict__ sc, int64_t ldsc,
                                                         int64_t col_tiles) {
    __shared__ uint32_t tile[128 * 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l = lane & 15, d = lane >> 4;
    const int64_t g = blockIdx.x / col_tiles;
    const int64_t c0 = (blockIdx.x % col_tiles) * 128;
    const int64_t gc = c0 >> 7;

    uint4 a[4], b[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int64_t r = g * 128 + 32 * p + 8 * wave + 2 * d;
        a[p] = ld_stream16(x + r * ldx + c0 + 8 * l);
        b[p] = ld_stream16(x + (r + 1) * ldx + c0 + 8 * l);
    }
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int64_t r = g * 128 + 32 * p + 8 * wave + 2 * d;
        const GroupScale ga = group_scale(row16_max(absmax8(a[p])), POW2);
        const GroupScale gb = group_scale(row16_max(absmax8(b[p])), POW2);
        st_stream8(qr + r * ldqr + c0 + 8 * l, quant8(a[p], ga.inv));
        st_stream8(qr + (r + 1) * ldqr + c0 + 8 * l, quant8(b[p], gb.inv));
        if (l == 0) {
            sr[gc * ldsr + r] = ga.s;
            sr[gc * ldsr + r + 1] = gb.s;
        }
        const int rp = 16 * p + 4 * wave + d;
        const uint32_t wa[4] = {a[p].x, a[p].y, a[p].z, a[p].w};
        const uint32_t wb[4] = {b[p].x, b[p].y, b[p].z, b[p].w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int c = 8 * l + 2 * j;
            tile[dual_lds_index(c, rp)] = perm(wb[j], wa[j], 0x05040100u);
            tile[dual_lds_index(c + 1, rp)] = perm(wb[j], wa[j], 0x07060302u);
        }
    }
    __syncthreads();

#pragma unroll 2
    for (int it = 0; it < 8; it++) {
        const int c = wave * 32 + it * 4 + d;
        const uint4 v = *(const uint4*)&tile[dual_lds_index(c, 4 * l)];
        const GroupScale gs = group_scale(row16_max(absmax8(v)), POW2);
        st_stream8(qc + (c0 + c) * ldqc + g * 128 + 8 * l, quant8(v, gs.inv));
        if (l == 0) sc[g * ldsc + c0 + c] = gs.s;
    }
}

// ---- backward re-tiling: 1x128 codes -> 128x1 codes ------------------------------------
//
// A workgroup covers one 128 x 128 tile, whose 128 columns share one 1x128
// scale per row.  Thread t reads the 8 x 8 code block at rows 8(t/16)..,
// columns 8(t%16).. (16 lanes read a row's 128 B), transposes it in
// registers and stores it column-major in LDS: column c holds its 128
// codes as 16 chunks of 8 rows, chunk index XOR-swizzled by c/8 so the 16
// lanes of a store hit distinct banks.  Then each 16-lane DPP row takes one
// column at a time: lane l dequantises rows 8l..8l+7 (exact decode, then
// one fp32 multiply by the row's scale), the row reduces the column's
// amax, and the 16 lanes write the 128 new codes as one 128-byte run of
// the transposed output.

// Exact values of the four E4M3 codes packed in a dword (low byte first):
// v_cvt_scalef32_pk_f32_fp8 with scale 1 (every finite code is exact in
// fp32; checked over all codes by the round-trip test of the re-tiling).
__device__ __forceinline__ void decode4(uint32_t w, float (&v)[4]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    const f2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
    v[0] = lo[0];
    v[1] = lo[1];
    v[2] = hi[0];
    v[3] = hi[1];
}

template <bool POW2>
__global__ __launch_bounds__(256) void requant_col_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                          const float* __restrict__ s, int64_t lds,
                                                          uint8_t* __restrict__ qt, int64_t ldqt,
                                                          float* __restrict__ st, int64_t ldst,
                                                          int64_t col_tiles) {
    __shared__ uint2 tile[128 * 16];
    const int t = threadIdx.x;
    // consecutive workgroups: consecutive row groups of one column tile (as
    // in quant_col_kernel)
    const int64_t gt = gridDim.x / col_tiles;
    const int64_t g = blockIdx.x % gt;
    const int64_t c0 = (blockIdx.x / gt) * 128;
    {
        const int rb = t >> 4, cb = t & 15;
        const uint8_t* src = q + (g * 128 + 8 * rb) * ldq + c0 + 8 * cb;
        uint2 r[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const u32x2 w = __builtin_nontemporal_load((const u32x2*)(src + i * ldq));
            r[i] = make_uint2(w.x, w.y);
        }
        uint32_t lo[8], hi[8];  // column j: rows 0-3 in lo[j], rows 4-7 in hi[j]
        transpose4x4(r[0].x, r[1].x, r[2].x, r[3].x, lo[0], lo[1], lo[2], lo[3]);
        transpose4x4(r[4].x, r[5].x, r[6].x, r[7].x, hi[0], hi[1], hi[2], hi[3]);
        transpose4x4(r[0].y, r[1].y, r[2].y, r[3].y, lo[4], lo[5], lo[6], lo[7]);
        transpose4x4(r[4].y, r[5].y, r[6].y, r[7].y, hi[4], hi[5], hi[6], hi[7]);
#pragma unroll
        for (int j = 0; j < 8; j++) tile[(8 * cb + j) * 16 + (rb ^ cb)] = make_uint2(lo[j], hi[j]);
    }
    const int lane = t & 63, wave = t >> 6, l = lane & 15;
    const float* sp = s + (c0 >> 7) * lds + g * 128 + 8 * l;
    const float4 sa = *(const float4*)sp, sb = *(const float4*)(sp + 4);
    const float rs[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    __syncthreads();

#pragma unroll 2
    for (int it = 0; it < 8; it++) {
        const int c = wave * 32 + it * 4 + (lane >> 4);
        const uint2 v = tile[c * 16 + (l ^ (c >> 3))];
        float x[8], d[4];
        decode4(v.x, d);
#pragma unroll
        for (int i = 0; i < 4; i++) x[i] = d[i] * rs[i];
        decode4(v.y, d);
#pragma unroll
        for (int i = 0; i < 4; i++) x[4 + i] = d[i] * rs[4 + i];
        float fam = 0.f;  // max |x| (non-negative, so its bits order like its values)
#pragma unroll
        for (int i = 0; i < 8; i++) fam = fmaxf(fam, fabsf(x[i]));
        const uint32_t am = row16_max(__float_as_uint(fam));
        const GroupScale gs = group_scale(am, POW2);
        const uint2 codes = make_uint2(pack4(x[0] * gs.inv, x[1] * gs.inv, x[2] * gs.inv, x[3] * gs.inv),
                                       pack4(x[4] * gs.inv, x[5] * gs.inv, x[6] * gs.inv, x[7] * gs.inv));
        st_stream8(qt + (c0 + c) * ldqt + g * 128 + 8 * l, codes);
        if (l == 0) st[g * ldst + c0 + c] = gs.s;
    }
}

// ---- launchers -------------------------------------------------------------------------------

hipError_t launch_quant_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                             bool pow2, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (axis == 0) {
        constexpr int RPW = 4;
        const int64_t ct = (cols + 511) / 512, rt = (rows + 4 * RPW - 1) / (4 * RPW);
        const dim3 grid((unsigned)(ct * rt));
        if (pow2)
            hipLaunchKernelGGL((quant_row_kernel<true, RPW>), grid, dim3(256), 0, st, x, rows, cols, ldx, q, ldq, s, lds, ct);
        else
            hipLaunchKernelGGL((quant_row_kernel<false, RPW>), grid, dim3(256), 0, st, x, rows, cols, ldx, q, ldq, s, lds, ct);
    } else {
        const int64_t ct = (cols + 63) / 64, gt = rows / 128;
        const dim3 grid((unsigned)(ct * gt));
        if (pow2)
            hipLaunchKernelGGL(quant_col_kernel<true>, grid, dim3(256), 0, st, x, rows, cols, ldx, q, ldq, s, lds, ct);
        else
            hipLaunchKernelGGL(quant_col_kernel<false>, grid, dim3(256), 0, st, x, rows, cols, ldx, q, ldq, s, lds, ct);
    }
    return hipGetLastError();
}

hipError_t launch_quant_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw, bool pow2,
                              uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s,
                              int64_t lds, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t cb = cols / 128, rb = (rows + 127) / 128;
    const dim3 grid((unsigned)(((cb + 1) / 2) * rb));
    if (pow2)
        hipLaunchKernelGGL(quant_block_kernel<true>, grid, dim3(256), 0, st, w, rows, ldw, q, ldq, qt, ldqt, s, lds, cb);
    else
        hipLaunchKernelGGL(quant_block_kernel<false>, grid, dim3(256), 0, st, w, rows, ldw, q, ldq, qt, ldqt, s, lds, cb);
    return hipGetLastError();
}

hipError_t launch_requant_col(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                              int64_t lds, bool pow2, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                              hipStream_t st_) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t ct = cols / 128, gt = rows / 128;
    const dim3 grid((unsigned)(ct * gt));
    if (pow2)
        hipLaunchKernelGGL(requant_col_kernel<true>, grid, dim3(256), 0, st_, q, ldq, s, lds, qt, ldqt, st, ldst, ct);
    else
        hipLaunchKernelGGL(requant_col_kernel<false>, grid, dim3(256), 0, st_, q, ldq, s, lds, qt, ldqt, st, ldst, ct);
    return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool pow2, uint8_t* qr,
                             int64_t ldqr, float* sr, int64_t ldsr, uint8_t* qc, int64_t ldqc, float* sc,
                             int64_t ldsc, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t ct = cols / 128, gt = rows / 128;
    const dim3 grid((unsigned)(ct * gt));
    if (pow2)
        hipLaunchKernelGGL(quant_dual_kernel<true>, grid, dim3(256), 0, st, x, ldx, qr, ldqr, sr, ldsr, qc, ldqc, sc,
                           ldsc, ct);
    else
        hipLaunchKernelGGL(quant_dual_kernel<false>, grid, dim3(256), 0, st, x, ldx, qr, ldqr, sr, ldsr, qc, ldqc, sc,
                           ldsc, ct);
    return hipGetLastError();
}

hipError_t launch_quant_grouped_col(const uint16_t* x, int64_t T, int64_t cols, int64_t ldx, int G,
                                    const int32_t* offsets, bool pow2, uint8_t* q, int64_t ldq, float* s,
                                    int64_t lds, hipStream_t st) {
    if (cols == 0 || G == 0) return hipSuccess;
    const int64_t ct = (cols + 63) / 64;
    const dim3 grid((unsigned)(ct * G));
    if (pow2)
        hipLaunchKernelGGL(quant_grouped_col_kernel<true>, grid, dim3(256), 0, st, x, cols, ldx, G, offsets, q, ldq,
                           s, lds);
    else
        hipLaunchKernelGGL(quant_grouped_col_kernel<false>, grid, dim3(256), 0, st, x, cols, ldx, G, offsets, q, ldq,
                           s, lds);
    return hipGetLastError();
}

}  // namespace fp8bs
