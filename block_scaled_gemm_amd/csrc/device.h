// device.h -- gfx950 device helpers shared by the quantisation and GEMM
// kernels: bf16 unpacking, the E4M3 rounding step, group-scale derivation,
// 16-lane DPP reductions and byte transposes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// ---- bf16 --------------------------------------------------------------------

// The two bf16 values packed in a dword, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- E4M3 rounding -------------------------------------------------------------
//
// Code of the E4M3 value nearest to y, ties to the even code, |y| >= 448
// saturating to 448, sign copied (so values rounding to zero keep it).
// v_cvt_pk_fp8_f32 rounds to nearest even into OCP E4M3; clamping to
// [-448, 448] first (v_med3_f32) gives the saturation.  Checked against the
// CPU oracle's encoder over every finite fp32 bit pattern.
__device__ __forceinline__ float sat448(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }

__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const float c = sat448(y);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Four codes packed little-endian into a dword.
__device__ __forceinline__ uint32_t pack4(float y0, float y1, float y2, float y3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(y0), sat448(y1), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(y2), sat448(y3), lo, true);
}

// Quantise the 8 bf16 values of a uint4 (two per dword) with factor inv;
// returns 8 codes in a uint2.
__device__ __forceinline__ uint2 quant8(uint4 v, float inv) {
    uint2 r;
    r.x = pack4(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
    r.y = pack4(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
    return r;
}

// ---- group scale -----------------------------------------------------------------
//
// amax_bits: bit pattern of the group's max |x| (a bf16 value widened to
// fp32, so its low 16 bits are zero).  The amax is floored at
// 448 * 2^-126 = 1.75 * 2^-118 (bits 0x04E00000) so that s stays normal and
// inv finite.
//   FP32 mode: s = amax / 448, inv = 448 / amax (IEEE divisions).
//   POW2 mode: s = 2^k with k the smallest integer such that amax <= 448*2^k:
//     amax = m * 2^E, m in [1, 2): k = E - 8, plus 1 when m > 1.75.
constexpr uint32_t kAmaxFloorBits = 0x04E00000u;

struct GroupScale {
    float s;
    float inv;
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits, bool pow2) {
    const uint32_t ab = amax_bits > kAmaxFloorBits ? amax_bits : kAmaxFloorBits;
    GroupScale g;
    if (pow2) {
        const int e = (int)(ab >> 23) - 127;
        const int k = e - 8 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);
        g.s = __uint_as_float((uint32_t)(k + 127) << 23);
        g.inv = __uint_as_float((uint32_t)(127 - k) << 23);
    } else {
        const float a = __uint_as_float(ab);
        g.s = a / 448.0f;
        g.inv = 448.0f / a;
    }
    return g;
}

// ---- |bf16| maxima on packed pairs --------------------------------------------------
//
// For non-negative floats the ordering of the bit patterns is the ordering
// of the values, so the max |x| of bf16 data is an unsigned 16-bit max of
// the patterns with the sign bit cleared.

// Per-half maximum of two packed pairs of |bf16| patterns.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 x = __builtin_bit_cast(us2, a);
    us2 y = __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Max |x| pattern (in the low 16 bits' units, returned as an fp32 pattern)
// over the 8 bf16 values of a uint4.
__device__ __forceinline__ uint32_t absmax8(uint4 v) {
    const uint32_t m = 0x7FFF7FFFu;
    uint32_t p = pk_max_u16(pk_max_u16(v.x & m, v.y & m), pk_max_u16(v.z & m, v.w & m));
    uint32_t lo = p & 0xFFFFu, hi = p >> 16;
    return (lo > hi ? lo : hi) << 16;
}

// ---- 16-lane reductions (one DPP row) ---------------------------------------------------
//
// Max over the 16 lanes of each DPP row; every lane of the row gets the
// result.  Butterfly: swap neighbours, swap pairs (quad_perm), mirror each
// half-row, mirror the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max(v, dpp<0x141>(v));  // row_half_mirror
    v = max(v, dpp<0x140>(v));  // row_mirror
    return v;
}

// Max over the whole wave (64 lanes); every lane gets the result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = row16_max(v);
    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// ---- byte transposes ---------------------------------------------------------------------
//
// v_perm_b32 picks 4 bytes out of 8: selector byte values 0-3 take bytes of
// the second operand, 4-7 bytes of the first.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4x4 byte transpose: r[i] byte j -> c[j] byte i.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3) {
    const uint32_t t0 = perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
    const uint32_t t1 = perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
    const uint32_t t2 = perm(r3, r2, 0x05010400u);
    const uint32_t t3 = perm(r3, r2, 0x07030602u);
    c0 = perm(t2, t0, 0x05040100u);
    c1 = perm(t2, t0, 0x07060302u);
    c2 = perm(t3, t1, 0x05040100u);
    c3 = perm(t3, t1, 0x07060302u);
}

}  // namespace fp8bs
