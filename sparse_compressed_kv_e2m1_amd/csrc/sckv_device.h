// sckv_device.h -- device helpers of the gfx950 kernels: bf16 bits, the e2m1
// grid, the two block-scale rules, and the ABI's host-side error plumbing.
//
// Rules (page "metrale_model_arch/deepseek_v41_ref/compress.rs": E2M1,
// FP4_MAX, to_e2m1_rne, fp4_quant_e8m0_inplace, fp4_quant_e4m3_inplace).
// Every function here is bit-exact by construction: integer bit work, or one
// correctly rounded binary32 operation per step.  The library is compiled
// with -ffp-contract=off so no multiply-add is fused behind our back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "sckv.h"

namespace sckv {

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> bf16 bits, round to nearest, ties to even (finite inputs; NaN
// stays a quiet NaN).  Adding 0x7fff plus the kept LSB and truncating rounds
// the dropped 16 bits half-to-even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------- e2m1 grid

// a = |y| (0 <= a <= 6) rounded to the nearest point of the e2m1 grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}, exact ties going to the even code (codes 0..7
// in grid order).
// The grid is the multiples of 0.5 below 2, of 1 in [2, 4) and of 2 from 4
// on, and at every midpoint the even code is the even multiple of that
// spacing (.25 -> 0, .75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
// 5 -> 4).  Adding and subtracting 1.5 * 2^(23 + log2 spacing) rounds a to a
// multiple of the spacing, half to even, in one binary32 add (exact
// otherwise).
__device__ __forceinline__ float e2m1_round_mag(float a) {
    const float m = (a < 2.0f) ? 0x1.8p22f : ((a < 4.0f) ? 0x1.8p23f : 0x1.8p24f);
    return (a + m) - m;
}

// ---------------------------------------------------------------- scale rules

// Power-of-two ceiling of a normal positive binary32 x (x >= 2^-126 here
// thanks to the amax floor, and x < 2^126 for any finite bf16 amax / 6).
__device__ __forceinline__ float pow2_ceil_normal(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x007fffffu) == 0u) return x;
    return __uint_as_float((u & 0x7f800000u) + 0x00800000u);
}

// x >= 0 rounded to the nearest OCP E4M3FN value (ties to the even code),
// saturating at 448.  Subnormal range (x < 2^-6): multiples of 2^-9, rounded
// with rintf (half-to-even) on the exactly scaled value.  Normal range: keep
// 3 mantissa bits with half-to-even on the binary32 bits (a carry moves to the
// next binade, which is the correct rounding).
__device__ __forceinline__ float e4m3_round_nonneg(float x) {
    if (x < 0.015625f) {
        float q = rintf(x * 512.0f);
        return q * 0.001953125f;
    }
    uint32_t u = __float_as_uint(x);
    u += 0x7ffffu + ((u >> 20) & 1u);
    u &= 0xfff00000u;
    float r = __uint_as_float(u);
    return fminf(r, 448.0f);
}

// Block scale for the two modes from the block's amax (binary32).
template <int MODE>
__device__ __forceinline__ float block_scale(float amax) {
    if (MODE == SCKV_FP4_E8M0_B32) {
        const float floor_amax = 0x1.8p-124f;  // 6 * 2^-126
        amax = fmaxf(amax, floor_amax);
        return pow2_ceil_normal(__fdiv_rn(amax, 6.0f));
    } else {
        const float floor_amax = 0x1.8p-7f;  // 6 * 2^-9
        amax = fmaxf(amax, floor_amax);
        return e4m3_round_nonneg(__fdiv_rn(amax, 6.0f));
    }
}

// e2m1 * s is exact in bf16 for both scale kinds (at most 2 + 4 significant
// bits, exponent within range), so the conversion is a truncation; the sign of
// v is put back afterwards (small negative values give -0).
__device__ __forceinline__ uint32_t signed_bf16_bits(float r, float v) {
    return (__float_as_uint(r) | (__float_as_uint(v) & 0x80000000u)) >> 16;
}

// One value of a block: bf16 bits of e2m1(clamp(v / s, -6, 6)) * s.  The
// quotient is the correctly rounded binary32 division (true division, not a
// reciprocal multiply: the two differ on some exact e2m1 midpoints); |v| / s
// is |v / s| since division is sign-symmetric.
__device__ __forceinline__ uint32_t fp4_value_bits(float v, float s) {
    const float a = fminf(__fdiv_rn(fabsf(v), s), 6.0f);
    return signed_bf16_bits(e2m1_round_mag(a) * s, v);
}

// Exact reciprocal of a power of two 2^-126 <= s <= 2^126 (exponent flip).
__device__ __forceinline__ float pow2_reciprocal(float s) {
    return __uint_as_float((254u - ((__float_as_uint(s) >> 23) & 0xffu)) << 23);
}

// The same value as fp4_value_bits(v, s) when s is a power of two: |v| * (1/s)
// rounds the same exact real number |v| / s once (1/s is exact), so the bits
// are identical, subnormal quotients included, and no division is needed.
__device__ __forceinline__ uint32_t fp4_value_bits_pow2(float v, float s, float inv_s) {
    const float a = fminf(fabsf(v) * inv_s, 6.0f);
    return signed_bf16_bits(e2m1_round_mag(a) * s, v);
}

// One value of a block in either mode (inv_s only used for power-of-two scales).
template <int MODE>
__device__ __forceinline__ uint32_t fp4_value(float v, float s, float inv_s) {
    if (MODE == SCKV_FP4_E8M0_B32) return fp4_value_bits_pow2(v, s, inv_s);
    return fp4_value_bits(v, s);
}

// ---------------------------------------------------------------- packed storage

// 4-bit code of a value of the round trip: the e2m1 grid index of its
// magnitude r (r / s, one of 0, .5, 1, 1.5, 2, 3, 4, 6) plus 8 when v is
// negative (the round trip keeps the sign of v, -0 included).
__device__ __forceinline__ uint32_t e2m1_code(float r, float v) {
    const uint32_t idx = (r < 2.0f) ? (uint32_t)(r * 2.0f) : ((r < 4.0f) ? (uint32_t)r + 2u : ((r < 5.0f) ? 6u : 7u));
    return idx | ((__float_as_uint(v) >> 28) & 8u);
}

// Scale byte of a block: the E8M0 exponent of a power-of-two scale, or the
// E4M3FN code of an e4m3 scale (s is exactly representable in either case).
template <int MODE>
__device__ __forceinline__ uint32_t scale_byte(float s) {
    const uint32_t u = __float_as_uint(s);
    if (MODE == SCKV_FP4_E8M0_B32) return (u >> 23) & 0xffu;
    if (s < 0.015625f) return (uint32_t)(s * 512.0f);  // subnormal: s = code * 2^-9
    return ((((u >> 23) & 0xffu) - 120u) << 3) | ((u >> 20) & 7u);
}

template <int MODE>
struct QuantMode;
template <>
struct QuantMode<SCKV_FP4_E4M3_B16> {
    static constexpr int BLOCK = 16;
};
template <>
struct QuantMode<SCKV_FP4_E8M0_B32> {
    static constexpr int BLOCK = 32;
};

// The round trip of one block held as bf16 pairs (w[i]: value 2i in the low
// half, 2i + 1 in the high half), in place.
template <int MODE>
__device__ __forceinline__ void quant_block(uint32_t (&w)[QuantMode<MODE>::BLOCK / 2]) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BLOCK / 2; ++i) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
    const float s = block_scale<MODE>(amax);
    const float inv_s = (MODE == SCKV_FP4_E8M0_B32) ? pow2_reciprocal(s) : 0.0f;
#pragma unroll
    for (int i = 0; i < BLOCK / 2; ++i) {
        const uint32_t lo = fp4_value<MODE>(bf16_bits_to_f32(w[i] & 0xffffu), s, inv_s);
        const uint32_t hi = fp4_value<MODE>(bf16_bits_to_f32(w[i] >> 16), s, inv_s);
        w[i] = lo | (hi << 16);
    }
}

// The packed form of one block (same input layout): BLOCK/8 code words (byte
// j holds the codes of values 2j, low nibble, and 2j + 1) and the scale byte,
// returned.
template <int MODE>
__device__ __forceinline__ uint32_t pack_block(const uint32_t (&w)[QuantMode<MODE>::BLOCK / 2],
                                               uint32_t (&cw)[QuantMode<MODE>::BLOCK / 8]) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BLOCK / 2; ++i) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
    const float s = block_scale<MODE>(amax);
    const float inv_s = (MODE == SCKV_FP4_E8M0_B32) ? pow2_reciprocal(s) : 0.0f;
#pragma unroll
    for (int i = 0; i < BLOCK / 8; ++i) cw[i] = 0;
#pragma unroll
    for (int i = 0; i < BLOCK; ++i) {
        const float v = bf16_bits_to_f32((i & 1) ? (w[i / 2] >> 16) : (w[i / 2] & 0xffffu));
        const float a = (MODE == SCKV_FP4_E8M0_B32) ? fminf(fabsf(v) * inv_s, 6.0f) : fminf(__fdiv_rn(fabsf(v), s), 6.0f);
        cw[i / 8] |= e2m1_code(e2m1_round_mag(a), v) << (4 * (i % 8));
    }
    return scale_byte<MODE>(s);
}

// ---------------------------------------------------------------- rotary turn

// Rotary turn of one pair (x0, x1) of a row's rope slice by the table entry
// (c, s) (pages: compress.rs attention_any and forward.rs AttnV41::forward
// rotate a new latent group before its fp4 round trip; the rotation itself is
// not printed -- the reading is x0 + i x1 times c + i s): binary32 products and
// sums, no fused multiply-add (the library is built with -ffp-contract=off),
// each result rounded to bf16.  w holds x0 in the low half, x1 in the high.
__device__ __forceinline__ uint32_t rope_pair_bits(uint32_t w, float c, float s) {
    const float x0 = bf16_bits_to_f32(w & 0xffffu), x1 = bf16_bits_to_f32(w >> 16);
    const float y0 = x0 * c - x1 * s;
    const float y1 = x0 * s + x1 * c;
    return f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
}

// Row of position q inside rows_a (the layout sckv_rows_a_len describes).
__device__ __forceinline__ int64_t window_row(int win, int64_t m, int64_t start_pos, int64_t q) {
    if (start_pos == 0) return q;
    if (m == 1) return q % win;
    return (q < start_pos) ? (q % win) : (win + (q - start_pos));
}

// Column j of query t's window part of the index list: the j-th oldest of the
// n_w = min(win, p + 1) positions ending at p = start_pos + t, as its row in
// rows_a, then -1 (forward.rs window_topk_idxs; reading in sckv_window_idx).
__device__ __forceinline__ int32_t window_col(int win, int64_t m, int64_t start_pos, int64_t t, int j) {
    const int64_t p = start_pos + t;
    const int64_t n_w = (p + 1 < win) ? (p + 1) : win;
    return (j < n_w) ? (int32_t)window_row(win, m, start_pos, p - n_w + 1 + j) : -1;
}

// Column j of query t's compressed part on a layer without an indexer:
// offset + j for the V_p = min(n_c, (p + 1) / ratio) visible compressed rows,
// then -1.
__device__ __forceinline__ int32_t visible_col(int64_t start_pos, int ratio, int64_t n_c, int32_t offset, int64_t t,
                                               int j) {
    int64_t v = (start_pos + t + 1) / ratio;
    v = v < n_c ? v : n_c;
    return (j < v) ? (int32_t)(offset + j) : -1;
}

// ---------------------------------------------------------------- host side

void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int check_launch(const char* what);

}  // namespace sckv
