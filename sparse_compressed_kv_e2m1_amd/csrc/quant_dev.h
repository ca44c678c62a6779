// quant_dev.h -- device code of the fp4 (e2m1) round trip over bf16 rows and
// of its packed storage, one lane per block of 16 (e4m3 scale) or 32
// (power-of-two scale) values, as bodies that take the lane's block number:
// the kernels of quant.hip run them over a whole launch, the prefill set-up
// (prefill.hip) over one range of its workgroups.
//
// Page "metrale_model_arch/deepseek_v41_ref/compress.rs": fp4_quant_e8m0_inplace,
// fp4_quant_e4m3_inplace, and the rotation of a new latent group before its
// round trip (attention_any).
#pragma once

#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int QUANT_THREADS = 256;

// rows x cols values, row strides ldx / ldy (elements); cols % BLOCK == 0.
// VEC: every block is 16-byte aligned in x and y (checked on the host).
// Rotation before the round trip (ROPE): the last rope_dim values of row r
// turn by the table row of position pos0 + r * pos_step (table [n_pos]
// [rope_dim / 2] pairs of binary32 cos, sin; pair i = values cols - rope_dim
// + 2i, + 2i + 1), each turned pair rounded to bf16 first.
struct RopeArgs {
    const float* table;
    int rope_dim;
    int64_t pos0, pos_step;
};

// The rotary turn of the pairs of one block (values col .. col + BLOCK - 1 of
// row `row`, held as bf16 pairs) that fall in the rope slice.
template <int BLOCK>
__device__ __forceinline__ void rope_block(uint32_t (&w)[BLOCK / 2], int64_t row, int64_t col, int64_t cols,
                                           const RopeArgs& rope) {
    const int64_t first = cols - rope.rope_dim;  // first value of the rope slice (even)
    if (col + BLOCK <= first) return;
    const int half = rope.rope_dim / 2;
    const float2* t = reinterpret_cast<const float2*>(rope.table) + (rope.pos0 + row * rope.pos_step) * half;
#pragma unroll
    for (int k = 0; k < BLOCK / 2; ++k) {
        const int64_t c = col + 2 * k;
        if (c >= first) {
            const float2 cs = t[(c - first) / 2];
            w[k] = rope_pair_bits(w[k], cs.x, cs.y);
        }
    }
}

// A block's BLOCK values as bf16 pairs (low half = lower index).
template <int BLOCK, bool VEC>
__device__ __forceinline__ void load_block(const uint16_t* src, uint32_t (&w)[BLOCK / 2]) {
    if (VEC) {
#pragma unroll
        for (int i = 0; i < BLOCK / 8; ++i) {
            const uint4 v = reinterpret_cast<const uint4*>(src)[i];
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BLOCK / 2; ++i) w[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
    }
}

// Block gid (row gid / blocks_per_row) of x round-tripped into y.
template <int MODE, bool VEC, bool ROPE>
__device__ __forceinline__ void quant_rows_block(const uint16_t* __restrict__ x, int64_t ldx,
                                                 uint16_t* __restrict__ y, int64_t ldy, int64_t blocks_per_row,
                                                 int64_t gid, const RopeArgs& rope) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    const int64_t row = gid / blocks_per_row;
    const int64_t col = (gid - row * blocks_per_row) * BLOCK;
    uint16_t* dst = y + row * ldy + col;
    uint32_t w[BLOCK / 2];
    load_block<BLOCK, VEC>(x + row * ldx + col, w);
    if (ROPE) rope_block<BLOCK>(w, row, col, blocks_per_row * BLOCK, rope);
    quant_block<MODE>(w);
    if (VEC) {
#pragma unroll
        for (int i = 0; i < BLOCK / 8; ++i)
            reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < BLOCK / 2; ++i) {
            dst[2 * i] = (uint16_t)(w[i] & 0xffffu);
            dst[2 * i + 1] = (uint16_t)(w[i] >> 16);
        }
    }
}

// Block gid of x stored packed: BLOCK/2 bytes of 4-bit codes (byte i holds
// elements 2i (low) and 2i + 1 (high)) and one scale byte.  vec: x's blocks
// 16-byte aligned and each code block aligned to its size.
template <int MODE, bool ROPE>
__device__ __forceinline__ void quant_pack_block(const uint16_t* __restrict__ x, int64_t ldx,
                                                 uint8_t* __restrict__ codes, int64_t ldc,
                                                 uint8_t* __restrict__ scales, int64_t lds, int64_t blocks_per_row,
                                                 int64_t gid, bool vec, const RopeArgs& rope) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    const int64_t row = gid / blocks_per_row;
    const int64_t blk = gid - row * blocks_per_row;
    const uint16_t* src = x + row * ldx + blk * BLOCK;
    uint32_t w[BLOCK / 2];
    if (vec)
        load_block<BLOCK, true>(src, w);
    else
        load_block<BLOCK, false>(src, w);
    if (ROPE) rope_block<BLOCK>(w, row, blk * BLOCK, blocks_per_row * BLOCK, rope);
    uint32_t cw[BLOCK / 8];
    const uint32_t sbyte = pack_block<MODE>(w, cw);
    uint8_t* cdst = codes + row * ldc + blk * (BLOCK / 2);
    if (vec) {
        if (BLOCK == 32)
            *reinterpret_cast<uint4*>(cdst) = make_uint4(cw[0], cw[BLOCK / 8 > 1 ? 1 : 0], cw[BLOCK / 8 > 2 ? 2 : 0],
                                                         cw[BLOCK / 8 > 3 ? 3 : 0]);
        else
            *reinterpret_cast<uint2*>(cdst) = make_uint2(cw[0], cw[BLOCK / 8 > 1 ? 1 : 0]);
    } else {
#pragma unroll
        for (int i = 0; i < BLOCK / 2; ++i) cdst[i] = (uint8_t)(cw[i / 4] >> (8 * (i % 4)));
    }
    scales[row * lds + blk] = (uint8_t)sbyte;
}

// Checks of a rotation table and the rows' positions (every row's position
// pos0 + r * pos_step inside the table).
inline int rope_checks(const char* name, int64_t rows, int64_t cols, const float* table, int64_t n_pos,
                       int rope_dim, int64_t pos0, int64_t pos_step) {
    if (n_pos < 0 || pos0 < 0 || pos_step < 0) return fail(SCKV_EINVAL, std::string(name) + ": negative position");
    if (rope_dim <= 0 || rope_dim % 2 != 0 || rope_dim > cols)
        return fail(SCKV_EINVAL, std::string(name) + ": rope_dim must be even, positive and at most the row length");
    if (!table || (uintptr_t)table % 8)
        return fail(SCKV_EINVAL, std::string(name) + ": null or misaligned (8 bytes) rotation table");
    if (rows > 0 && pos0 + (rows - 1) * pos_step >= n_pos)
        return fail(SCKV_EINVAL, std::string(name) + ": a row's position is outside the rotation table");
    return SCKV_OK;
}

}  // namespace
}  // namespace sckv
