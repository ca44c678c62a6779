// quant.hip -- the fp4 (e2m1) round trip over bf16 rows (page
// "metrale_model_arch/deepseek_v41_ref/compress.rs": fp4_quant_e8m0_inplace,
// fp4_quant_e4m3_inplace; page "metrale_model_arch/attn_v41/forward.rs": the
// fp4_quant of the new latent groups before the cache copy).
//
// HBM-bound: one lane owns one block (16 or 32 values = 32 or 64 bytes), reads
// it with 16-byte loads, and writes it back with 16-byte stores; neighbouring
// lanes own neighbouring blocks, so a wave streams 2 or 4 KiB contiguously.
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

// Checks of a rotation table and the rows' positions (every row's position
// pos0 + r * pos_step inside the table).
int rope_checks(const char* name, int64_t rows, int64_t cols, const float* table, int64_t n_pos, int rope_dim,
                int64_t pos0, int64_t pos_step) {
    if (n_pos < 0 || pos0 < 0 || pos_step < 0) return fail(SCKV_EINVAL, std::string(name) + ": negative position");
    if (rope_dim <= 0 || rope_dim % 2 != 0 || rope_dim > cols)
        return fail(SCKV_EINVAL, std::string(name) + ": rope_dim must be even, positive and at most the row length");
    if (!table || (uintptr_t)table % 8)
        return fail(SCKV_EINVAL, std::string(name) + ": null or misaligned (8 bytes) rotation table");
    if (rows > 0 && pos0 + (rows - 1) * pos_step >= n_pos)
        return fail(SCKV_EINVAL, std::string(name) + ": a row's position is outside the rotation table");
    return SCKV_OK;
}

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

template <int MODE, bool VEC, bool ROPE = false>
__global__ __launch_bounds__(QUANT_THREADS) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                    uint16_t* __restrict__ y, int64_t ldy,
                                                                    int64_t blocks_per_row, int64_t nblocks,
                                                                    RopeArgs rope = RopeArgs{}) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    const int64_t gid = (int64_t)blockIdx.x * QUANT_THREADS + threadIdx.x;
    if (gid >= nblocks) return;
    const int64_t row = gid / blocks_per_row;
    const int64_t col = (gid - row * blocks_per_row) * BLOCK;
    const uint16_t* src = x + row * ldx + col;
    uint16_t* dst = y + row * ldy + col;

    uint32_t w[BLOCK / 2];  // bf16 pairs, low half = lower index
    if (VEC) {
#pragma unroll
        for (int i = 0; i < BLOCK / 8; ++i) {
            uint4 v = reinterpret_cast<const uint4*>(src)[i];
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BLOCK / 2; ++i) w[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
    }
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

template <int MODE>
int launch_quant(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int64_t rows, int64_t cols,
                 hipStream_t stream) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    const int64_t bpr = cols / BLOCK;
    const int64_t nblocks = rows * bpr;
    if (nblocks == 0) return SCKV_OK;
    const int64_t grid = (nblocks + QUANT_THREADS - 1) / QUANT_THREADS;
    if (grid > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_quant: too many blocks for one launch");
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0) && (ldx % 8 == 0) && (ldy % 8 == 0);
    if (vec)
        quant_rows_kernel<MODE, true><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, stream>>>(x, ldx, y, ldy, bpr,
                                                                                                  nblocks);
    else
        quant_rows_kernel<MODE, false><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, stream>>>(x, ldx, y, ldy,
                                                                                                   bpr, nblocks);
    return check_launch("sckv_quant");
}

int quant_rows_impl(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols, int mode,
                    void* stream) {
    if (mode != SCKV_FP4_E4M3_B16 && mode != SCKV_FP4_E8M0_B32) return fail(SCKV_EINVAL, "sckv_quant: bad mode");
    const int block = (mode == SCKV_FP4_E4M3_B16) ? 16 : 32;
    if (rows < 0 || cols < 0) return fail(SCKV_EINVAL, "sckv_quant: negative size");
    if (cols % block != 0) return fail(SCKV_EINVAL, "sckv_quant: row length is not a multiple of the block");
    if (rows == 0 || cols == 0) return SCKV_OK;
    if (!x || !y) return fail(SCKV_EINVAL, "sckv_quant: null pointer");
    if (ldx < cols || ldy < cols) return fail(SCKV_EINVAL, "sckv_quant: row stride shorter than the row");
    if ((uintptr_t)x % 2 || (uintptr_t)y % 2) return fail(SCKV_EINVAL, "sckv_quant: pointer not 2-byte aligned");
    if (x != y) {
        // ranges [x, x + span) and [y, y + span) must not overlap
        const uintptr_t xs = (uintptr_t)x, ys = (uintptr_t)y;
        const uintptr_t xe = xs + (uintptr_t)(((rows - 1) * ldx + cols) * 2);
        const uintptr_t ye = ys + (uintptr_t)(((rows - 1) * ldy + cols) * 2);
        if (xs < ye && ys < xe) return fail(SCKV_EINVAL, "sckv_quant: x and y overlap without being equal");
    } else if (ldx != ldy) {
        return fail(SCKV_EINVAL, "sckv_quant: in place needs ldx == ldy");
    }
    hipStream_t s = (hipStream_t)stream;
    if (mode == SCKV_FP4_E4M3_B16)
        return launch_quant<SCKV_FP4_E4M3_B16>((const uint16_t*)x, ldx, (uint16_t*)y, ldy, rows, cols, s);
    return launch_quant<SCKV_FP4_E8M0_B32>((const uint16_t*)x, ldx, (uint16_t*)y, ldy, rows, cols, s);
}

// The latent path of new compressed rows: rotation of the rope slice, then
// the E4M3_B16 round trip, one lane per block of 16.
int rope_quant_rows_impl(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                         const float* table, int64_t n_pos, int rope_dim, int64_t pos0, int64_t pos_step,
                         void* stream) {
    const char* name = "sckv_rope_quant_rows";
    if (rows < 0 || cols < 0) return fail(SCKV_EINVAL, std::string(name) + ": negative size");
    if (cols % 16 != 0) return fail(SCKV_EINVAL, std::string(name) + ": row length is not a multiple of 16");
    if (const int rc = rope_checks(name, rows, cols, table, n_pos, rope_dim, pos0, pos_step)) return rc;
    if (rows == 0 || cols == 0) return SCKV_OK;
    if (!x || !y) return fail(SCKV_EINVAL, std::string(name) + ": null pointer");
    if (ldx < cols || ldy < cols) return fail(SCKV_EINVAL, std::string(name) + ": row stride shorter than the row");
    if ((uintptr_t)x % 2 || (uintptr_t)y % 2)
        return fail(SCKV_EINVAL, std::string(name) + ": misaligned pointer (bf16 rows 2 bytes)");
    if (x != y) {
        const uintptr_t xs = (uintptr_t)x, ys = (uintptr_t)y;
        const uintptr_t xe = xs + (uintptr_t)(((rows - 1) * ldx + cols) * 2);
        const uintptr_t ye = ys + (uintptr_t)(((rows - 1) * ldy + cols) * 2);
        if (xs < ye && ys < xe) return fail(SCKV_EINVAL, std::string(name) + ": x and y overlap without being equal");
    } else if (ldx != ldy) {
        return fail(SCKV_EINVAL, std::string(name) + ": in place needs ldx == ldy");
    }
    const int64_t bpr = cols / 16, nblocks = rows * bpr;
    const int64_t grid = (nblocks + QUANT_THREADS - 1) / QUANT_THREADS;
    if (grid > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": too many blocks for one launch");
    const RopeArgs r{table, rope_dim, pos0, pos_step};
    const uint16_t* xx = (const uint16_t*)x;
    uint16_t* yy = (uint16_t*)y;
    hipStream_t s = (hipStream_t)stream;
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0) && (ldx % 8 == 0) && (ldy % 8 == 0);
    if (vec)
        quant_rows_kernel<SCKV_FP4_E4M3_B16, true, true><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, s>>>(
            xx, ldx, yy, ldy, bpr, nblocks, r);
    else
        quant_rows_kernel<SCKV_FP4_E4M3_B16, false, true><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, s>>>(
            xx, ldx, yy, ldy, bpr, nblocks, r);
    return check_launch(name);
}

// ---- packed storage: 4-bit codes (two a byte, the even element low) and one
// scale byte per block; one lane per block, as above.
template <int MODE, bool ROPE = false>
__global__ __launch_bounds__(QUANT_THREADS) void quant_pack_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                    uint8_t* __restrict__ codes, int64_t ldc,
                                                                    uint8_t* __restrict__ scales, int64_t lds,
                                                                    int64_t blocks_per_row, int64_t nblocks,
                                                                    bool vec, RopeArgs rope = RopeArgs{}) {
    constexpr int BLOCK = QuantMode<MODE>::BLOCK;
    const int64_t gid = (int64_t)blockIdx.x * QUANT_THREADS + threadIdx.x;
    if (gid >= nblocks) return;
    const int64_t row = gid / blocks_per_row;
    const int64_t blk = gid - row * blocks_per_row;
    const uint16_t* src = x + row * ldx + blk * BLOCK;
    uint32_t w[BLOCK / 2];
    if (vec) {
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
    if (ROPE) rope_block<BLOCK>(w, row, blk * BLOCK, blocks_per_row * BLOCK, rope);
    // BLOCK/2 bytes of codes: byte i holds elements 2i (low) and 2i+1 (high)
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

}  // namespace

int quant_pack_launch(const void* x, int64_t ldx, void* codes, int64_t ldc, void* scales, int64_t lds, int64_t rows,
                      int64_t cols, int mode, void* stream, const RopeArgs* rope = nullptr) {
    if (mode != SCKV_FP4_E4M3_B16 && mode != SCKV_FP4_E8M0_B32) return fail(SCKV_EINVAL, "sckv_quant_pack: bad mode");
    const int block = (mode == SCKV_FP4_E4M3_B16) ? 16 : 32;
    if (rows < 0 || cols < 0) return fail(SCKV_EINVAL, "sckv_quant_pack: negative size");
    if (cols % block != 0) return fail(SCKV_EINVAL, "sckv_quant_pack: row length is not a multiple of the block");
    if (rows == 0 || cols == 0) return SCKV_OK;
    if (!x || !codes || !scales) return fail(SCKV_EINVAL, "sckv_quant_pack: null pointer");
    if (ldx < cols || ldc < cols / 2 || lds < cols / block)
        return fail(SCKV_EINVAL, "sckv_quant_pack: a row stride is shorter than its row");
    if ((uintptr_t)x % 2) return fail(SCKV_EINVAL, "sckv_quant_pack: x not 2-byte aligned");
    const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(((rows - 1) * ldx + cols) * 2);
    const uintptr_t cs = (uintptr_t)codes, ce = cs + (uintptr_t)((rows - 1) * ldc + cols / 2);
    const uintptr_t ss = (uintptr_t)scales, se = ss + (uintptr_t)((rows - 1) * lds + cols / block);
    if ((xs < ce && cs < xe) || (xs < se && ss < xe) || (cs < se && ss < ce))
        return fail(SCKV_EINVAL, "sckv_quant_pack: x, codes and scales overlap");
    const int64_t bpr = cols / block;
    const int64_t nblocks = rows * bpr;
    const int64_t grid = (nblocks + QUANT_THREADS - 1) / QUANT_THREADS;
    if (grid > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_quant_pack: too many blocks for one launch");
    const bool vec = (xs % 16 == 0) && (ldx % 8 == 0) && (cs % (block / 2) == 0) && (ldc % (block / 2) == 0);
    hipStream_t s = (hipStream_t)stream;
    if (rope)  // the latent: rotation, then the e4m3-scale round trip
        quant_pack_kernel<SCKV_FP4_E4M3_B16, true><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, s>>>(
            (const uint16_t*)x, ldx, (uint8_t*)codes, ldc, (uint8_t*)scales, lds, bpr, nblocks, vec, *rope);
    else if (mode == SCKV_FP4_E4M3_B16)
        quant_pack_kernel<SCKV_FP4_E4M3_B16><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, s>>>(
            (const uint16_t*)x, ldx, (uint8_t*)codes, ldc, (uint8_t*)scales, lds, bpr, nblocks, vec);
    else
        quant_pack_kernel<SCKV_FP4_E8M0_B32><<<dim3((unsigned)grid), dim3(QUANT_THREADS), 0, s>>>(
            (const uint16_t*)x, ldx, (uint8_t*)codes, ldc, (uint8_t*)scales, lds, bpr, nblocks, vec);
    return check_launch("sckv_quant_pack");
}


}  // namespace sckv

extern "C" int sckv_quant(const void* x, void* y, int64_t n, int mode, void* stream) {
    if (n < 0) return sckv::fail(SCKV_EINVAL, "sckv_quant: negative n");
    if (mode != SCKV_FP4_E4M3_B16 && mode != SCKV_FP4_E8M0_B32)
        return sckv::fail(SCKV_EINVAL, "sckv_quant: bad mode");
    const int block = (mode == SCKV_FP4_E4M3_B16) ? 16 : 32;
    if (n % block != 0) return sckv::fail(SCKV_EINVAL, "sckv_quant: n is not a multiple of the block");
    // a flat array is one row of n values
    return sckv::quant_rows_impl(x, n, y, n, n ? 1 : 0, n, mode, stream);
}

extern "C" int sckv_quant_rows(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                               int mode, void* stream) {
    return sckv::quant_rows_impl(x, ldx, y, ldy, rows, cols, mode, stream);
}

extern "C" int sckv_quant_pack(const void* x, int64_t ldx, void* codes, int64_t ldc, void* scales, int64_t lds,
                               int64_t rows, int64_t cols, int mode, void* stream) {
    return sckv::quant_pack_launch(x, ldx, codes, ldc, scales, lds, rows, cols, mode, stream);
}

extern "C" int sckv_rope_quant_rows(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                                    const float* table, int64_t n_pos, int rope_dim, int64_t pos0, int64_t pos_step,
                                    void* stream) {
    return sckv::rope_quant_rows_impl(x, ldx, y, ldy, rows, cols, table, n_pos, rope_dim, pos0, pos_step, stream);
}

extern "C" int sckv_rope_quant_pack(const void* x, int64_t ldx, void* codes, int64_t ldc, void* scales, int64_t lds,
                                    int64_t rows, int64_t cols, const float* table, int64_t n_pos, int rope_dim,
                                    int64_t pos0, int64_t pos_step, void* stream) {
    using namespace sckv;
    const char* name = "sckv_rope_quant_pack";
    if (rows < 0 || cols < 0) return fail(SCKV_EINVAL, std::string(name) + ": negative size");
    if (cols % 16 != 0) return fail(SCKV_EINVAL, std::string(name) + ": row length is not a multiple of 16");
    if (const int rc = rope_checks(name, rows, cols, table, n_pos, rope_dim, pos0, pos_step)) return rc;
    const RopeArgs r{table, rope_dim, pos0, pos_step};
    return quant_pack_launch(x, ldx, codes, ldc, scales, lds, rows, cols, SCKV_FP4_E4M3_B16, stream, &r);
}
