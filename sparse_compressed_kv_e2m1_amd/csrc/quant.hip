// quant.hip -- the fp4 (e2m1) round trip over bf16 rows (page
// "metrale_model_arch/deepseek_v41_ref/compress.rs": fp4_quant_e8m0_inplace,
// fp4_quant_e4m3_inplace; page "metrale_model_arch/attn_v41/forward.rs": the
// fp4_quant of the new latent groups before the cache copy).
//
// HBM-bound: one lane owns one block (16 or 32 values = 32 or 64 bytes), reads
// it with 16-byte loads, and writes it back with 16-byte stores; neighbouring
// lanes own neighbouring blocks, so a wave streams 2 or 4 KiB contiguously.
#include "quant_dev.h"

namespace sckv {
namespace {

template <int MODE, bool VEC, bool ROPE = false>
__global__ __launch_bounds__(QUANT_THREADS) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                    uint16_t* __restrict__ y, int64_t ldy,
                                                                    int64_t blocks_per_row, int64_t nblocks,
                                                                    RopeArgs rope = RopeArgs{}) {
    const int64_t gid = (int64_t)blockIdx.x * QUANT_THREADS + threadIdx.x;
    if (gid >= nblocks) return;
    quant_rows_block<MODE, VEC, ROPE>(x, ldx, y, ldy, blocks_per_row, gid, rope);
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
    const int64_t gid = (int64_t)blockIdx.x * QUANT_THREADS + threadIdx.x;
    if (gid >= nblocks) return;
    quant_pack_block<MODE, ROPE>(x, ldx, codes, ldc, scales, lds, blocks_per_row, gid, vec, rope);
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
