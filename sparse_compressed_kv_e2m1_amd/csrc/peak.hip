// peak.hip -- measurement kernels for the roofline denominators (C ABI in
// include/sckv_peak.h): a streaming HBM copy, a streaming HBM read, a gather
// of 1 KiB rows through an index list (the attention's access pattern), and dense
// matrix-core loops for the two contractions of the hot path (bf16 products;
// e2m1 x e2m1 products with power-of-two block scales).  Not part of the hot
// path; built into libsckv_peak.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "sckv.h"
#include "sckv_peak.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int THREADS = 256;
constexpr int CHAINS = 8;  // independent accumulators a wave: products issue back to back

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SCKV_OK : fail(SCKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// DEPTH 16-byte vectors a thread in flight per round, grid-strided.
template <int DEPTH>
__global__ __launch_bounds__(THREADS) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t n16) {
    const int64_t nt = (int64_t)gridDim.x * THREADS;
    int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    for (; i + (DEPTH - 1) * nt < n16; i += DEPTH * nt) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) v[j] = __builtin_nontemporal_load(src + i + j * nt);
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) __builtin_nontemporal_store(v[j], dst + i + j * nt);
    }
    for (; i < n16; i += nt) dst[i] = src[i];
}

template <int DEPTH>
__global__ __launch_bounds__(THREADS) void peak_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                            uint32_t* __restrict__ out) {
    const int64_t nt = (int64_t)gridDim.x * THREADS;
    int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    u32x4 x = {0u, 0u, 0u, 0u};
    for (; i + (DEPTH - 1) * nt < n16; i += DEPTH * nt) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) v[j] = __builtin_nontemporal_load(src + i + j * nt);
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) x ^= v[j];
    }
    for (; i < n16; i += nt) x ^= src[i];
    out[(int64_t)blockIdx.x * THREADS + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// Gather of 1 KiB rows named by an index list: each wave takes DEPTH
// consecutive list entries at a time (grid-strided) and reads those rows with
// one 16-byte load a lane per row, XOR folded per thread.
template <int DEPTH>
__global__ __launch_bounds__(THREADS) void peak_gather_kernel(const u32x4* __restrict__ rows,
                                                              const int32_t* __restrict__ idx, int64_t n_idx,
                                                              uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t nw = (int64_t)gridDim.x * (THREADS / 64);
    int64_t e = ((int64_t)blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6)) * DEPTH;
    u32x4 x = {0u, 0u, 0u, 0u};
    for (; e < n_idx; e += nw * DEPTH) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int64_t r = e + j < n_idx ? idx[e + j] : idx[e];
            v[j] = rows[r * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) x ^= v[j];
    }
    out[(int64_t)blockIdx.x * THREADS + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

__global__ __launch_bounds__(THREADS) void peak_mfma_bf16_kernel(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(0.125f * (float)((lane + k) & 7));
        b[k] = (__bf16)(0.0625f * (float)((lane * 3 + k) & 7));
    }
    f32x16 acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < CHAINS; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(int64_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

// e2m1 x e2m1 (format 4 for both operands: 32 codes a lane in the low four
// registers), E8M0 scale 127 (= 1) for both.
__global__ __launch_bounds__(THREADS) void peak_mfma_fp4_kernel(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const i32x8 a = {0x13572468 ^ lane, 0x24681357 + lane, 0x11223344, 0x55667711, 0, 0, 0, 0};
    const i32x8 b = {0x21436587 + lane, 0x12345671 ^ lane, 0x01020304, 0x05060701, 0, 0, 0, 0};
    f32x16 acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < CHAINS; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, 127, 0, 127);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(int64_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

}  // namespace

extern "C" int sckv_peak_copy(const void* src, void* dst, int64_t bytes, int blocks, int depth, void* stream) {
    if (bytes < 0 || bytes % 64 || blocks <= 0 || !src || !dst || (uintptr_t)src % 16 || (uintptr_t)dst % 16 ||
        (depth != 4 && depth != 8 && depth != 16))
        return fail(SCKV_EINVAL, "sckv_peak_copy: bad arguments");
    if (bytes == 0) return SCKV_OK;
    const dim3 g((unsigned)blocks), t(THREADS);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* a = (const u32x4*)src;
    u32x4* d = (u32x4*)dst;
    if (depth == 4) peak_copy_kernel<4><<<g, t, 0, s>>>(a, d, bytes / 16);
    else if (depth == 8) peak_copy_kernel<8><<<g, t, 0, s>>>(a, d, bytes / 16);
    else peak_copy_kernel<16><<<g, t, 0, s>>>(a, d, bytes / 16);
    return launched("sckv_peak_copy");
}

extern "C" int sckv_peak_read(const void* src, int64_t bytes, uint32_t* out, int blocks, int depth, void* stream) {
    if (bytes < 0 || bytes % 64 || blocks <= 0 || !src || !out || (uintptr_t)src % 16 || (uintptr_t)out % 4 ||
        (depth != 4 && depth != 8 && depth != 16))
        return fail(SCKV_EINVAL, "sckv_peak_read: bad arguments");
    const dim3 g((unsigned)blocks), t(THREADS);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* a = (const u32x4*)src;
    if (depth == 4) peak_read_kernel<4><<<g, t, 0, s>>>(a, bytes / 16, out);
    else if (depth == 8) peak_read_kernel<8><<<g, t, 0, s>>>(a, bytes / 16, out);
    else peak_read_kernel<16><<<g, t, 0, s>>>(a, bytes / 16, out);
    return launched("sckv_peak_read");
}

extern "C" int sckv_peak_gather(const void* rows, int64_t n_rows, const int32_t* idx, int64_t n_idx, uint32_t* out,
                                int blocks, int depth, void* stream) {
    if (n_rows <= 0 || n_idx < 0 || blocks <= 0 || !rows || !idx || !out || (uintptr_t)rows % 16 ||
        (uintptr_t)idx % 4 || (uintptr_t)out % 4 || (depth != 4 && depth != 8 && depth != 16))
        return fail(SCKV_EINVAL, "sckv_peak_gather: bad arguments");
    if (n_idx == 0) return SCKV_OK;
    const dim3 g((unsigned)blocks), t(THREADS);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* a = (const u32x4*)rows;
    if (depth == 4) peak_gather_kernel<4><<<g, t, 0, s>>>(a, idx, n_idx, out);
    else if (depth == 8) peak_gather_kernel<8><<<g, t, 0, s>>>(a, idx, n_idx, out);
    else peak_gather_kernel<16><<<g, t, 0, s>>>(a, idx, n_idx, out);
    return launched("sckv_peak_gather");
}

extern "C" double sckv_peak_mfma_flops(int kind, int64_t iters, int blocks) {
    const double per = kind == SCKV_PEAK_MFMA_BF16 ? 32.0 * 32 * 16 * 2 : kind == SCKV_PEAK_MFMA_FP4 ? 32.0 * 32 * 64 * 2
                                                                                                    : 0.0;
    return per * CHAINS * (double)iters * (double)blocks * (THREADS / 64);
}

extern "C" int sckv_peak_mfma(int kind, int64_t iters, int blocks, float* out, void* stream) {
    if (iters < 0 || blocks <= 0 || !out || (uintptr_t)out % 4) return fail(SCKV_EINVAL, "sckv_peak_mfma: bad arguments");
    hipStream_t s = (hipStream_t)stream;
    if (kind == SCKV_PEAK_MFMA_BF16)
        peak_mfma_bf16_kernel<<<dim3((unsigned)blocks), dim3(THREADS), 0, s>>>(iters, out);
    else if (kind == SCKV_PEAK_MFMA_FP4)
        peak_mfma_fp4_kernel<<<dim3((unsigned)blocks), dim3(THREADS), 0, s>>>(iters, out);
    else
        return fail(SCKV_EINVAL, "sckv_peak_mfma: unknown kind");
    return launched("sckv_peak_mfma");
}

extern "C" const char* sckv_peak_last_error(void) { return g_err.c_str(); }
