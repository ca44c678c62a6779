// mfma.h -- gfx950 bf16 matrix-core tiles and wave-level helpers.
//
// v_mfma_f32_32x32x16_bf16 (one wave, D[32x32] += A[32x16] * B[16x32]), lane l:
//   A: row l%32, k = (l/32)*8 + 0..7      B: column l%32, k = (l/32)*8 + 0..7
//   D: 16 f32, element i at row (i/4)*8 + (l/32)*4 + i%4, column l%32
// (layout checked on the device by the library's tests).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sckv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 (one wave, D[16x16] += A[16x32] * B[32x16]), lane l:
//   A: row l%16, k = (l/16)*8 + 0..7      B: column l%16, k = (l/16)*8 + 0..7
//   D: 4 f32, element i at row (l/16)*4 + i, column l%16
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// Row of element i of a 32x32 D tile held by lane `lane`.
__device__ __forceinline__ int d_row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (same wave: no hardware barrier needed, only no reordering).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sckv

namespace sckv {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS byte offset of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes from `gaddr` land at LDS byte lds_byte + 16 * i.  Written
// as inline asm so the compiler does not add its own conservative vmcnt(0)
// waits in front of every LDS read; the caller waits with wait_vmcnt<N>().
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_byte) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gaddr), "s"(lds_byte) : "memory", "m0");
}

// Same copy with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (the saddr form): no 64-bit address arithmetic per lane.
// lds_byte must be wave-uniform; it is read from the first lane so that it
// always sits in a scalar register.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_byte) {
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lb)
                 : "memory", "m0");
}

// 4-byte-per-lane form (global_load_lds_dword): lane i's 4 bytes land at
// LDS byte lds_byte + 4 * i.
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds_byte) {
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "s"(lb)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lanes 4j..4j+3 each point at 4 consecutive 16-bit values, together one row
// j of a 4 x 16 block; lane i of the group receives column i (rows 0..3).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) char*)p);
}

}  // namespace sckv
