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

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
