// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Head geometry fixed by the indexer: 4 query heads share one 128-wide key.
constexpr int kHeads = 4;
constexpr int kDim = 128;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ u32x4 load_u32x4(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 zero_u32x4() { return u32x4{0u, 0u, 0u, 0u}; }

// ReLU that maps -0.0 to +0.0, so an all-negative head set gives +0.0.
__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

// One MFMA accumulator quad holds the 4 head dots of one (query, key) pair:
// score = scale * sum_h relu(dot_h).
__device__ __forceinline__ float head_sum_score(f32x4 acc, float scale) {
    float s = relu(acc[0]) + relu(acc[1]);
    s += relu(acc[2]);
    s += relu(acc[3]);
    return s * scale;
}

// 16x16x32 bf16 MFMA (gfx950): lane l supplies A[m = l%16][k = 8*(l/16) .. +7]
// and B[k = 8*(l/16) .. +7][n = l%16]; it receives C[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace qsa
