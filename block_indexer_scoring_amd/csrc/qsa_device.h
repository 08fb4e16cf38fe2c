// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Head geometry fixed by the indexer: 4 query heads share one 128-wide key.
constexpr int kHeads = 4;
constexpr int kDim = 128;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ u32x4 load_u32x4(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Load through the constant address space.  At a wave-uniform address this
// becomes a scalar load, which the vector-memory counter does not track, so
// waiting for it does not also wait for the wave's outstanding vector loads.
// Only for memory that no kernel writes while the reading kernel runs (the
// scalar cache is invalidated at each kernel launch).
template <typename T>
__device__ __forceinline__ T load_uniform(const T *ptr) {
    typedef const __attribute__((address_space(4))) T *constant_ptr;
    return *(constant_ptr)(ptr);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ u32x4 zero_u32x4() { return u32x4{0u, 0u, 0u, 0u}; }

// 16-byte load with the non-temporal (streaming) policy, for data read once.
// Only for loads whose instruction covers whole 128-byte lines: a line that
// two instructions read half each is fetched from HBM twice under this
// policy.
__device__ __forceinline__ u32x4 load_u32x4_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Exchange between lane pairs (2m, 2m+1).  Whole-line loads give each pair
// two registers: r0 holds pieces of the even lane's item (its own piece in
// the even lane, the even lane's next piece in the odd lane), r1 the same
// for the odd lane's item.  Afterwards each lane holds its own two pieces:
// lo (from the even lane's register) and hi (from the odd lane's).  The
// partner's value is read with a DPP quad permutation [1, 0, 3, 2].
__device__ __forceinline__ u32x4 lane_pair_swap(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[i], 0xB1, 0xF, 0xF, true);
    return r;
}

__device__ __forceinline__ void lane_pair_exchange(bool even, u32x4 r0, u32x4 r1, u32x4 &lo, u32x4 &hi) {
    const u32x4 s0 = lane_pair_swap(r0), s1 = lane_pair_swap(r1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = even ? r0[i] : s1[i];
        hi[i] = even ? s0[i] : r1[i];
    }
}

// ReLU as a signed-integer max on the bit pattern: positive floats order
// like their bits, every non-positive float (-0 included) has the sign bit
// set and maps to the bits of +0.0.  One VALU op, and an all-negative head
// set gives exactly +0.0.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// One MFMA accumulator quad holds the 4 head dots of one (query, key) pair:
// score = scale * sum_h relu(dot_h).
__device__ __forceinline__ float head_sum_score(f32x4 acc, float scale) {
    const float s = (relu(acc[0]) + relu(acc[1])) + (relu(acc[2]) + relu(acc[3]));
    return s * scale;
}

// Order-preserving 32-bit key of a score: unsigned comparison of keys
// orders the floats, +0 and -0 share one key, and -inf and NaN get 0 (below
// every other value: never picked).
__device__ __forceinline__ uint32_t order_key(float v) {
    if (!(v > neg_inf())) return 0u;
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top halves of the order keys of two scores a, b that are >= +0, +inf or
// NaN (what the score epilogue gives for a positive scale), packed as
// (key(b) >> 16) << 16 | key(a) >> 16.  For such a score the top half is
// (bits >> 16) | 0x8000 (the sign bit is clear); a NaN is first replaced by
// the bits of -0, whose top half 0x8000 then becomes 0, the key of a cell
// that is never picked.  Cells outside a row's keys pass ok = false (0).
__device__ __forceinline__ uint32_t score_keys16(float a, float b, bool ok_a = true, bool ok_b = true) {
    const uint32_t ua = ok_a && a == a ? __float_as_uint(a) : 0x80000000u;
    const uint32_t ub = ok_b && b == b ? __float_as_uint(b) : 0x80000000u;
    return __builtin_amdgcn_perm(ub, ua, 0x07060302u) ^ 0x80008000u;
}

// 16x16x32 bf16 MFMA (gfx950): lane l supplies A[m = l%16][k = 8*(l/16) .. +7]
// and B[k = 8*(l/16) .. +7][n = l%16]; it receives C[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The same product on fp16 operands (same lane layout).
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// Query . key product for 16-bit operands in bf16 (kF16 false) or fp16.
template <bool kF16>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (kF16) return mfma16x16x32_f16(a, b, c);
    else return mfma16x16x32(a, b, c);
}

// Eight OCP e4m3 codes (two words, code i in byte i%4 of word i/4) -> the
// same eight values as 16-bit bf16 (kF16 false) or fp16, element i in half
// i%2 of word i/2.  Exact: every e4m3 value is representable in both
// (3 fraction bits, exponents 2^-9 .. 2^8).  The gfx950 conversion reads
// its fp8 operand as OCP e4m3; a scale of 1.0 leaves the value unchanged.
template <bool kF16>
__device__ __forceinline__ u32x4 e4m3x8_to_16bit(uint32_t w0, uint32_t w1) {
    u32x4 r;
    if constexpr (kF16) {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
    } else {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    }
    return r;
}

// Nearest finite OCP e4m3 value, ties to the even code; NaN -> 0x7f (the
// e4m3 store of qsa_prepare's _to_dst_dtype: magnitudes from 448 up,
// infinities included, saturate to 448).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;
    if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448, infinities included
    if (a < 0x3c800000u)                         // below 2^-6: multiples of 2^-9
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // biased exponent and 3 fraction bits
    const uint32_t code = r - ((127u - 7u) << 3);
    return sign | (code > 0x7eu ? 0x7eu : code);
}

}  // namespace qsa
