// Query preparation for the indexer: Gemma RMSNorm and NeoX rotary
// embedding of every query head, stored as bf16 or e4m3 (vLLM
// "vllm.models.qwen4_exp.amd.ops.qsa_prepare", functions _norm_rope,
// _store_rotated and _to_dst_dtype; supports_fused_pre_indexer fixes head
// dim 128, rotary dim 64, NeoX halves and interleaved MRoPE).
//
// For one head x (128 bf16 features) the kernel computes, in fp32:
//   rrms = 1 / sqrt(sum(x^2) / 128 + eps),  y_d = (x_d * rrms) * (w_d + 1),
// rounds y to the cos/sin table's type (bf16 or fp32) and rotates the NeoX
// pairs (j, j + 32), j < 32, in that type with one rounding per operation:
//   out_j = y_j c - y_{j+32} s,   out_{j+32} = y_{j+32} c + y_j s,
// where row p of the table holds 32 cos then 32 sin.  Features 64..127 pass
// through.  Under interleaved MRoPE with section (t, h, w) pair j reads the
// row of the height position when j % 3 == 1 and j < 3h, of the width
// position when j % 3 == 2 and j < 3w, else of the temporal one.  The store
// rounds to bf16; for an e4m3 destination it divides that value by the
// scale and converts to the nearest finite e4m3 value.
//
// Where the page leaves the arithmetic open: the sum of squares is the fp32
// rounding of the exact sum (accumulated in fp64 here), rrms the fp32
// rounding of 1/sqrt (computed in fp64), no multiply-add is fused, and the
// MRoPE table entry is read as the page's masked sum (so -0 becomes +0).  A
// position outside the table gives NaN for the pairs that use it.
//
// HBM-bound: each (token, head) row is 256 bytes in and 256 (bf16) or 128
// (e4m3) bytes out.  Sixteen lanes hold one row, 16 bytes each, so every
// load and store instruction moves whole rows; a lane's NeoX partner is the
// lane 4 away (features +-32), reached with a cross-lane swizzle.
#include <cmath>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads, 16 lanes per (token, head) row

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_value(float f) { return __uint_as_float(bf16_rne(f) << 16); }

// Nearest finite OCP e4m3 value, ties to the even code; NaN -> 0x7f.
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

template <bool kTabF32>
__device__ __forceinline__ float in_type(float v) {
    if constexpr (kTabF32) return v;
    else return bf16_value(v);
}

__device__ __forceinline__ void unpack_bf16x8(u32x4 raw, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(raw[i] << 16);
        v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
}

// Eight consecutive table (or weight) entries starting at `base + index`.
template <bool kF32>
__device__ __forceinline__ void load8(const void *base, int64_t index, float (&v)[8]) {
    if constexpr (kF32) {
        const u32x4 a = load_u32x4(static_cast<const float *>(base) + index);
        const u32x4 b = load_u32x4(static_cast<const float *>(base) + index + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    } else {
        unpack_bf16x8(load_u32x4(static_cast<const uint16_t *>(base) + index), v);
    }
}

template <bool kTabF32, bool kWF32, bool kFp8, bool kMrope>
__global__ __launch_bounds__(kRowsPerBlock * 16) void prepare_q_kernel(PrepareQParams p) {
#pragma clang fp contract(off)
    const int sub = threadIdx.x & 15;  // features 8*sub .. 8*sub+7 of the row
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
    const bool live = row < (int64_t)p.num_tokens * p.num_heads;
    const int64_t t = live ? row / p.num_heads : 0;
    const int64_t h = live ? row - t * p.num_heads : 0;

    float x[8];
    unpack_bf16x8(live ? load_u32x4(p.q + t * p.q_stride_token + h * 128 + 8 * sub) : zero_u32x4(), x);
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += (double)(x[i] * x[i]);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
    const float mean_eps = (float)ss / 128.0f + p.eps;
    const float rrms = (float)(1.0 / std::sqrt((double)mean_eps));

    float g[8], y[8], partner[8];
    load8<kWF32>(p.weight, 8 * sub, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = in_type<kTabF32>((x[i] * rrms) * (g[i] + 1.0f));
#pragma unroll
    for (int i = 0; i < 8; ++i) partner[i] = __shfl_xor(y[i], 4);

    float o[8];
    if (sub < 8) {
        const int jb = 8 * (sub & 3);  // first pair held by this lane
        float c[8], s[8];
        if constexpr (kMrope) {
            int64_t pos[3];
            bool ok[3];
            float ca[3][8], sa[3][8];
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                pos[a] = live ? p.positions[a * p.pos_stride_axis + t * p.pos_stride_token] : 0;
                ok[a] = pos[a] >= 0 && pos[a] < p.cos_sin_rows;
                if (ok[a]) {  // only rows inside the table are read
                    load8<kTabF32>(p.cos_sin, pos[a] * 64 + jb, ca[a]);
                    load8<kTabF32>(p.cos_sin, pos[a] * 64 + 32 + jb, sa[a]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) ca[a][i] = sa[a][i] = 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = jb + i;
                const int a = (j % 3 == 1 && j < 3 * p.mrope_h) ? 1 : (j % 3 == 2 && j < 3 * p.mrope_w) ? 2 : 0;
                const float ci = a == 0 ? ca[0][i] : a == 1 ? ca[1][i] : ca[2][i];
                const float si = a == 0 ? sa[0][i] : a == 1 ? sa[1][i] : sa[2][i];
                const bool oki = a == 0 ? ok[0] : a == 1 ? ok[1] : ok[2];
                c[i] = oki ? ci + 0.0f : __builtin_nanf("");
                s[i] = oki ? si + 0.0f : __builtin_nanf("");
            }
        } else {
            const int64_t pos = live ? p.positions[t * p.pos_stride_token] : 0;
            if (pos >= 0 && pos < p.cos_sin_rows) {  // only rows inside the table are read
                load8<kTabF32>(p.cos_sin, pos * 64 + jb, c);
                load8<kTabF32>(p.cos_sin, pos * 64 + 32 + jb, s);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = s[i] = __builtin_nanf("");
            }
        }
        if (sub < 4) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = in_type<kTabF32>(in_type<kTabF32>(y[i] * c[i]) - in_type<kTabF32>(partner[i] * s[i]));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = in_type<kTabF32>(in_type<kTabF32>(y[i] * c[i]) + in_type<kTabF32>(partner[i] * s[i]));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = y[i];
    }
    if (!live) return;

    const int64_t at = t * p.out_stride_token + h * p.out_stride_head + 8 * sub;
    if constexpr (kFp8) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = __uint_as_float(bf16_rne(o[i]) << 16) / p.out_scale;
            w[i / 4] |= e4m3_rne_sat(v) << (8 * (i % 4));
        }
        *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.out) + at) = make_uint2(w[0], w[1]);
    } else {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = bf16_rne(o[2 * i]) | (bf16_rne(o[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p.out) + at) = w;
    }
}

template <bool kTabF32, bool kWF32, bool kFp8>
hipError_t launch_out(const PrepareQParams &p, dim3 grid, dim3 block, hipStream_t stream) {
    if (p.mrope) return launch_kernel(prepare_q_kernel<kTabF32, kWF32, kFp8, true>, grid, block, stream, p);
    return launch_kernel(prepare_q_kernel<kTabF32, kWF32, kFp8, false>, grid, block, stream, p);
}

template <bool kTabF32, bool kWF32>
hipError_t launch_w(const PrepareQParams &p, dim3 grid, dim3 block, hipStream_t stream) {
    if (p.out_fp8) return launch_out<kTabF32, kWF32, true>(p, grid, block, stream);
    return launch_out<kTabF32, kWF32, false>(p, grid, block, stream);
}

}  // namespace

hipError_t launch_prepare_q(const PrepareQParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.num_tokens * p.num_heads;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    const dim3 block(kRowsPerBlock * 16);
    if (p.table_f32) {
        if (p.weight_f32) return launch_w<true, true>(p, grid, block, stream);
        return launch_w<true, false>(p, grid, block, stream);
    }
    if (p.weight_f32) return launch_w<false, true>(p, grid, block, stream);
    return launch_w<false, false>(p, grid, block, stream);
}

}  // namespace qsa
