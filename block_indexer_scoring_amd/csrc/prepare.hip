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
// Each (token, head) row is 256 bytes in and 256 (bf16) or 128 (e4m3) bytes
// out.  Sixteen lanes hold one row, 16 bytes each, so every load and store
// instruction moves whole rows; a lane's NeoX partner is the lane 4 away
// (features +-32), reached with a cross-lane swizzle.  At these sizes the
// kernel is limited by vector-ALU issue and by the dependent position ->
// table read rather than by HBM bandwidth, so the arithmetic is kept lean
// and every load is issued in one fixed order (see the kernel).
#include <cmath>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads, 16 lanes per (token, head) row

// fp32 -> the nearest-even bf16 value, as fp32 (three integer operations).
// A NaN whose payload sits in the upper 16 bits stays NaN; the kernel only
// feeds it such NaNs (bf16 inputs, quiet arithmetic results, and fp32
// weights canonicalized at load).
__device__ __forceinline__ float bf16_round(float f) {
    const uint32_t u = __float_as_uint(f);
    return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

// Two values that are already bf16 (low 16 bits zero) packed, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}


// Rounds eight values to the rotation type (bf16, or fp32: unchanged).
template <bool kTabF32>
__device__ __forceinline__ void round_to_type(float (&v)[8]) {
    if constexpr (!kTabF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_round(v[i]);
    }
}

__device__ __forceinline__ void unpack_bf16x8(u32x4 raw, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(raw[i] << 16);
        v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
}

// Raw table words of this lane's eight pairs in one table row: cos and sin,
// one 16-byte load each for bf16, two for fp32.
template <bool kTabF32>
struct TableWords {
    u32x4 c[kTabF32 ? 2 : 1], s[kTabF32 ? 2 : 1];
};

constexpr int kBufferWord3 = 0x00020000;     // buffer descriptor word 3: raw dword access
constexpr uint32_t kOffTable = 0x80000000u;  // a byte offset past any table: the load returns zeros

__device__ __forceinline__ u32x4 load_buffer16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
}

// The table is read through a buffer resource bounded by its size, so a row
// off the table (offset kOffTable) reads zeros without touching memory and
// without a branch: every row's loads then issue in one fixed order.
template <bool kTabF32>
__device__ __forceinline__ void load_table(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, TableWords<kTabF32> &w) {
    if constexpr (kTabF32) {
        w.c[0] = load_buffer16(rsrc, off);
        w.c[1] = load_buffer16(rsrc, off + 16);
        w.s[0] = load_buffer16(rsrc, off + 128);
        w.s[1] = load_buffer16(rsrc, off + 144);
    } else {
        w.c[0] = load_buffer16(rsrc, off);
        w.s[0] = load_buffer16(rsrc, off + 64);
    }
}

template <bool kTabF32>
__device__ __forceinline__ void unpack_words(const u32x4 (&w)[kTabF32 ? 2 : 1], float (&v)[8]) {
    if constexpr (kTabF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(w[0][i]);
            v[4 + i] = __uint_as_float(w[1][i]);
        }
    } else {
        unpack_bf16x8(w[0], v);
    }
}

// Vector-ALU issue, not HBM, limits this kernel at its sizes (a wave64
// instruction holds a 16-lane SIMD for 4 cycles), so the arithmetic is kept
// lean: bf16 roundings are three integer operations (the packed hardware
// convert measured slower here), the subtract of the first half is an add of
// the negated partner (the same IEEE result), so all 16 lanes of a row run
// one instruction stream, lanes of the pass-through half select y at the end,
// and NaN is made canonical once, at the store.
template <bool kTabF32, bool kWF32, bool kFp8, bool kMrope>
__global__ __launch_bounds__(kRowsPerBlock * 16) void prepare_q_kernel(PrepareQParams p) {
#pragma clang fp contract(off)
    const int sub = threadIdx.x & 15;  // features 8*sub .. 8*sub+7 of the row
    const uint32_t row = blockIdx.x * (uint32_t)kRowsPerBlock + (threadIdx.x >> 4);
    const uint32_t heads = (uint32_t)p.num_heads;
    const bool live = row < (uint32_t)p.num_tokens * heads;  // the host keeps this below 2^31
    const uint32_t t = live ? row / heads : 0u;
    const uint32_t h = live ? row - t * heads : 0u;

    // Issue order: positions, the row, the weight, then the table rows
    // (which wait only for the positions), so the norm below overlaps the
    // table reads.
    // Lanes past the last row read token 0, head 0 (which exists whenever the
    // kernel runs) and store nothing: unconditional loads keep the issue order.
    constexpr int kAxes = kMrope ? 3 : 1;
    int64_t pos[kAxes];
#pragma unroll
    for (int a = 0; a < kAxes; ++a) pos[a] = p.positions[a * p.pos_stride_axis + (int64_t)t * p.pos_stride_token];
    const u32x4 raw = load_u32x4(p.q + (int64_t)t * p.q_stride_token + h * 128 + 8 * sub);
    u32x4 wraw[kWF32 ? 2 : 1];
    if constexpr (kWF32) {
        wraw[0] = load_u32x4(static_cast<const float *>(p.weight) + 8 * sub);
        wraw[1] = load_u32x4(static_cast<const float *>(p.weight) + 8 * sub + 4);
    } else {
        wraw[0] = load_u32x4(static_cast<const uint16_t *>(p.weight) + 8 * sub);
    }
    const int jb = 8 * (sub & 3);  // first pair of this lane (sub < 8)
    constexpr uint32_t kRowBytes = kTabF32 ? 256 : 128;
    // The host keeps the table below 2^31 bytes.
    const __amdgpu_buffer_rsrc_t tab = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(p.cos_sin), 0, (int)(p.cos_sin_rows * kRowBytes), kBufferWord3);
    TableWords<kTabF32> tw[kAxes];
    bool ok[kAxes];
#pragma unroll
    for (int a = 0; a < kAxes; ++a) {
        ok[a] = sub < 8 && pos[a] >= 0 && pos[a] < p.cos_sin_rows;  // only rows inside the table are read
        const uint32_t off = ok[a] ? (uint32_t)pos[a] * kRowBytes + jb * (kRowBytes / 64) : kOffTable;
        load_table<kTabF32>(tab, off, tw[a]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the table reads issued ahead of the norm
    float gain[8];
    unpack_words<kWF32>(wraw, gain);
    if constexpr (kWF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gain[i] = gain[i] == gain[i] ? gain[i] : __builtin_nanf("");
    }

    float x[8];
    unpack_bf16x8(raw, x);
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += (double)(x[i] * x[i]);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
    const float mean_eps = (float)ss / 128.0f + p.eps;
    const float rrms = (float)(1.0 / std::sqrt((double)mean_eps));
    __builtin_amdgcn_sched_barrier(0);  // the table words are first needed below

    float y[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (x[i] * rrms) * (gain[i] + 1.0f);
    round_to_type<kTabF32>(y);
    float c[8], s[8];
    if constexpr (kMrope) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = s[i] = __builtin_nanf("");
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            if (!ok[a]) continue;
            float ca[8], sa[8];
            unpack_words<kTabF32>(tw[a].c, ca);
            unpack_words<kTabF32>(tw[a].s, sa);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = jb + i;
                const int axis = (j % 3 == 1 && j < 3 * p.mrope_h) ? 1 : (j % 3 == 2 && j < 3 * p.mrope_w) ? 2 : 0;
                if (axis == a) {
                    c[i] = ca[i] + 0.0f;  // the page's masked sum from +0
                    s[i] = sa[i] + 0.0f;
                }
            }
        }
    } else if (ok[0]) {
        unpack_words<kTabF32>(tw[0].c, c);
        unpack_words<kTabF32>(tw[0].s, s);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = s[i] = __builtin_nanf("");
    }
    // Lanes 0-3 hold y_j and subtract their partner's term, lanes 4-7 hold
    // y_{j+32} and add it: out = y c + (+-partner) s.
    const uint32_t flip = sub < 4 ? 0x80000000u : 0u;
    float a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float partner = __uint_as_float(__float_as_uint(__shfl_xor(y[i], 4)) ^ flip);
        a[i] = y[i] * c[i];
        b[i] = partner * s[i];
    }
    round_to_type<kTabF32>(a);
    round_to_type<kTabF32>(b);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = a[i] + b[i];
    round_to_type<kTabF32>(o);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        o[i] = sub < 8 ? o[i] : y[i];
        o[i] = o[i] == o[i] ? o[i] : __builtin_nanf("");  // one NaN: 0x7fc0 in bf16
    }
    if (!live) return;

    const int64_t at = (int64_t)t * p.out_stride_token + (int64_t)h * p.out_stride_head + 8 * sub;
    if constexpr (kTabF32) {  // bf16 rotation values are already rounded
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = bf16_round(o[i]);
    }
    if constexpr (kFp8) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i / 4] |= e4m3_rne_sat(o[i] / p.out_scale) << (8 * (i % 4));
        *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.out) + at) = make_uint2(w[0], w[1]);
    } else {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
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
