// Paged decode scores for the QSA MQA indexer on gfx950.
//
// Definition (MATE "QSA (Qwen Sparse Attention)", section "MQA score"):
// every decode row (request r, query j) scores each compressed key c of its
// request as scale * sum_h relu(q[r][j][h] . k(c)), where k(c) is row
// c % page_size of page page_table[r][c / page_size]; keys at or past the
// row's visible count, and keys on a missing page, score -inf.
//
// Work split: one wavefront per (request, 64-key span).  A span's keys are
// read from HBM exactly once and shared by all DQL rows of the request, so
// HBM traffic is the unique key bytes plus the output.
//
// Inside a span the wave runs the dot products on the matrix cores: the
// query vectors of the request, ordered (row j, head h) -> m = 4j + h, form
// the A operand of v_mfma_f32_16x16x32_bf16 (one 16-row tile per 4 rows),
// and 16 keys form the B columns.  In the MFMA result layout a lane holds the
// 4 consecutive m rows of one column, i.e. all 4 heads of one (row, key):
// ReLU, head sum, scale and mask are applied in-lane with no shuffles.
// Span key c0 + 4n + g (n = column 0..15, g = group 0..3) goes to column n of
// group g, so after 4 groups each lane owns 4 consecutive keys and writes
// them with one 16-byte store.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kSpan = 64;          // keys per wavefront task
constexpr int kWavesPerBlock = 4;

// Q fragment for 16x16x32 step `ks` (features 32*ks .. 32*ks+31): lane
// (n, q4) supplies query vector m = n of tile mt, features 32*ks + 8*q4 .. +7.
__device__ __forceinline__ u32x4 load_q_fragment(const DecodeParams &p, int r, int j, int h,
                                                 int feature) {
    const uint16_t *src = p.q + (int64_t)r * p.q_stride_req + (int64_t)j * p.q_stride_row +
                          (int64_t)h * p.q_stride_head + feature;
    if (p.q_vec) return load_u32x4(src);
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
    return v;
}

template <int MT, bool PAGE_ALIGNED>
__global__ __launch_bounds__(kWavesPerBlock * 64) void decode_kernel(DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t num_tasks = (int64_t)p.num_reqs * p.spans;
    if (task >= num_tasks) return;
    // Span-major order: every request's first spans (which always hold keys)
    // are dispatched before the later, mostly masked, spans.
    const int span = (int)(task / p.num_reqs);
    const int r = (int)(task % p.num_reqs);
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const int c0 = span * kSpan;

    const int comp = p.comp_lens[r];
    int vis_row[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vis_row[mt] = 0;
    int vis_max = 0;
    for (int j = 0; j < p.dql; ++j) {
        int v = p.visible ? p.visible[(int64_t)r * p.dql + j] : comp;
        v = v < 0 ? 0 : (v > comp ? comp : v);
        vis_max = v > vis_max ? v : vis_max;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (j == 4 * mt + q4) vis_row[mt] = v;
    }

    float res[MT][4];
    if (c0 < vis_max) {
        // Keys of this span: issue all 16 loads before any MFMA.
        u32x4 kb[4][4];
        bool key_ok[4];
        int64_t key_row[4];
        if (PAGE_ALIGNED) {
            // page_size is a multiple of 64: the whole span is on one page.
            const int slot = c0 / p.page_size;
            int page = -1;
            if (slot < p.page_table_cols) page = p.page_table[(int64_t)r * p.page_table_stride + slot];
            const bool page_ok = page >= 0 && page < p.num_pages;
            const int64_t base = (int64_t)page * p.page_size + (c0 % p.page_size);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = c0 + 4 * n + g;
                key_ok[g] = page_ok && c < vis_max;
                key_row[g] = base + 4 * n + g;
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = c0 + 4 * n + g;
                int page = -1;
                if (c < vis_max) {
                    const int slot = c / p.page_size;
                    if (slot < p.page_table_cols)
                        page = p.page_table[(int64_t)r * p.page_table_stride + slot];
                }
                key_ok[g] = page >= 0 && page < p.num_pages;
                key_row[g] = (int64_t)page * p.page_size + (c % p.page_size);
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[g][ks] = key_ok[g] ? load_u32x4(p.k + key_row[g] * kDim + 32 * ks + 8 * q4)
                                      : zero_u32x4();
        }

        // Query fragments: tile mt holds rows j = 4*mt .. 4*mt+3.
        u32x4 qa[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int j = 4 * mt + (n >> 2);
            const int h = n & 3;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = j < p.dql ? load_q_fragment(p, r, j, h, 32 * ks + 8 * q4) : zero_u32x4();
        }

#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(qa[mt][ks], kb[g][ks], acc);
                const int c = c0 + 4 * n + g;
                const bool ok = key_ok[g] && c < vis_row[mt];
                res[mt][g] = ok ? head_sum_score(acc, p.scale) : neg_inf();
            }
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) res[mt][g] = neg_inf();
    }

    // Lane (n, q4) owns row j = 4*mt + q4, keys c0 + 4n .. c0 + 4n + 3.
    const int col = c0 + 4 * n;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int j = 4 * mt + q4;
        if (j >= p.dql) continue;
        float *dst = p.out + ((int64_t)r * p.dql + j) * p.out_stride + col;
        if (p.out_vec && col + 3 < p.out_cols) {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{res[mt][0], res[mt][1], res[mt][2], res[mt][3]};
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (col + g < p.out_cols) dst[g] = res[mt][g];
        }
    }
}

template <int MT>
hipError_t launch_mt(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    if (p.page_size % kSpan == 0)
        hipLaunchKernelGGL((decode_kernel<MT, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<MT, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
    const int64_t tasks = (int64_t)p.num_reqs * p.spans;
    const dim3 grid((unsigned)((tasks + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kWavesPerBlock * 64);
    switch ((p.dql + 3) / 4) {
        case 1: return launch_mt<1>(p, stream, grid, block);
        case 2: return launch_mt<2>(p, stream, grid, block);
        case 3: return launch_mt<3>(p, stream, grid, block);
        default: return launch_mt<4>(p, stream, grid, block);
    }
}

}  // namespace qsa
