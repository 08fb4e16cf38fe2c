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
// HBM traffic is the unique key bytes plus the output.  Spans that hold keys
// are dispatched first (request-major), spans past a request's keys (-inf
// only) after them, so every key-reading wave starts in the first wave of
// the launch.  A wave issues all 16 KB of its span's loads before the first
// MFMA; a mapped page is read without per-lane predication.
//
// Inside a span the dot products run on the matrix cores: the query vectors
// of the request, ordered (row j, head h) -> m = 4j + h, form the A operand
// of v_mfma_f32_16x16x32_bf16 (one 16-row tile per 4 rows), and 16 keys form
// the B columns.  In the MFMA result layout a lane holds the 4 consecutive m
// rows of one column, i.e. all 4 heads of one (row, key): ReLU, head sum,
// scale and mask are applied in-lane with no shuffles.  Key c0 + 4n + g of a
// span (n = column 0..15, g = group 0..3) goes to column n of group g, so
// after 4 groups each lane owns 4 consecutive keys and writes them with one
// 16-byte store.
//
// Element formats: queries and keys in bf16 or fp16 (MATE "MQA score": both
// are canonical inputs), or fp8 e4m3 keys (the optional e4m3 compressed
// indexer cache of the vLLM QSA state backend) with bf16 or fp16 queries.
// An e4m3 key row is 128 bytes: lane q4 reads its contiguous quarter (32
// codes, two 16-byte loads per key), converts it exactly to the query's
// 16-bit format, and the query fragments use the same feature order
// (features 32*q4 + 8*ks .. +7 in k-step ks), so the products are
// unchanged.  The cache scale multiplies the head sum together with the
// score scale (relu commutes with a positive factor).
#include "qsa_device.h"
#include "qsa_internal.h"

#ifndef QSA_DECODE_WAVES_PER_BLOCK
#define QSA_DECODE_WAVES_PER_BLOCK 1
#endif

namespace qsa {
namespace {

constexpr int kSpan = 64;     // keys per wavefront task
constexpr int kPadSpans = 4;  // spans per -inf-only task
constexpr int kWavesPerBlock = QSA_DECODE_WAVES_PER_BLOCK;

enum PageMode { kPageGeneric = 0, kPageMultiple64 = 1, kPage64 = 2 };

// Kernel formats: query format plus whether keys are e4m3 codes.
enum DecodeFormat { kBf16 = 0, kFp16 = 1, kBf16Fp8 = 2, kFp16Fp8 = 3 };

// Q fragment: lane (n, q4) supplies query vector (row j, head h) of its
// tile, features `feature` .. +7.
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

__device__ __forceinline__ int wave_inclusive_sum(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

struct Task {
    int r;
    int span;  // first span of the task
    bool compute;
    bool valid;
};

// Task order: first every span that holds keys (request-major, one span per
// task), then the spans past a request's keys (-inf only, kPadSpans spans per
// task).  Spans of request r that hold keys: ceil(comp_r / 64), capped at the
// spans covering out_cols.  Each wave derives its task from the compressed
// lengths with a wave-wide prefix sum, 64 requests per pass, so no task list
// is needed.
__device__ Task map_task(const DecodeParams &p, int task, int lane) {
    int before = 0;  // tasks of earlier requests in the current pass
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll 1
        for (int r0 = 0; r0 < p.num_reqs; r0 += 64) {
            const int rr = r0 + lane;
            int cnt = 0;
            if (rr < p.num_reqs) {
                const int comp = p.comp_lens[rr];
                int keyed = comp > 0 ? (comp + kSpan - 1) / kSpan : 0;
                keyed = keyed < p.spans ? keyed : p.spans;
                cnt = pass == 0 ? keyed : (p.spans - keyed + kPadSpans - 1) / kPadSpans;
            }
            const int incl = wave_inclusive_sum(cnt, lane);
            const int chunk_total = __builtin_amdgcn_readlane(incl, 63);
            const int local = task - before;
            if (local < chunk_total) {
                const uint64_t below = __ballot(incl <= local);
                const int idx = __popcll(below);  // first lane whose range holds `local`
                const int excl = __builtin_amdgcn_readlane(incl - cnt, idx);
                if (pass == 0) return Task{r0 + idx, local - excl, true, true};
                const int comp = load_uniform(p.comp_lens + r0 + idx);
                int keyed_r = comp > 0 ? (comp + kSpan - 1) / kSpan : 0;
                keyed_r = keyed_r < p.spans ? keyed_r : p.spans;
                return Task{r0 + idx, keyed_r + (local - excl) * kPadSpans, false, true};
            }
            before += chunk_total;
        }
        task -= before;
        before = 0;
    }
    // The launch covers num_reqs * spans tasks, an upper bound of the real
    // count (keyed spans plus padding groups); the surplus waves do nothing.
    return Task{0, 0, false, false};
}

template <int MT, int PAGE_MODE, int FMT>
__global__ __launch_bounds__(kWavesPerBlock * 64) void decode_kernel(DecodeParams p) {
    constexpr bool kQF16 = FMT == kFp16 || FMT == kFp16Fp8;
    constexpr bool kKFp8 = FMT == kBf16Fp8 || FMT == kFp16Fp8;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int task_id = blockIdx.x * kWavesPerBlock + wave;
    const Task task = map_task(p, task_id, lane);
    if (!task.valid) return;
    const int r = __builtin_amdgcn_readfirstlane(task.r);
    const int span = __builtin_amdgcn_readfirstlane(task.span);
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const int c0 = span * kSpan;

    float res[MT][4];
    if (task.compute) {
        // Request-level reads are scalar loads, so the page-table read that
        // gates the key loads never waits behind the query loads.
        const int comp = load_uniform(p.comp_lens + r);
        const int64_t pt_row = (int64_t)r * p.page_table_stride;
        // Per-row visible counts (lane row j = 4*mt + q4), read as scalars.
        int vis_row[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int v4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * mt + i;
                int v = 0;
                if (j < p.dql) v = p.visible ? load_uniform(p.visible + (int64_t)r * p.dql + j) : comp;
                v4[i] = v < 0 ? 0 : (v > comp ? comp : v);
            }
            vis_row[mt] = q4 == 0 ? v4[0] : (q4 == 1 ? v4[1] : (q4 == 2 ? v4[2] : v4[3]));
        }

        // Query fragments (issued first: they hit in L2): tile mt holds rows
        // j = 4*mt .. 4*mt+3.
        u32x4 qa[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int j = 4 * mt + (n >> 2);
            const int h = n & 3;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = j < p.dql ? load_q_fragment(p, r, j, h, kKFp8 ? 32 * q4 + 8 * ks : 32 * ks + 8 * q4)
                                       : zero_u32x4();
        }

        // Key c0 + 4n + g, features 32ks + 8q4 .. +7, for every g and ks:
        // all 16 loads issued before any MFMA.
        u32x4 kb[4][4];
        bool key_ok[4];
        if (PAGE_MODE != kPageGeneric) {
            // The span lies on one page; a mapped page is read whole (keys
            // past comp are in bounds and masked below).
            const int slot = PAGE_MODE == kPage64 ? span : c0 / p.page_size;
            const int page = slot < p.page_table_cols ? load_uniform(p.page_table + pt_row + slot) : -1;
            const bool page_ok = page >= 0 && page < p.num_pages;
            if (page_ok) {
                const int in_page = PAGE_MODE == kPage64 ? 0 : c0 % p.page_size;
                const int64_t key0 = (int64_t)page * p.page_size + in_page + 4 * n;
                if (kKFp8) {
                    const uint8_t *src = reinterpret_cast<const uint8_t *>(p.k) + key0 * kDim + 32 * q4;
                    u32x4 raw[4][2];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        raw[g][0] = load_u32x4(src + g * kDim);
                        raw[g][1] = load_u32x4(src + g * kDim + 16);
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        kb[g][0] = e4m3x8_to_16bit<kQF16>(raw[g][0][0], raw[g][0][1]);
                        kb[g][1] = e4m3x8_to_16bit<kQF16>(raw[g][0][2], raw[g][0][3]);
                        kb[g][2] = e4m3x8_to_16bit<kQF16>(raw[g][1][0], raw[g][1][1]);
                        kb[g][3] = e4m3x8_to_16bit<kQF16>(raw[g][1][2], raw[g][1][3]);
                    }
                } else {
                    const uint16_t *src = p.k + key0 * kDim + 8 * q4;
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) kb[g][ks] = load_u32x4(src + g * kDim + 32 * ks);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) kb[g][ks] = zero_u32x4();
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) key_ok[g] = page_ok && c0 + 4 * n + g < comp;
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = c0 + 4 * n + g;
                int page = -1;
                if (c < comp) {
                    const int slot = c / p.page_size;
                    if (slot < p.page_table_cols) page = p.page_table[pt_row + slot];
                }
                key_ok[g] = page >= 0 && page < p.num_pages;
                const int64_t key = (int64_t)page * p.page_size + (c % p.page_size);
                if (kKFp8) {
                    const uint8_t *src = reinterpret_cast<const uint8_t *>(p.k) + key * kDim + 32 * q4;
                    const u32x4 lo = key_ok[g] ? load_u32x4(src) : zero_u32x4();
                    const u32x4 hi = key_ok[g] ? load_u32x4(src + 16) : zero_u32x4();
                    kb[g][0] = e4m3x8_to_16bit<kQF16>(lo[0], lo[1]);
                    kb[g][1] = e4m3x8_to_16bit<kQF16>(lo[2], lo[3]);
                    kb[g][2] = e4m3x8_to_16bit<kQF16>(hi[0], hi[1]);
                    kb[g][3] = e4m3x8_to_16bit<kQF16>(hi[2], hi[3]);
                } else {
                    const uint16_t *src = p.k + key * kDim + 8 * q4;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) kb[g][ks] = key_ok[g] ? load_u32x4(src + 32 * ks) : zero_u32x4();
                }
            }
        }

#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma_qk<kQF16>(qa[mt][ks], kb[g][ks], acc);
                const int c = c0 + 4 * n + g;
                res[mt][g] = (key_ok[g] && c < vis_row[mt]) ? head_sum_score(acc, p.scale) : neg_inf();
            }
        }
    } else {
        // -inf only: spans span .. span + kPadSpans - 1 (clipped to out_cols).
        const float ni = neg_inf();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int j = 4 * mt + q4;
            if (j >= p.dql) continue;
            float *row = p.out + ((int64_t)r * p.dql + j) * p.out_stride;
#pragma unroll
            for (int s = 0; s < kPadSpans; ++s) {
                const int col = c0 + s * kSpan + 4 * n;
                if (p.out_vec && col + 3 < p.out_cols) {
                    *reinterpret_cast<f32x4 *>(row + col) = f32x4{ni, ni, ni, ni};
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if (col + g < p.out_cols) row[col + g] = ni;
                }
            }
        }
        return;
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

template <int MT, int FMT>
hipError_t launch_fmt(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    if (p.page_size == kSpan) return launch_kernel(decode_kernel<MT, kPage64, FMT>, grid, block, stream, p);
    if (p.page_size % kSpan == 0)
        return launch_kernel(decode_kernel<MT, kPageMultiple64, FMT>, grid, block, stream, p);
    return launch_kernel(decode_kernel<MT, kPageGeneric, FMT>, grid, block, stream, p);
}

template <int MT>
hipError_t launch_mt(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    if (p.k_fp8) {
        if (p.q_f16) return launch_fmt<MT, kFp16Fp8>(p, stream, grid, block);
        return launch_fmt<MT, kBf16Fp8>(p, stream, grid, block);
    }
    if (p.q_f16) return launch_fmt<MT, kFp16>(p, stream, grid, block);
    return launch_fmt<MT, kBf16>(p, stream, grid, block);
}

}  // namespace

int decode_span_keys() { return kSpan; }

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
