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
// the launch.  A wave finds its task either from the compressed lengths (a
// wave-wide prefix sum) or, in a planned launch, from one 16-byte entry of a
// task table built once per step (qsa_build_decode_plan), which also holds
// the span's physical page: one scalar load stands between the wave's start
// and its key loads.
//
// Loads, in issue order: the request's query fragments (shared by all spans
// of the request, so they stay in L2), then the span's 16 KB of keys.  When
// the span lies on one page (page sizes that are multiples of 64), every key
// load instruction covers whole 128-byte lines: lanes 2m and 2m+1 read the
// two halves of one line, of key pair (2m, 2m+1) in turn, and swap halves
// with a DPP permutation afterwards.  Keys are read with the streaming
// (non-temporal) policy: they are used once, and keeping them out of the
// caches keeps the queries and tables there.  (Under that policy a line read
// in halves by two instructions is fetched twice, hence the whole-line
// layout.)
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
// An e4m3 key row is 128 bytes: lane q4 holds its contiguous quarter (32
// codes), converts it exactly to the query's 16-bit format, and the query
// fragments use the same feature order (features 32*q4 + 8*ks .. +7 in
// k-step ks), so the products are unchanged.  The cache scale multiplies the
// head sum together with the score scale (relu commutes with a positive
// factor).
#include <mutex>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

// The library's own decode task table, for callers that cannot allocate
// (qsa_mqa_decode_static_plan): 262,144 entries of 16 bytes (4 MiB) per
// device, held until the process ends.  In host code `scratch` names only a
// host-side stand-in; kernels get the device address from
// static_plan_pointer().
constexpr int64_t kStaticPlanEntries = 262144;
static __device__ __align__(256) int32_t scratch[kStaticPlanEntries * 4];

constexpr int kSpan = 64;     // keys per wavefront task
constexpr int kPadSpans = 4;  // spans per -inf-only task

enum PageMode { kPageGeneric = 0, kPageMultiple64 = 1, kPage64 = 2 };

// Kernel formats: query format plus whether keys are e4m3 codes.
enum DecodeFormat { kBf16 = 0, kFp16 = 1, kBf16Fp8 = 2, kFp16Fp8 = 3 };

// Where a wave's task comes from.
enum TaskSource { kMapped = 0, kPlanned = 1 };

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Q fragment: lane (n, q4) supplies query vector (row j, head h) of its
// tile, features `feature` .. +7.
__device__ __forceinline__ const uint16_t *q_fragment_ptr(const DecodeParams &p, int r, int j, int h,
                                                          int feature) {
    return p.q + (int64_t)r * p.q_stride_req + (int64_t)j * p.q_stride_row + (int64_t)h * p.q_stride_head +
           feature;
}

// The same 8 elements read one by one (Q off the 16-byte grid).
__device__ __forceinline__ u32x4 load_q_elements(const uint16_t *src) {
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

// Spans of a request that hold keys: ceil(comp / 64), capped at the spans
// covering out_cols.
__device__ __forceinline__ int keyed_spans(int comp, int spans) {
    const int keyed = comp > 0 ? (comp + kSpan - 1) / kSpan : 0;
    return keyed < spans ? keyed : spans;
}

struct Task {
    int r;
    int span;  // first span of the task
    bool compute;
    bool valid;
};

// Task order: first every span that holds keys (request-major, one span per
// task), then the spans past a request's keys (-inf only, kPadSpans spans per
// task).  Each wave derives its task from the compressed lengths with a
// wave-wide prefix sum, 64 requests per pass.
__device__ Task map_task(const DecodeParams &p, int task, int lane) {
    int before = 0;  // tasks of earlier requests in the current pass
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll 1
        for (int r0 = 0; r0 < p.num_reqs; r0 += 64) {
            const int rr = r0 + lane;
            int cnt = 0;
            if (rr < p.num_reqs) {
                const int keyed = keyed_spans(p.comp_lens[rr], p.spans);
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
                const int keyed_r = keyed_spans(load_uniform(p.comp_lens + r0 + idx), p.spans);
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

template <int MT, int PAGE_MODE, int FMT, int SRC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(MT <= 1 ? 5 : (MT <= 2 ? 4 : 2)))) void decode_kernel(
    const int32_t *plan, DecodeParams p) {
    constexpr bool kQF16 = FMT == kFp16 || FMT == kFp16Fp8;
    constexpr bool kKFp8 = FMT == kBf16Fp8 || FMT == kFp16Fp8;
    constexpr bool kUniform = PAGE_MODE != kPageGeneric;
    const int lane = threadIdx.x & 63;
    const int task_id = blockIdx.x;

    // Every kernel argument the key path reads is required before the first
    // branch: their scalar loads then go out together in one round trip,
    // rather than one round trip for each branch that first needs some of
    // them (the start-up of a short launch like this one is a chain of such
    // round trips).  The empty asm only requires the values.
    auto require_args = [&]() {
        asm volatile("" ::"s"(p.q), "s"(p.q_stride_req), "s"(p.q_stride_row), "s"(p.q_stride_head), "s"(p.k),
                     "s"(p.num_pages), "s"(p.page_size), "s"(p.visible), "s"(p.num_reqs), "s"(p.dql), "s"(p.scale));
        asm volatile("" ::"s"(p.out), "s"(p.out_stride), "s"(p.out_cols), "s"(p.spans), "s"(p.q_vec), "s"(p.out_vec));
        if (SRC == kMapped)
            asm volatile("" ::"s"(p.comp_lens), "s"(p.page_table), "s"(p.page_table_stride), "s"(p.page_table_cols));
    };

    int r, span, comp, page = -1;
    bool compute;
    if (SRC == kPlanned) {
        // The entry is wave-uniform: one scalar load.  Any contents are safe:
        // requests, spans and pages outside the launch's ranges are refused.
        // The table pointer is the first kernel argument (preloaded into
        // SGPRs at wave launch), so the entry's load goes out with the other
        // arguments' loads: one round trip for all of them.
        const i32x4 e = load_uniform(reinterpret_cast<const i32x4 *>(plan) + task_id);
        asm volatile("" ::"s"(e[0]), "s"(e[1]), "s"(e[2]), "s"(e[3]));
        require_args();
        r = e[0];
        if (r < 0 || r >= p.num_reqs) return;
        span = e[1] & 0x7fffffff;
        if (span >= p.spans) return;
        compute = e[1] >= 0;
        page = e[2];
        comp = e[3] > 0 ? e[3] : 0;
    } else {
        require_args();
        const Task task = map_task(p, task_id, lane);
        if (!task.valid) return;
        r = __builtin_amdgcn_readfirstlane(task.r);
        span = __builtin_amdgcn_readfirstlane(task.span);
        compute = task.compute;
        comp = 0;
    }
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const int c0 = span * kSpan;

    if (__builtin_expect(!compute, 0)) {
        // -inf only: spans span .. span + kPadSpans - 1 (clipped to out_cols).
        // Laid out after the key path (unlikely), so a key-reading wave's
        // first instructions are contiguous from the kernel's entry.
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

    // Query fragments first: tile mt holds rows j = 4*mt .. 4*mt+3.
    u32x4 qa[MT][4];
    const int qh = n & 3;
    if (__builtin_expect(p.q_vec, 1)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int j = 4 * mt + (n >> 2);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = j < p.dql ? load_u32x4(q_fragment_ptr(p, r, j, qh, kKFp8 ? 32 * q4 + 8 * ks : 32 * ks + 8 * q4))
                                       : zero_u32x4();
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int j = 4 * mt + (n >> 2);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = j < p.dql ? load_q_elements(q_fragment_ptr(p, r, j, qh, kKFp8 ? 32 * q4 + 8 * ks : 32 * ks + 8 * q4))
                                       : zero_u32x4();
        }
    }

    // The visible count of the lane's row j = 4*mt + q4, as one vector load
    // issued ahead of the key loads: it returns with them, so the mask adds
    // no wait of its own.
    int vis_raw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int j = 4 * mt + q4;
        vis_raw[mt] = (p.visible && j < p.dql) ? p.visible[(int64_t)r * p.dql + j] : 0x7fffffff;
    }

    // A mapped launch reads the request's length and the span's page here
    // (scalar loads, so the page read never waits behind the query loads);
    // a planned one has both from its entry.
    const int64_t pt_row = (int64_t)r * p.page_table_stride;
    if (SRC == kMapped) {
        comp = load_uniform(p.comp_lens + r);
        if (kUniform) {
            const int slot = PAGE_MODE == kPage64 ? span : c0 / p.page_size;
            page = slot < p.page_table_cols ? load_uniform(p.page_table + pt_row + slot) : -1;
        }
    }

    // Key c0 + 4n + g, features 32ks + 8q4 .. +7 (16-bit keys) or codes
    // 32q4 .. +31 (e4m3), for every g and ks: all loads issued before any
    // MFMA.
    u32x4 kb[4][4];
    bool key_ok[4];
    if (kUniform) {
        // The span lies on one page; a mapped page is read whole (keys past
        // comp are in bounds and masked below).  Load t of a pair reads key
        // 4 (2m + t) + g: lanes 2m, 2m+1 (same q4) cover one 128-byte line.
        const bool page_ok = page >= 0 && page < p.num_pages;
        const bool even = (n & 1) == 0;
        const int m2 = n & ~1;
        if (page_ok) {
            const int ps = PAGE_MODE == kPage64 ? kSpan : p.page_size;
            const int in_page = PAGE_MODE == kPage64 ? 0 : c0 % ps;
            const uint8_t *base =
                reinterpret_cast<const uint8_t *>(p.k) + ((int64_t)page * ps + in_page) * (kKFp8 ? kDim : 2 * kDim);
            if (kKFp8) {
                // Row of 128 codes = one line; lane (q4, 2m + par) reads its
                // 16-byte piece 2 q4 + par, so each lane ends with pieces
                // 2 q4 and 2 q4 + 1 (codes 32 q4 .. +31) of its own key.
                const uint8_t *src = base + 16 * (2 * q4 + (n & 1));
                u32x4 raw[4][2];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int t = 0; t < 2; ++t) raw[g][t] = load_u32x4_stream(src + (4 * (m2 + t) + g) * kDim);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x4 lo, hi;
                    lane_pair_exchange(even, raw[g][0], raw[g][1], lo, hi);
                    kb[g][0] = e4m3x8_to_16bit<kQF16>(lo[0], lo[1]);
                    kb[g][1] = e4m3x8_to_16bit<kQF16>(lo[2], lo[3]);
                    kb[g][2] = e4m3x8_to_16bit<kQF16>(hi[0], hi[1]);
                    kb[g][3] = e4m3x8_to_16bit<kQF16>(hi[2], hi[3]);
                }
            } else {
                // Row of 256 bytes = two lines; in line hl lane (q4, 2m + par)
                // reads piece 4 par + q4, so each lane ends with features
                // 64 hl + 8 q4 and 64 hl + 32 + 8 q4 (k-steps 2 hl, 2 hl + 1).
                const uint8_t *src = base + 16 * (4 * (n & 1) + q4);
                u32x4 raw[4][2][2];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
                            raw[g][hl][t] = load_u32x4_stream(src + (4 * (m2 + t) + g) * (2 * kDim) + 128 * hl);
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        lane_pair_exchange(even, raw[g][hl][0], raw[g][hl][1], kb[g][2 * hl], kb[g][2 * hl + 1]);
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
        // Any page size: one page lookup per key; loads with the default
        // policy (a lane reads half of a line).
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = c0 + 4 * n + g;
            int pg = -1;
            if (c < comp) {
                const int slot = c / p.page_size;
                if (slot < p.page_table_cols) pg = p.page_table[pt_row + slot];
            }
            key_ok[g] = pg >= 0 && pg < p.num_pages;
            const int64_t key = (int64_t)pg * p.page_size + (c % p.page_size);
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

    // Visible counts of the lane's rows, clamped to [0, comp].
    int vis_row[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int v = vis_raw[mt];
        vis_row[mt] = v < 0 ? 0 : (v > comp ? comp : v);
    }

    // Four independent accumulator chains (one per key group), interleaved
    // k-step by k-step, so the matrix core never waits on its own result.
    float res[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[g] = mfma_qk<kQF16>(qa[mt][ks], kb[g][ks], acc[g]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = c0 + 4 * n + g;
            res[mt][g] = (key_ok[g] && c < vis_row[mt]) ? head_sum_score(acc[g], p.scale) : neg_inf();
        }
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

// Task table of a planned launch (qsa_build_decode_plan): entry e of
// num_reqs * spans.  Every workgroup scans the per-request task counts into
// LDS (keyed spans, then -inf groups), so workgroups need no grid-wide
// ordering, then fills its entries by binary search over the offsets.
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(PlanParams p) {
    __shared__ int32_t keyed_off[kPlanMaxReqs + 1];
    __shared__ int32_t pad_off[kPlanMaxReqs + 1];
    __shared__ int32_t wave_sum[2][kPlanThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Thread tid counts requests [tid*per, (tid+1)*per).
    const int per = (p.num_reqs + kPlanThreads - 1) / kPlanThreads;
    const int r0 = tid * per;
    int my_keyed = 0, my_pad = 0;
    for (int r = r0; r < r0 + per && r < p.num_reqs; ++r) {
        const int keyed = keyed_spans(p.comp_lens[r], p.spans);
        const int pad = (p.spans - keyed + kPadSpans - 1) / kPadSpans;
        keyed_off[r] = keyed;  // counts for now; offsets below
        pad_off[r] = pad;
        my_keyed += keyed;
        my_pad += pad;
    }
    const int ik = wave_inclusive_sum(my_keyed, lane);
    const int ip = wave_inclusive_sum(my_pad, lane);
    if (lane == 63) {
        wave_sum[0][wave] = ik;
        wave_sum[1][wave] = ip;
    }
    __syncthreads();
    int bk = 0, bp = 0;
    for (int w = 0; w < wave; ++w) {
        bk += wave_sum[0][w];
        bp += wave_sum[1][w];
    }
    int run_k = bk + ik - my_keyed, run_p = bp + ip - my_pad;
    for (int r = r0; r < r0 + per && r < p.num_reqs; ++r) {
        const int ck = keyed_off[r], cp = pad_off[r];
        keyed_off[r] = run_k;
        pad_off[r] = run_p;
        run_k += ck;
        run_p += cp;
    }
    if (tid == kPlanThreads - 1) {
        keyed_off[p.num_reqs] = run_k;  // all keyed tasks
        pad_off[p.num_reqs] = run_p;    // all -inf tasks
    }
    __syncthreads();
    const int64_t total_keyed = keyed_off[p.num_reqs];
    const int64_t total = total_keyed + pad_off[p.num_reqs];
    const bool uniform = p.page_size % kSpan == 0;
    i32x4 *plan = reinterpret_cast<i32x4 *>(p.plan);
    for (int64_t e = (int64_t)blockIdx.x * kPlanThreads + tid; e < p.entries; e += (int64_t)gridDim.x * kPlanThreads) {
        i32x4 v = {-1, 0, -1, 0};
        if (e < total) {
            const bool keyed = e < total_keyed;
            const int32_t *off = keyed ? keyed_off : pad_off;
            const int64_t local = keyed ? e : e - total_keyed;
            // Last request whose first task is <= local (requests without
            // tasks share the next one's offset).
            int lo = 0, hi = p.num_reqs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= local) lo = mid;
                else hi = mid - 1;
            }
            const int r = lo;
            const int comp = p.comp_lens[r];
            if (keyed) {
                const int span = (int)(local - off[r]);
                int page = -1;
                if (uniform) {
                    const int slot = span * kSpan / p.page_size;
                    if (slot < p.page_table_cols) page = p.page_table[(int64_t)r * p.page_table_stride + slot];
                    if (page < 0 || page >= p.num_pages) page = -1;
                }
                v = i32x4{r, span, page, comp};
            } else {
                const int span = keyed_spans(comp, p.spans) + (int)(local - off[r]) * kPadSpans;
                v = i32x4{r, (int32_t)((uint32_t)span | 0x80000000u), -1, comp};
            }
        }
        plan[e] = v;
    }
}

template <int MT, int FMT, int SRC>
hipError_t launch_fmt(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    // The task table goes first among the kernel arguments, where it can be
    // preloaded into SGPRs at wave launch.
    const int32_t *plan = SRC == kPlanned ? p.plan : nullptr;
    if (p.page_size == kSpan) return launch_kernel(decode_kernel<MT, kPage64, FMT, SRC>, grid, block, stream, plan, p);
    if (p.page_size % kSpan == 0)
        return launch_kernel(decode_kernel<MT, kPageMultiple64, FMT, SRC>, grid, block, stream, plan, p);
    return launch_kernel(decode_kernel<MT, kPageGeneric, FMT, SRC>, grid, block, stream, plan, p);
}

template <int MT, int SRC>
hipError_t launch_mt(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    if (p.k_fp8) {
        if (p.q_f16) return launch_fmt<MT, kFp16Fp8, SRC>(p, stream, grid, block);
        return launch_fmt<MT, kBf16Fp8, SRC>(p, stream, grid, block);
    }
    if (p.q_f16) return launch_fmt<MT, kFp16, SRC>(p, stream, grid, block);
    return launch_fmt<MT, kBf16, SRC>(p, stream, grid, block);
}

template <int SRC>
hipError_t launch_src(const DecodeParams &p, hipStream_t stream, dim3 grid, dim3 block) {
    switch ((p.dql + 3) / 4) {
        case 1: return launch_mt<1, SRC>(p, stream, grid, block);
        case 2: return launch_mt<2, SRC>(p, stream, grid, block);
        case 3: return launch_mt<3, SRC>(p, stream, grid, block);
        default: return launch_mt<4, SRC>(p, stream, grid, block);
    }
}

}  // namespace

int decode_span_keys() { return kSpan; }

int64_t static_plan_entries() { return kStaticPlanEntries; }

hipError_t static_plan_pointer(int32_t **table) {
    static std::mutex mu;
    static int32_t *addr[64] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        addr[dev] = static_cast<int32_t *>(ptr);
    }
    *table = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
    const int64_t tasks = (int64_t)p.num_reqs * p.spans;
    const dim3 grid((unsigned)tasks);
    const dim3 block(64);
    if (p.plan) return launch_src<kPlanned>(p, stream, grid, block);
    return launch_src<kMapped>(p, stream, grid, block);
}

hipError_t launch_decode_plan(const PlanParams &p, hipStream_t stream) {
    const int64_t blocks = (p.entries + kPlanThreads - 1) / kPlanThreads;
    const dim3 grid((unsigned)(blocks < 512 ? blocks : 512));
    return launch_kernel(decode_plan_kernel, grid, dim3(kPlanThreads), stream, p);
}

}  // namespace qsa
