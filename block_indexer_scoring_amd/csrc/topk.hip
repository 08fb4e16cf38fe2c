// Per-row top-k block selection on gfx950.
//
// Rule (MATE "QSA (Qwen Sparse Attention)": the caller keeps the
// top-scoring blocks; "Core Attention": request-local int32 indices, -1
// padding): among the cells greater than -inf keep the k largest, equal
// values going to the lower column, and write the picks in ascending column
// order followed by -1.
//
// One 1024-thread workgroup per row.  Each float maps to an order-preserving
// 32-bit key (+0 and -0 share one key; non-candidates get key 0, below every
// candidate).  An exact radix select over the key bits (11 + 11 + 10, LDS
// histograms) finds the k-th largest key T and how many of the keys equal to
// T are needed.  The picks are then compacted in column order: a cell is
// taken if key > T, or key == T and fewer than `need` equal keys precede it;
// its output slot is (#greater before it) + min(#equal before it, need).
// Rows up to 32768 columns stay in registers for the whole select; longer
// rows are re-read from memory in each phase.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float v) {
    if (!(v > neg_inf())) return 0u;  // -inf and NaN are never picked
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0u) u = 0u;       // -0 ties +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the
// sum.  Arithmetic is modulo 2^32 (callers may pack two counters in one word).
__device__ int block_exclusive_scan(int v, int *s_wave, int *total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t x = (uint32_t)v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_wave[wave] = (int)x;
    __syncthreads();
    if (wave == 0) {
        uint32_t w = lane < kWaves ? (uint32_t)s_wave[lane] : 0u;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)w, d, 64);
            if (lane >= d) w += y;
        }
        if (lane < kWaves) s_wave[lane] = (int)w;
    }
    __syncthreads();
    const uint32_t before = (wave > 0 ? (uint32_t)s_wave[wave - 1] : 0u) + x - (uint32_t)v;
    *total = s_wave[kWaves - 1];
    __syncthreads();
    return (int)before;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    const int lane = threadIdx.x & 63;
    return __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

// Key source: registers (RESIDENT, E slots per thread) or the row in memory.
template <int E, bool RESIDENT>
struct RowKeys {
    uint32_t reg[RESIDENT ? E : 1];
    const float *row;
    int cols;
    __device__ __forceinline__ uint32_t get(int e) const {
        if (RESIDENT) return reg[e];
        const int i = e * kThreads + (int)threadIdx.x;
        return i < cols ? order_key(row[i]) : 0u;
    }
};

struct SelectShared {
    int hist[2048];
    int wave_tmp[kWaves];
    int pick_bin, pick_above;
};

// Radix-select the k-th largest candidate key.  Returns T and sets *need to
// the number of keys equal to T that are picked.  Requires candidates > k.
template <int E, bool RESIDENT>
__device__ uint32_t radix_threshold(const RowKeys<E, RESIDENT> &keys, int slots, int k,
                                    SelectShared &sh, int *need) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < nb; b += kThreads) sh.hist[b] = 0;
        __syncthreads();
        for (int e = 0; e < slots; ++e) {
            const uint32_t key = keys.get(e);
            if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1);
        }
        __syncthreads();
        // Thread tid owns the bins_per bins starting at the top, descending.
        const int bins_per = nb / kThreads;
        const int hi = nb - 1 - tid * bins_per;
        int s = 0;
        for (int b = 0; b < bins_per; ++b) s += sh.hist[hi - b];
        int total;
        int above = block_exclusive_scan(s, sh.wave_tmp, &total);
        if (above < kk && kk <= above + s) {
            for (int b = 0; b < bins_per; ++b) {
                const int c = sh.hist[hi - b];
                if (above + c >= kk) {
                    sh.pick_bin = hi - b;
                    sh.pick_above = above;
                    break;
                }
                above += c;
            }
        }
        __syncthreads();
        kk -= sh.pick_above;
        prefix |= (uint32_t)sh.pick_bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }
    *need = kk;
    return prefix;
}

template <int E>
__global__ __launch_bounds__(kThreads) void topk_resident_kernel(TopkParams p) {
    __shared__ SelectShared sh;
    __shared__ int s_off[E * kWaves];  // packed (greater << 16) | equal, per (slot, wave)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const float *x = p.logits + row * p.logits_stride;
    int32_t *out = p.out + row * p.out_stride;

    RowKeys<E, true> keys;
    keys.row = x;
    keys.cols = p.num_cols;
    int cand = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * kThreads + tid;
        keys.reg[e] = i < p.num_cols ? order_key(x[i]) : 0u;
        cand += keys.reg[e] != 0u;
    }
    int num_cand;
    block_exclusive_scan(cand, sh.wave_tmp, &num_cand);

    uint32_t T = 0u;
    int need = 0;
    if (num_cand > p.k) T = radix_threshold<E, true>(keys, E, p.k, sh, &need);

    // Counts of greater / equal keys per (slot, wave), then one scan in
    // column order (slot-major, wave-minor, lane within the wave).
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t key = keys.reg[e];
        const uint64_t gt = __ballot(key > T);
        const uint64_t eq = __ballot(key == T && key != 0u);
        if (lane == 0) s_off[e * kWaves + wave] = (int)(((uint32_t)__popcll(gt) << 16) | (uint32_t)__popcll(eq));
    }
    __syncthreads();
    {
        const int v = tid < E * kWaves ? s_off[tid] : 0;
        int total;
        const int before = block_exclusive_scan(v, sh.wave_tmp, &total);
        if (tid < E * kWaves) s_off[tid] = before;
        __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t key = keys.reg[e];
        const bool is_gt = key > T;
        const bool is_eq = key == T && key != 0u;
        const uint64_t gt = __ballot(is_gt);
        const uint64_t eq = __ballot(is_eq);
        // Both counts are at most 32768 (at most 32768 columns), so the low
        // half of the packed prefix never carries into the high half.
        const uint32_t base = (uint32_t)s_off[e * kWaves + wave];
        const int gt_before = (int)(base >> 16) + lanes_below(gt);
        const int eq_before = (int)(base & 0xffffu) + lanes_below(eq);
        const int col = e * kThreads + tid;
        if (is_gt) out[gt_before + min(eq_before, need)] = col;
        else if (is_eq && eq_before < need) out[gt_before + eq_before] = col;
    }
    const int picked = min(num_cand, p.k);
    for (int i = picked + tid; i < p.k; i += kThreads) out[i] = -1;
}

// Rows longer than the register-resident limit: each phase re-reads the row.
__global__ __launch_bounds__(kThreads) void topk_streaming_kernel(TopkParams p) {
    __shared__ SelectShared sh;
    __shared__ int s_cnt[2][kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const float *x = p.logits + row * p.logits_stride;
    int32_t *out = p.out + row * p.out_stride;
    const int slots = (p.num_cols + kThreads - 1) / kThreads;

    RowKeys<1, false> keys;
    keys.row = x;
    keys.cols = p.num_cols;
    int cand = 0;
    for (int e = 0; e < slots; ++e) cand += keys.get(e) != 0u;
    int num_cand;
    block_exclusive_scan(cand, sh.wave_tmp, &num_cand);

    uint32_t T = 0u;
    int need = 0;
    if (num_cand > p.k) T = radix_threshold<1, false>(keys, slots, p.k, sh, &need);

    int gt_run = 0, eq_run = 0;  // greater / equal keys in earlier slots
    for (int e = 0; e < slots; ++e) {
        const uint32_t key = keys.get(e);
        const bool is_gt = key > T;
        const bool is_eq = key == T && key != 0u;
        const uint64_t gt = __ballot(is_gt);
        const uint64_t eq = __ballot(is_eq);
        if (lane == 0) {
            s_cnt[0][wave] = __popcll(gt);
            s_cnt[1][wave] = __popcll(eq);
        }
        __syncthreads();
        int gt_wave = 0, eq_wave = 0, gt_slot = 0, eq_slot = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) {
                gt_wave += s_cnt[0][w];
                eq_wave += s_cnt[1][w];
            }
            gt_slot += s_cnt[0][w];
            eq_slot += s_cnt[1][w];
        }
        const int gt_before = gt_run + gt_wave + lanes_below(gt);
        const int eq_before = eq_run + eq_wave + lanes_below(eq);
        const int col = e * kThreads + tid;
        if (is_gt) out[gt_before + min(eq_before, need)] = col;
        else if (is_eq && eq_before < need) out[gt_before + eq_before] = col;
        gt_run += gt_slot;
        eq_run += eq_slot;
        __syncthreads();
    }
    const int picked = min(num_cand, p.k);
    for (int i = picked + tid; i < p.k; i += kThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)p.num_rows);
    const dim3 block(kThreads);
    const int slots = (p.num_cols + kThreads - 1) / kThreads;
    if (slots <= 4)
        hipLaunchKernelGGL(topk_resident_kernel<4>, grid, block, 0, stream, p);
    else if (slots <= 8)
        hipLaunchKernelGGL(topk_resident_kernel<8>, grid, block, 0, stream, p);
    else if (slots <= 16)
        hipLaunchKernelGGL(topk_resident_kernel<16>, grid, block, 0, stream, p);
    else if (slots <= 32)
        hipLaunchKernelGGL(topk_resident_kernel<32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(topk_streaming_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace qsa
