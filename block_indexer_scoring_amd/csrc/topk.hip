// Per-row top-k block selection on gfx950.
//
// Rule (MATE "QSA (Qwen Sparse Attention)": the caller keeps the
// top-scoring blocks; "Core Attention": request-local int32 indices, -1
// padding): among the cells greater than -inf keep the k largest, equal
// values going to the lower column, and write the picks in ascending column
// order followed by -1.
//
// One 512-thread workgroup per row, four rows per CU.  Each float maps to an
// order-preserving 32-bit key (+0 and -0 share one key; non-candidates get
// key 0, below every candidate).  An exact radix select over the key bits
// finds the k-th largest key T and how many of the keys equal to T are
// needed; a cell is picked if key > T, or key == T and fewer than `need`
// equal keys precede it.
//
// Rows up to 32768 columns stay in registers, each thread owning a
// contiguous run of columns (kept as the keys' top 16 bits), so thread order
// is column order and the picks are placed with a single prefix sum.
// Before the select, a floor F is taken from the maxima of four sub-runs per
// thread: each maximum is a distinct key, so when k of them are >= F at least
// k keys are, and T >= F.  The keys >= F (a few hundred for score rows) are
// compacted in column order into an LDS list, and one wave runs the select
// over the list without workgroup barriers: 11 + 5 bits on the top halves,
// then, only if some of the keys sharing T's top half are left out, those
// keys are re-read in full and two 8-bit passes finish T.  If the list would
// overflow, the select runs over the row itself.  Longer rows are re-read
// from memory in each phase.
#include <climits>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kMaxWaves = 16;  // workgroups of at most 1024 threads

__device__ __forceinline__ uint32_t order_key(float v) {
    if (!(v > neg_inf())) return 0u;  // -inf and NaN are never picked
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0u) u = 0u;       // -0 ties +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over a wavefront with DPP moves (no LDS): a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8 with zero
// fill), then row 0's total broadcast into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2 and 3 (row_bcast:31).
// Arithmetic is modulo 2^32.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false); // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false); // row_bcast:31
    return x;
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the
// sum.  Arithmetic is modulo 2^32 (callers may pack two counters in one word).
template <int THREADS>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave, int *total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan((uint32_t)v);
    if (lane == 63) s_wave[wave] = (int)x;
    __syncthreads();
    uint32_t before = x - (uint32_t)v, all = 0u;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        const uint32_t t = (uint32_t)s_wave[w];
        before += w < wave ? t : 0u;
        all += t;
    }
    *total = (int)all;
    __syncthreads();
    return (int)before;
}

struct SelectShared {
    alignas(16) int hist[2048];  // 16-byte aligned: wave_find_bin reads it in int4 units
    int wave_tmp[kMaxWaves];
    int pick_bin, pick_above;
};

// One wave finds the bin of hist[0..NB) (NB a power of two, at most 4096)
// holding the kk-th largest counted key: lane l sums the max(NB/64, 1) bins
// counted down from the top, a wave scan of the sums picks the lane whose
// bins hold it, then a second wave scan over that lane's bins picks the bin.
// Returns the bin (-1 if fewer than kk keys were counted) and sets
// *above_out to the count in higher bins.  Wave-uniform; no barriers.
template <int NB>
__device__ __forceinline__ int wave_find_bin(const int *hist, int kk, int *above_out) {
    constexpr int kPer = NB >= 64 ? NB / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int hi = NB - 1 - lane * kPer;
    int sum = 0;
    if (NB >= 64 || lane < NB) {
        if constexpr (kPer % 4 == 0) {
            // The lane's bins are contiguous: 16-byte reads, two in flight
            // (a kernel-wide register budget is shared with the other waves).
            const int4 *q = reinterpret_cast<const int4 *>(hist + hi - (kPer - 1));
#pragma unroll 2
            for (int j = 0; j < kPer / 4; ++j) {
                const int4 v = q[j];
                sum += (v.x + v.y) + (v.z + v.w);
            }
        } else {
#pragma unroll
            for (int b = 0; b < kPer; ++b) sum += hist[hi - b];
        }
    }
    const int incl = (int)wave_inclusive_scan((uint32_t)sum);
    const uint64_t hit = __ballot(incl - sum < kk && kk <= incl);
    if (hit == 0) {
        *above_out = 0;
        return -1;
    }
    const int src = __builtin_ctzll(hit);
    const int above0 = __builtin_amdgcn_readlane(incl - sum, src);
    const int top = NB - 1 - src * kPer;  // highest bin of lane src
    const int c = lane < kPer ? hist[top - lane] : 0;
    const int incl2 = (int)wave_inclusive_scan((uint32_t)c);
    const uint64_t hit2 = __ballot(lane < kPer && above0 + incl2 >= kk);
    const int f = __builtin_ctzll(hit2);
    *above_out = above0 + __builtin_amdgcn_readlane(incl2 - c, f);
    return top - f;
}

// The same search for the whole workgroup: call once the histogram is
// complete (after a barrier); wave 0 searches and publishes the result.
// Uniform result.
__device__ __forceinline__ int find_bin(SelectShared &sh, int nb, int kk, int *above_out) {
    if (threadIdx.x < 64) {
        int above;
        const int bin = nb == 2048 ? wave_find_bin<2048>(sh.hist, kk, &above)
                                   : wave_find_bin<1024>(sh.hist, kk, &above);
        if (threadIdx.x == 0) {
            sh.pick_bin = bin;
            sh.pick_above = above;
        }
    }
    __syncthreads();
    const int bin = sh.pick_bin;
    *above_out = sh.pick_above;
    __syncthreads();
    return bin;
}

// Where a thread's keys come from during the select: the LDS list of keys
// >= floor (entries tid, tid+1024, ... for counting; one contiguous slice
// for placing), the row in memory as columns col0 .. col0+E-1 (the
// register-resident layout, re-read), or the row in memory as columns
// e*1024 + tid (rows too long for registers).
enum KeySource { kFromList, kFromRowRun, kFromMemory };

struct ListView {
    const uint32_t *key;
    const int *col;
    int size;
};

struct RowView {
    const float *x;
    int cols;
    int slots;
    int col0;  // first column of this thread's run (kFromRowRun)
};

// Count into hist the keys >= floor whose bits under mask equal prefix.
template <int E, int SRC, int THREADS>
__device__ __forceinline__ void count_bins(const ListView &list, const RowView &row,
                                           uint32_t floor, uint32_t mask,
                                           uint32_t prefix, int shift, int nb, int *hist) {
    auto visit = [&](uint32_t k) {
        if (k >= floor && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1);
    };
    if (SRC == kFromRowRun) {
#pragma unroll 1
        for (int e = 0; e < E; ++e) {
            const int c = row.col0 + e;
            visit(c < row.cols ? order_key(row.x[c]) : 0u);
        }
    } else if (SRC == kFromList) {
#pragma unroll 1
        for (int i = threadIdx.x; i < list.size; i += THREADS) visit(list.key[i]);
    } else {
#pragma unroll 1
        for (int e = 0; e < row.slots; ++e) {
            const int i = e * THREADS + (int)threadIdx.x;
            visit(i < row.cols ? order_key(row.x[i]) : 0u);
        }
    }
}

// Radix-select the k-th largest key among this thread's keys >= floor
// (summed over the workgroup).  Requires at least k such keys.  Returns T
// and sets *need to the number of keys equal to T that are picked.
template <int E, int SRC, int THREADS>
__device__ __forceinline__ uint32_t radix_threshold(const ListView &list, const RowView &row, int k,
                                                    uint32_t floor, SelectShared &sh, int *need) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < nb; b += THREADS) sh.hist[b] = 0;
        __syncthreads();
        count_bins<E, SRC, THREADS>(list, row, floor, mask, prefix, shift, nb, sh.hist);
        __syncthreads();
        int above;
        const int bin = find_bin(sh, nb, kk, &above);
        kk -= above;
        prefix |= (uint32_t)bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    *need = kk;
    return prefix;
}

// Writes the picks of this thread's keys, which it visits in column order
// (a run of the row, or the contiguous list slice [lo, hi)): one prefix sum
// of packed (greater, equal) counts places every pick.  Counts stay below
// 2^16 (at most 32768 keys per row here), so the low half never carries
// into the high half.
template <int E, int SRC, int THREADS>
__device__ __forceinline__ void place_picks(const ListView &list, const RowView &row, int lo, int hi,
                                            uint32_t T, int need, int32_t *out, SelectShared &sh) {
    auto row_key = [&](int e) {
        const int c = row.col0 + e;
        return c < row.cols ? order_key(row.x[c]) : 0u;
    };
    int gt = 0, eq = 0;
    if (SRC == kFromRowRun) {
#pragma unroll 1
        for (int e = 0; e < E; ++e) {
            const uint32_t k = row_key(e);
            gt += k > T;
            eq += k == T && k != 0u;
        }
    } else {
#pragma unroll 1
        for (int i = lo; i < hi; ++i) {
            gt += list.key[i] > T;
            eq += list.key[i] == T;
        }
    }
    int total;
    const uint32_t base = (uint32_t)block_exclusive_scan<THREADS>((gt << 16) | eq, sh.wave_tmp, &total);
    int gt_before = (int)(base >> 16);
    int eq_before = (int)(base & 0xffffu);
    auto place = [&](uint32_t k, int col) {
        const bool is_gt = k > T;
        const bool is_eq = k == T && k != 0u;
        if (is_gt) out[gt_before + min(eq_before, need)] = col;
        else if (is_eq && eq_before < need) out[gt_before + eq_before] = col;
        gt_before += is_gt;  // counters advance arithmetically (no branches on them)
        eq_before += is_eq;
    };
    if (SRC == kFromRowRun) {
#pragma unroll 1
        for (int e = 0; e < E; ++e) place(row_key(e), row.col0 + e);
    } else {
#pragma unroll 1
        for (int i = lo; i < hi; ++i) place(list.key[i], list.col[i]);
    }
}

// The k-th largest key T of the listed keys and how many keys equal to T
// are picked, by one wave (wave 0).  The list holds each key's top 16 bits
// (key >> 16 << 16); hist0 counts the list by the top 11 bits.  A radix
// select over the top 16 bits (11 + 5) finds T's top half.  If only some of
// the keys sharing it are picked, those keys are re-read in full from the
// row and written back into the list; with at most 64 of them, one per
// lane, T is the kk-th largest by direct comparison, otherwise two 8-bit
// passes over the list finish it.  Keys with other top halves compare with
// T correctly either way.  tied_idx is 64 ints of scratch.  Requires at
// least k listed keys.
__device__ __forceinline__ uint32_t wave_list_select(uint32_t *list, const int *cols, int n, int k,
                                                     const int *hist0, int *hist, int *tied_idx,
                                                     const float *x, int *need_out) {
    const int lane = threadIdx.x & 63;
    int above;
    int kk = k;
    const int b0 = wave_find_bin<2048>(hist0, kk, &above);
    kk -= above;
    // One wave: its LDS operations take effect in issue order.
    if (lane < 32) hist[lane] = 0;
#pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += 256) {
        uint32_t key[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + 64 * u + lane;
            key[u] = i < n ? list[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if ((key[u] >> 21) == (uint32_t)b0) atomicAdd(&hist[(key[u] >> 16) & 31], 1);
    }
    const int b1 = wave_find_bin<32>(hist, kk, &above);
    kk -= above;
    const uint32_t top = ((uint32_t)b0 << 5) | (uint32_t)b1;
    const int tied = hist[b1];  // listed keys whose top half is `top`
    if (kk == tied) {           // all of them are picked
        *need_out = kk;
        return top << 16;
    }
    if (tied <= 64) {
        // Lane p takes the p-th tied entry in list (column) order.
        int base = 0;
#pragma unroll 1
        for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + lane;
            const bool match = i < n && (list[i] >> 16) == top;
            const uint64_t m = __ballot(match);
            if (match) tied_idx[base + __popcll(m & ((1ull << lane) - 1ull))] = i;
            base += __popcll(m);
        }
        uint32_t key = 0u;
        if (lane < tied) {
            const int idx = tied_idx[lane];
            key = order_key(x[cols[idx]]);
            list[idx] = key;
        }
        int gt = 0, eq = 0;
        for (int m = 0; m < tied; ++m) {
            const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)key, m);
            gt += km > key;
            eq += km == key;
        }
        const uint64_t hit = __ballot(lane < tied && gt < kk && kk <= gt + eq);
        const int src = __builtin_ctzll(hit);
        *need_out = kk - __builtin_amdgcn_readlane(gt, src);
        return (uint32_t)__builtin_amdgcn_readlane((int)key, src);
    }
    for (int i = lane; i < n; i += 64)
        if ((list[i] >> 16) == top) list[i] = order_key(x[cols[i]]);
    uint32_t prefix = top << 16, shift_mask = 0xffffu << 16;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 8 : 0;
        for (int b = lane; b < 256; b += 64) hist[b] = 0;
        for (int i = lane; i < n; i += 64) {
            const uint32_t key = list[i];
            if ((key & shift_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
        const int bin = wave_find_bin<256>(hist, kk, &above);
        kk -= above;
        prefix |= (uint32_t)bin << shift;
        shift_mask |= 255u << shift;
    }
    *need_out = kk;
    return prefix;
}

// THREADS threads per row; WPE waves per SIMD the registers are sized for.
template <int E, int THREADS, int WPE>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(WPE)))
void topk_resident_kernel(TopkParams p) {
    constexpr int kListCap = THREADS * 4;  // keys >= floor kept in LDS
    constexpr int kSub = 4;  // sub-runs per thread, one maximum each
    constexpr int kSubLen = (E + kSub - 1) / kSub;
    __shared__ SelectShared sh;
    __shared__ __attribute__((aligned(16))) int hist_list[2048];  // listed keys by their top 11 bits
    __shared__ uint32_t list_key[kListCap];
    __shared__ int list_col[kListCap];
    __shared__ int tied_idx[64];
    __shared__ uint32_t s_floor, s_T;
    __shared__ int s_need;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t row = blockIdx.x;
    const float *x = p.logits + row * p.logits_stride;
    int32_t *out = p.out + row * p.out_stride;
    const int col0 = tid * E;  // this thread's columns: col0 .. col0 + E - 1

    for (int b = tid; b < 2048; b += THREADS) {
        sh.hist[b] = 0;
        hist_list[b] = 0;
    }

    // Keys stay in registers as their top 16 bits, two per register: enough
    // to test key >= floor exactly (the floor is a multiple of 2^21).  The
    // maximum of each sub-run of the thread's keys is kept in full; the
    // sub-run maxima are distinct keys, each witnessing one key >= itself.
    uint32_t top16[(E + 1) / 2];
    uint32_t smax[kSub] = {};
    int cand = 0;
    auto absorb = [&](int e, uint32_t k) {
        cand += k != 0u;
        smax[e / kSubLen] = max(smax[e / kSubLen], k);
        if (e % 2 == 0) top16[e / 2] = k >> 16;
        else top16[e / 2] |= k & 0xffff0000u;
    };
    if (p.vec && col0 + E <= p.num_cols) {
        // The whole run is inside the row: 16-byte loads, all in flight at
        // once (so each cache line is read while its neighbours' loads are
        // still pending, before it can be evicted).
        f32x4 v[E / 4];
#pragma unroll
        for (int e = 0; e < E / 4; ++e) v[e] = *reinterpret_cast<const f32x4 *>(x + col0 + 4 * e);
#pragma unroll
        for (int e = 0; e < E; ++e) absorb(e, order_key(v[e / 4][e % 4]));
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) absorb(e, col0 + e < p.num_cols ? order_key(x[col0 + e]) : 0u);
    }
    auto key_top = [&](int e) { return e % 2 == 0 ? (top16[e / 2] & 0xffffu) : (top16[e / 2] >> 16); };
    int num_cand;
    block_exclusive_scan<THREADS>(cand, sh.wave_tmp, &num_cand);  // its barriers also publish the cleared histograms

    // Paths that need every key again (few candidates, or a list overflow)
    // re-read this thread's run of the row.
    const RowView run{x, p.num_cols, 0, col0};
    const ListView no_list{nullptr, nullptr, 0};
    if (num_cand <= p.k) {
        place_picks<E, kFromRowRun, THREADS>(no_list, run, 0, 0, 0u, 0, out, sh);  // every candidate
    } else {
        // Floor: the lower edge of the 11-bit bin holding the k-th largest
        // sub-run maximum; at least k keys are >= it.  1 (no filtering) when
        // fewer than k sub-runs hold a candidate.
#pragma unroll
        for (int j = 0; j < kSub; ++j)
            if (smax[j] != 0u) atomicAdd(&sh.hist[smax[j] >> 21], 1);
        __syncthreads();
        if (tid < 64) {
            int above;
            const int bin = wave_find_bin<2048>(sh.hist, p.k, &above);
            if (lane == 0) s_floor = bin <= 0 ? 1u : ((uint32_t)bin << 21);
        }
        __syncthreads();
        const uint32_t floor = s_floor;
        // Listed: top half >= floor_top (candidates' top halves are never 0,
        // so floor_top >= 1 also drops the non-candidates).  Counted with
        // integer arithmetic: for 16-bit t and f, (t + 2^16 - f) >> 16 is
        // 1 exactly when t >= f.
        const uint32_t floor_top = max(floor >> 16, 1u);
        uint32_t mine_u = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) mine_u += (key_top(e) + 0x10000u - floor_top) >> 16;
        const int mine = (int)mine_u;
        int listed;
        const int at = block_exclusive_scan<THREADS>(mine, sh.wave_tmp, &listed);
        int need = 0;
        if (listed <= kListCap) {
            // The keys >= floor in column order (top halves), counted by
            // their top 11 bits.
            if (mine > 0) {
                int w = at;
                // The same test as the count above, against a copy of the
                // floor the compiler cannot prove equal, so it recomputes the
                // tests here instead of keeping one lane mask per key alive.
                const uint32_t floor_top2 = __builtin_amdgcn_readfirstlane(floor_top);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint32_t t = key_top(e);
                    const bool in = t >= floor_top2;
                    if (in) {
                        list_key[w] = t << 16;
                        list_col[w] = col0 + e;
                        atomicAdd(&hist_list[t >> 5], 1);
                    }
                    w += in;
                }
            }
            __syncthreads();
            if (tid < 64) {
                const uint32_t T = wave_list_select(list_key, list_col, listed, p.k, hist_list, sh.hist, tied_idx, x, &need);
                if (lane == 0) {
                    s_T = T;
                    s_need = need;
                }
            }
            __syncthreads();
            const uint32_t T = s_T;
            need = s_need;
            // Contiguous slices of the list (column order) per thread.
            const ListView list{list_key, list_col, listed};
            const int per = (listed + THREADS - 1) / THREADS;
            const int lo = min(tid * per, listed), hi = min(lo + per, listed);
            place_picks<E, kFromList, THREADS>(list, run, lo, hi, T, need, out, sh);
        } else {
            // More keys above the floor than the list holds: select and place
            // over the row itself (re-read).
            __syncthreads();
            const uint32_t T = radix_threshold<E, kFromRowRun, THREADS>(no_list, run, p.k, floor, sh, &need);
            place_picks<E, kFromRowRun, THREADS>(no_list, run, 0, 0, T, need, out, sh);
        }
    }
    const int picked = min(num_cand, p.k);
    for (int i = picked + tid; i < p.k; i += THREADS) out[i] = -1;
}

// Rows longer than the register-resident limit: each phase re-reads the row,
// column c owned by thread c % 1024; picks are placed slot by slot.
__global__ __launch_bounds__(1024) void topk_streaming_kernel(TopkParams p) {
    constexpr int kThreads = 1024;
    constexpr int kWaves = kThreads / 64;
    __shared__ SelectShared sh;
    __shared__ int s_cnt[2][kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const float *x = p.logits + row * p.logits_stride;
    int32_t *out = p.out + row * p.out_stride;
    const int slots = (p.num_cols + kThreads - 1) / kThreads;
    auto key_at = [&](int e) {
        const int i = e * kThreads + tid;
        return i < p.num_cols ? order_key(x[i]) : 0u;
    };

    int cand = 0;
    for (int e = 0; e < slots; ++e) cand += key_at(e) != 0u;
    int num_cand;
    block_exclusive_scan<kThreads>(cand, sh.wave_tmp, &num_cand);

    uint32_t T = 0u;
    int need = 0;
    if (num_cand > p.k) {
        const ListView no_list{nullptr, nullptr, 0};
        const RowView mem{x, p.num_cols, slots, 0};
        T = radix_threshold<1, kFromMemory, kThreads>(no_list, mem, p.k, 1u, sh, &need);
    }

    int gt_run = 0, eq_run = 0;  // greater / equal keys in earlier slots
    for (int e = 0; e < slots; ++e) {
        const uint32_t key = key_at(e);
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
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int gt_before = gt_run + gt_wave + __popcll(gt & below);
        const int eq_before = eq_run + eq_wave + __popcll(eq & below);
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

// ---- Fused prefill top-k: the per-row floor and the final select. ----
//
// The fused path never writes the score matrix.  A first pass over the
// scores keeps, per row, the maximum of each 16-key group.  The k-th largest
// group maximum is the floor F: at least k keys of the row are >= F, so every
// key of the row's top k is >= F; and keys > F can lie only in the fewer
// than k groups whose maximum is > F (at most 16 (k-1) keys).  Of the keys
// equal to F only the lowest columns can be picked, so each column chunk
// keeps at most its first k of them.  A second pass writes those candidates,
// per (row, column chunk) segment in column order, and the select below
// takes the exact top k of the concatenated segments (column order), which
// is the top k of the row.

// F per row as a score key: the k-th largest group maximum, or 0 (every
// visible key is a candidate) when fewer than k groups hold a visible key.
// One wave per row, an exact radix select over the keys' 11 + 11 + 10 bits.
// Then each column chunk's room in the row's candidate pool: 16 per group
// whose maximum is above F (every key in it may be), plus the keys equal to
// F it may keep, at most k and at most 16 per group whose maximum is >= F.
// These sum to at most 16 (k - 1) + chunks * k, the pool's size.
__global__ __launch_bounds__(256) void topk_floor_kernel(FusedTopkParams p) {
    __shared__ __attribute__((aligned(16))) int hist[4][2048];
    __shared__ int groups_gt[4][kFusedMaxSegs], groups_eq[4][kFusedMaxSegs];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= p.num_rows) return;  // wave-uniform; this wave works alone below
    const float *g = p.gmax + row * p.gmax_stride;
    int *h = hist[wave];
    uint32_t prefix = 0u, mask = 0u;
    int kk = p.k;
    bool found = true;
    // Rows of up to 64 * kFloorRegs groups keep their keys in registers
    // (lane l: groups l, l + 64, ...), loaded all at once; longer rows are
    // read from memory in each pass.
    constexpr int kFloorRegs = 32;
    const bool in_regs = p.gmax_stride <= 64 * kFloorRegs;
    uint32_t rk[kFloorRegs];
#pragma unroll
    for (int j = 0; j < kFloorRegs; ++j) {
        const int i = lane + 64 * j;
        rk[j] = (in_regs && i < p.gmax_stride) ? order_key(g[i]) : 0u;
    }
    // One wave: its LDS operations take effect in issue order.
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = lane; b < nb; b += 64) h[b] = 0;
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kFloorRegs; ++j) {
                const uint32_t key = rk[j];
                if (key != 0u && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1);
            }
        } else {
            for (int i = lane; i < p.gmax_stride; i += 64) {
                const uint32_t key = order_key(g[i]);
                if (key != 0u && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1);
            }
        }
        int above;
        const int bin = nb == 2048 ? wave_find_bin<2048>(h, kk, &above) : wave_find_bin<1024>(h, kk, &above);
        if (bin < 0) {  // fewer than k visible group maxima
            found = false;
            break;
        }
        kk -= above;
        prefix |= (uint32_t)bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    const uint32_t T = found ? prefix : 0u;
    if (lane == 0) p.floor_key[row] = T;
    int *cgt = groups_gt[wave], *ceq = groups_eq[wave];
    for (int sg = lane; sg < p.segs; sg += 64) {
        cgt[sg] = 0;
        ceq[sg] = 0;
    }
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kFloorRegs; ++j) {
            const int i = lane + 64 * j;
            const uint32_t key = rk[j];
            if (i < p.gmax_stride) {
                const int sg = i / p.groups_per_seg;
                if (key > T) atomicAdd(&cgt[sg], 1);
                else if (key == T && key != 0u) atomicAdd(&ceq[sg], 1);
            }
        }
    } else {
        for (int i = lane; i < p.gmax_stride; i += 64) {
            const uint32_t key = order_key(g[i]);
            const int sg = i / p.groups_per_seg;
            if (key > T) atomicAdd(&cgt[sg], 1);
            else if (key == T && key != 0u) atomicAdd(&ceq[sg], 1);
        }
    }
    int32_t *off = p.seg_off + row * (p.segs + 1);
    int run = 0;
    for (int s0 = 0; s0 < p.segs; s0 += 64) {
        const int sg = s0 + lane;
        int room = 0;
        if (sg < p.segs) room = 16 * cgt[sg] + min(p.k, 16 * (cgt[sg] + ceq[sg]));
        const int incl = (int)wave_inclusive_scan((uint32_t)room);
        if (sg < p.segs) off[sg] = run + incl - room;
        run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) off[p.segs] = run;
}

// The exact top k of one row's candidates: larger keys first, equal keys to
// the lower column (the earlier position, segments being in column order);
// the picks are written in ascending column order, -1 padded.  Lists of up
// to kFusedListCap entries are staged in LDS and reuse the row select above;
// longer ones are read in place.  One workgroup per row.
constexpr int kFusedListCap = 2048;
__global__ __launch_bounds__(256) void topk_candidates_kernel(FusedTopkParams p) {
    constexpr int kThreads = 256;
    __shared__ SelectShared sh;
    __shared__ uint32_t lkey[kFusedListCap];
    __shared__ int lcol[kFusedListCap];
    __shared__ int seg_start[kFusedMaxSegs + 1];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    int32_t *out = p.out + row * p.out_stride;
    const int k = p.k;
    const int segs = p.segs;
    const int64_t rbase = row * (int64_t)p.pool_cap;
    const uint32_t *gkey = p.cand_key + rbase;
    const int32_t *gcol = p.cand_col + rbase;
    const int32_t *off = p.seg_off + row * (segs + 1);
    __shared__ int seg_base[kFusedMaxSegs];
    {
        // Candidates written per segment, never more than the segment's room.
        const int c = (p.cand_cnt && tid < segs) ? min(p.cand_cnt[row * segs + tid], off[tid + 1] - off[tid]) : 0;
        if (tid < segs) seg_base[tid] = off[tid];
        int total;
        const int before = block_exclusive_scan<kThreads>(c, sh.wave_tmp, &total);
        if (tid < segs) seg_start[tid] = before;
        if (tid == 0) seg_start[segs] = total;
        __syncthreads();
    }
    const int n = seg_start[segs];
    // Index into the row's region of candidate number pos (column order).
    auto locate = [&](int pos) {
        int lo = 0, hi = segs - 1;  // the last segment starting at or before pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seg_start[mid] <= pos) lo = mid;
            else hi = mid - 1;
        }
        return (int64_t)seg_base[lo] + (pos - seg_start[lo]);
    };
    if (n <= k) {
        for (int pos = tid; pos < k; pos += kThreads) out[pos] = pos < n ? gcol[locate(pos)] : -1;
        return;
    }
    const RowView none{nullptr, 0, 0, 0};
    if (n <= kFusedListCap) {
        for (int pos = tid; pos < n; pos += kThreads) {
            const int64_t e = locate(pos);
            lkey[pos] = gkey[e];
            lcol[pos] = gcol[e];
        }
        __syncthreads();
        const ListView list{lkey, lcol, n};
        int need;
        const uint32_t T = radix_threshold<1, kFromList, kThreads>(list, none, k, 1u, sh, &need);
        const int per = (n + kThreads - 1) / kThreads;
        const int lo = min(tid * per, n), hi = min(lo + per, n);
        place_picks<1, kFromList, kThreads>(list, none, lo, hi, T, need, out, sh);
        return;
    }
    // Long lists, read in place: the same radix select, counting segment by
    // segment, then placement over contiguous position slices.
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < nb; b += kThreads) sh.hist[b] = 0;
        __syncthreads();
        for (int sgi = 0; sgi < segs; ++sgi) {
            const int cnt = seg_start[sgi + 1] - seg_start[sgi];
            const uint32_t *sk = gkey + seg_base[sgi];
            for (int i = tid; i < cnt; i += kThreads) {
                const uint32_t key = sk[i];
                if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1);
            }
        }
        __syncthreads();
        int above;
        const int bin = find_bin(sh, nb, kk, &above);
        kk -= above;
        prefix |= (uint32_t)bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    const uint32_t T = prefix;
    const int need = kk;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    int gt = 0, eq = 0;
    // The segment holding position pos (the last one starting at or before it).
    auto seg_of = [&](int pos) {
        int a = 0, b = segs - 1;
        while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (seg_start[mid] <= pos) a = mid;
            else b = mid - 1;
        }
        return a;
    };
    if (lo < hi) {
        int sgi = seg_of(lo);
        for (int pos = lo; pos < hi; ++pos) {
            while (pos >= seg_start[sgi + 1]) ++sgi;
            const uint32_t key = gkey[(int64_t)seg_base[sgi] + (pos - seg_start[sgi])];
            gt += key > T;
            eq += key == T;
        }
    }
    int gt_total, eq_total;
    int gt_before = block_exclusive_scan<kThreads>(gt, sh.wave_tmp, &gt_total);
    int eq_before = block_exclusive_scan<kThreads>(eq, sh.wave_tmp, &eq_total);
    if (lo < hi) {
        int sgi = seg_of(lo);
        for (int pos = lo; pos < hi; ++pos) {
            while (pos >= seg_start[sgi + 1]) ++sgi;
            const int64_t e = (int64_t)seg_base[sgi] + (pos - seg_start[sgi]);
            const uint32_t key = gkey[e];
            const bool is_gt = key > T, is_eq = key == T;
            if (is_gt) out[gt_before + min(eq_before, need)] = gcol[e];
            else if (is_eq && eq_before < need) out[gt_before + eq_before] = gcol[e];
            gt_before += is_gt;
            eq_before += is_eq;
        }
    }
}

template <int E, int THREADS, int WPE>
hipError_t launch_resident(const TopkParams &p, hipStream_t stream) {
    return launch_kernel(topk_resident_kernel<E, THREADS, WPE>, dim3((unsigned)p.num_rows),
                         dim3(THREADS), stream, p);
}

// Columns per thread, rounded up to a multiple of 4 (16-byte loads), up to
// MAXE; the caller routes longer rows elsewhere.
template <int THREADS, int WPE, int MAXE, int E = 4>
hipError_t launch_config(const TopkParams &p, hipStream_t stream) {
    const int per = ((p.num_cols + THREADS - 1) / THREADS + 3) / 4 * 4;
    if (per <= E || E == MAXE) return launch_resident<E, THREADS, WPE>(p, stream);
    if constexpr (E + 4 <= MAXE) return launch_config<THREADS, WPE, MAXE, E + 4>(p, stream);
    return hipErrorInvalidValue;  // not reached
}

}  // namespace

hipError_t launch_topk_floor(const FusedTopkParams &p, hipStream_t stream) {
    return launch_kernel(topk_floor_kernel, dim3((unsigned)((p.num_rows + 3) / 4)), dim3(256), stream, p);
}

hipError_t launch_topk_candidates(const FusedTopkParams &p, hipStream_t stream) {
    return launch_kernel(topk_candidates_kernel, dim3((unsigned)p.num_rows), dim3(256), stream, p);
}

hipError_t launch_topk(const TopkParams &p, hipStream_t stream, int num_cus) {
    if (p.num_cols > 32768)  // longer than the register-resident shapes hold
        return launch_kernel(topk_streaming_kernel, dim3((unsigned)p.num_rows), dim3(1024), stream, p);
    // At most one row per CU: the latency of one row is the whole cost, so
    // 1024-thread rows (registers for four waves per SIMD).  Many rows:
    // 512-thread rows, four per CU (registers for eight waves per SIMD),
    // up to 56 columns per thread; longer rows, 1024-thread rows two per CU.
    if (p.num_rows <= (num_cus > 0 ? num_cus : 256)) return launch_config<1024, 4, 32>(p, stream);
    if (p.num_cols <= 512 * 56) return launch_config<512, 8, 56>(p, stream);
    return launch_config<1024, 8, 32>(p, stream);
}

}  // namespace qsa
