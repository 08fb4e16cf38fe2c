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
// Rows up to 32,768 columns (65,535 when there is at most one row per CU)
// stay in registers (as the keys' top 16 bits).
// Thread t of a workgroup of n threads holds the 4-column chunks t, t + n,
// t + 2n, ...: each of its 16-byte loads is part of one contiguous read of
// 16n bytes by the workgroup, so every 128-byte line is fetched by one
// instruction.  Before the select, a floor F is taken from the maxima of
// four sub-sets of each thread's keys: each maximum is a distinct key, so
// when k of them are >= F at least k keys are, and T >= F.  The keys >= F (a
// few hundred for score rows) are compacted in column order into an LDS
// list: column order is chunk-major, so each wave's segment of each chunk is
// placed by a DPP scan of per-lane counts and a scan over the per-(chunk,
// wave) totals.  One wave runs the select over the list without workgroup
// barriers: 11 + 5 bits on the top halves, then, only if some of the keys
// sharing T's top half are left out, those keys are re-read in full and two
// 8-bit passes finish T.  The picks are placed from the list, in column
// order, with a single prefix sum.  Rows with at most k candidates, and
// lists that would overflow, re-read the row as one contiguous run of
// columns per thread.  Longer rows are re-read from memory in each phase.
#include <climits>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kMaxWaves = 16;  // workgroups of at most 1024 threads
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: raw dword access
constexpr int kLoadNT = 2;                // cache policy of the row loads: non-temporal (the "nt" bit)


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
        // Four reads in flight per step (index clamped into the list).
#pragma unroll 1
        for (int i0 = threadIdx.x; i0 < list.size; i0 += 4 * THREADS) {
            uint32_t kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) kb[u] = list.key[min(i0 + u * THREADS, list.size - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + u * THREADS < list.size) visit(kb[u]);
        }
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
// 2^16 (at most 65,535 keys per row here), so the low half never carries
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
// T correctly either way.  tied_idx is 128 ints of scratch.  Requires at
// least k listed keys.
// kFull: the list already holds full keys (nothing is re-read).
template <bool kFull>
__device__ __forceinline__ uint32_t wave_list_select(uint32_t *list, const int *cols, int n, int k,
                                                     const int *hist0, int *hist, int *tied_idx,
                                                     const float *x, int *need_out, uint32_t rel_base) {
    const int lane = threadIdx.x & 63;
    int above;
    int kk = k;
    const int b0 = wave_find_bin<2048>(hist0, kk, &above);
    kk -= above;
    uint32_t top;
    int tied;
    if (rel_base != 0u) {
        // hist0 counts the listed top halves t by t - rel_base: the bin is
        // T's top half itself, and no second pass over the list is needed.
        top = rel_base + (uint32_t)b0;
        tied = hist0[b0];
    } else {
    // One wave: its LDS operations take effect in issue order.
    if (lane < 32) hist[lane] = 0;
#pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += 256) {
        uint32_t key[4];
        // Unconditional reads (index clamped into the list) so the four are
        // in flight together; entries past the end are then dropped.
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = list[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + 64 * u + lane >= n) key[u] = 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if ((key[u] >> 21) == (uint32_t)b0) atomicAdd(&hist[(key[u] >> 16) & 31], 1);
    }
    const int b1 = wave_find_bin<32>(hist, kk, &above);
    kk -= above;
    top = ((uint32_t)b0 << 5) | (uint32_t)b1;
    tied = hist[b1];  // listed keys whose top half is `top`
    }
    if (kk == tied) {           // all of them are picked
        *need_out = kk;
        return top << 16;
    }
    if (tied <= 64) {
        // Lane p takes the p-th tied entry in list (column) order; four
        // 64-entry blocks per step, their reads in flight together.
        int base = 0;
#pragma unroll 1
        for (int i0 = 0; i0 < n; i0 += 256) {
            uint32_t key4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) key4[u] = list[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + 64 * u + lane;
                const bool match = i < n && (key4[u] >> 16) == top;
                const uint64_t m = __ballot(match);
                // Without a branch: lanes that do not match write a slot of
                // their own past the first 64.
                const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                tied_idx[match ? at : 64 + lane] = i;
                base += __popcll(m);
            }
        }
        uint32_t key = 0u;
        if (lane < tied) {
            const int idx = tied_idx[lane];
            if (kFull) {
                key = list[idx];
            } else {
                key = order_key(x[cols[idx]]);
                list[idx] = key;
            }
        }
        // The kk-th largest of the tied keys (kk <= tied), which share the
        // top half: most significant bit first over the low half, counting
        // the keys that still match by ballot.  Keys with a 1 where T has a
        // 0 are above T, so kr ends as the number of keys equal to T picked.
        const bool act = lane < tied;
        uint32_t t = 0u, msk = 0u;
        int kr = kk;
#pragma unroll
        for (int bit = 15; bit >= 0; --bit) {
            const uint32_t b = 1u << bit;
            const int ones = __popcll(__ballot(act && (key & msk) == t && (key & b) != 0u));
            if (kr <= ones) t |= b;
            else kr -= ones;
            msk |= b;
        }
        *need_out = kr;
        return (top << 16) | t;
    }
    for (int i = lane; i < n; i += 64)
        if (!kFull && (list[i] >> 16) == top) list[i] = order_key(x[cols[i]]);
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
// The row's address, length and load shape come first among the kernel
// arguments, where they are preloaded into SGPRs at wave launch: a
// workgroup's row loads go out without waiting on an argument load.
// kFull (rows of at most one per CU, where registers are plentiful): the
// full keys are kept in registers as well and listed in full, so the select
// never re-reads the row for the keys that share T's top half.
template <int E, int THREADS, int WPE, bool kFull>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(WPE)))
void topk_resident_kernel(const float *logits, int64_t logits_stride, int32_t num_cols, int32_t vec_rows,
                          TopkParams p) {
    constexpr int kListCap = THREADS * 4;  // keys >= floor kept in LDS
    constexpr int kSub = 4;  // sub-runs per thread, one maximum each
    constexpr int kSubLen = (E + kSub - 1) / kSub;
    constexpr int kChunks = E / 4;  // 16-byte loads per thread
    constexpr int kWords = (kChunks + 2) / 3;
    constexpr int kWaves = THREADS / 64;
    static_assert(E % 4 == 0 && THREADS % 64 == 0 && THREADS <= 1024, "layout");
    __shared__ SelectShared sh;
    __shared__ int seg_count[kChunks * kWaves];
    __shared__ __attribute__((aligned(16))) int hist_list[2048];  // listed keys by their top 11 bits
    __shared__ uint32_t list_key[kListCap];
    __shared__ int list_col[kListCap];
    __shared__ int tied_idx[128];
    __shared__ uint32_t s_floor, s_T;
    __shared__ int s_need, s_num_cand;
    __shared__ uint32_t s_range[kWaves];  // per wave: largest sub-run maximum << 16 | smallest nonzero one
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const float *x = logits + row * logits_stride;
    int32_t *out = p.out + row * p.out_stride;
    const int col0 = tid * E;  // the thread's run for the re-reading paths: col0 .. col0 + E - 1

    // Keys stay in registers as their top 16 bits, two per register: enough
    // to test key >= floor exactly (the floor is a multiple of 2^16).  The
    // maximum top half of each sub-run of the thread's keys is kept; the
    // sub-run maxima are distinct cells, each witnessing one key >= itself.
    // Element j = 4e + i of this thread is column 4 * (tid + THREADS * e) + i:
    // load e of the workgroup covers 16 * THREADS contiguous bytes, every
    // 128-byte line read by one instruction of one wave.
    uint32_t top16[(E + 1) / 2];
    uint32_t full[kFull ? E : 1];
    uint32_t smax[kSub] = {};
    int cand = 0;
    auto absorb = [&](int e, uint32_t k) {
        if (kFull) full[e] = k;
        cand += k != 0u;
        smax[e / kSubLen] = max(smax[e / kSubLen], k >> 16);
        if (e % 2 == 0) top16[e / 2] = k >> 16;
        else top16[e / 2] |= k & 0xffff0000u;
    };
    auto chunk_col = [&](int e) { return 4 * (tid + THREADS * e); };
    if (vec_rows) {
        // All of the thread's 16-byte loads in flight at once, and none of
        // them conditional, so each chunk's keys are formed as soon as its
        // load lands: the row is one buffer resource (a load past its end
        // returns zeros), and the cells of chunks past the end are compared
        // with +inf instead of -inf, so none of them is a candidate.
        // The loads are non-temporal (the rows are read once; every line is
        // read whole by one instruction): the prefill that runs next then finds
        // its keys and queries still in the caches (the step's prefill measured
        // 3% faster; this kernel the same).
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, num_cols * 4, kBufferWord3);
        f32x4 v[kChunks];
#pragma unroll
        for (int e = 0; e < kChunks; ++e)
            v[e] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * (tid + THREADS * e), 0, kLoadNT));
        // Every load issued before any key is formed: the chunks are then
        // consumed in load order, each freeing its registers.
        __builtin_amdgcn_sched_barrier(0);
        // The key of a candidate f (> -inf, not NaN) is order_key(f): the
        // bits of f + 0 (which turns -0 into +0 and changes nothing else,
        // fp32 denormals being kept) with the sign bit set when it is clear,
        // all bits flipped when it is set.  Candidates are counted per wave
        // (ballot) rather than per lane.
        uint32_t wcand = 0u;
#pragma unroll
        for (int e = 0; e < kChunks; ++e) {
            const float bound = chunk_col(e) < num_cols ? neg_inf() : __builtin_inff();
            uint32_t k[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = v[e][i];
                const bool is_cand = f > bound;
                const uint32_t u = __float_as_uint(f + 0.0f);
                const uint32_t sgn = (uint32_t)((int32_t)u >> 31);
                k[i] = is_cand ? u ^ (sgn | 0x80000000u) : 0u;
                if (kFull) full[4 * e + i] = k[i];
                wcand += (uint32_t)__popcll(__ballot(is_cand));
            }
            // Top halves, two to a register (even key low).
            top16[2 * e] = __builtin_amdgcn_perm(k[1], k[0], 0x07060302u);
            top16[2 * e + 1] = __builtin_amdgcn_perm(k[3], k[2], 0x07060302u);
        }
        cand = lane == 0 ? (int)wcand : 0;
        // Sub-run maxima of the top halves (sub-run j: the chunks e with
        // kSub e / kChunks == j), two halves at a time.
        u16x2 m2[kSub];
#pragma unroll
        for (int j = 0; j < kSub; ++j) m2[j] = u16x2{0, 0};
#pragma unroll
        for (int e = 0; e < kChunks; ++e) {
            const int j = kSub * e / kChunks;
            m2[j] = __builtin_elementwise_max(m2[j], __builtin_elementwise_max(__builtin_bit_cast(u16x2, top16[2 * e]),
                                                                               __builtin_bit_cast(u16x2, top16[2 * e + 1])));
        }
#pragma unroll
        for (int j = 0; j < kSub; ++j) smax[j] = max((uint32_t)m2[j][0], (uint32_t)m2[j][1]);
    } else {
        // Rows without 16-byte alignment or with a ragged last chunk.
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = chunk_col(e / 4) + e % 4;
            absorb(e, c < num_cols ? order_key(x[c]) : 0u);
        }
    }
    auto key_top = [&](int e) { return e % 2 == 0 ? (top16[e / 2] & 0xffffu) : (top16[e / 2] >> 16); };
    // The histograms are cleared after the row's loads are issued.
    for (int b = tid; b < 2048; b += THREADS) {
        sh.hist[b] = 0;
        hist_list[b] = 0;
    }
    // The range of the sub-run maxima (top halves) per wave, published by
    // the scan's barriers: when they span fewer than 2,048 values the floor
    // takes one histogram pass.
    {
        uint32_t mx = 0u, mn = 0xffffu;
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            mx = max(mx, smax[j]);
            mn = min(mn, smax[j] != 0u ? smax[j] : 0xffffu);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        }
        if (lane == 0) s_range[wave] = (mx << 16) | mn;
    }
    int num_cand;
    block_exclusive_scan<THREADS>(cand, sh.wave_tmp, &num_cand);  // its barriers also publish the cleared histograms
    if (tid == 0) s_num_cand = num_cand;  // read after later barriers

    // Paths that need every key again (few candidates, or a list overflow)
    // re-read this thread's run of the row.
    const RowView run{x, num_cols, 0, col0};
    const ListView no_list{nullptr, nullptr, 0};
    if (num_cand <= p.k) {
        place_picks<E, kFromRowRun, THREADS>(no_list, run, 0, 0, 0u, 0, out, sh);  // every candidate
    } else {
        // Floor: the lower edge of the 16-bit bin holding the k-th largest
        // sub-run maximum (its top 11 bits, then the next 5 among the
        // maxima in that bin); at least k keys are >= it.  16 bits rather
        // than 11 keep the list short when scores spread evenly over the
        // 11-bit bin.  1 (no filtering) when fewer than k sub-runs hold a
        // candidate.
        uint32_t mx = 0u, mn = 0xffffu;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mx = max(mx, s_range[w] >> 16);
            mn = min(mn, s_range[w] & 0xffffu);
        }
        // One pass when the maxima span fewer than 2,048 values: bin b is the
        // top half mn + b itself, so the bin of the k-th largest maximum is
        // the 16-bit floor.
        const bool one_pass = mn <= mx && mx - mn < 2048u;
#pragma unroll
        for (int j = 0; j < kSub; ++j)
            if (smax[j] != 0u) atomicAdd(&sh.hist[one_pass ? smax[j] - mn : smax[j] >> 5], 1);
        __syncthreads();
        if (tid < 64) {
            int above;
            const int bin = wave_find_bin<2048>(sh.hist, p.k, &above);
            if (lane == 0) {
                if (one_pass) s_floor = bin < 0 ? 1u : ((mn + (uint32_t)bin) << 16);
                else s_floor = bin <= 0 ? 1u : ((uint32_t)bin << 21);
                s_need = p.k - above;  // rank of the k-th largest maximum within its bin
            }
        }
        __syncthreads();
        if (!one_pass && s_floor > 1u) {  // uniform; hist_list is still all zero here
            const uint32_t b0 = s_floor >> 21;
#pragma unroll
            for (int j = 0; j < kSub; ++j)
                if ((smax[j] >> 5) == b0) atomicAdd(&hist_list[smax[j] & 31], 1);
            __syncthreads();
            if (tid < 64) {
                int above;
                const int b1 = wave_find_bin<32>(hist_list, s_need, &above);
                if (lane == 0) s_floor |= (uint32_t)b1 << 16;
            }
            __syncthreads();
            if (tid < 32) hist_list[tid] = 0;  // the list's histogram starts from zero
        }
        const uint32_t floor = s_floor;
        // Listed: top half >= floor_top (candidates' top halves are never 0,
        // so floor_top >= 1 also drops the non-candidates).  Counted with
        // integer arithmetic: for 16-bit t and f, (t + 2^16 - f) >> 16 is
        // 1 exactly when t >= f.
        const uint32_t floor_top = max(floor >> 16, 1u);
        // The list's histogram: by t - floor_top when every listed top half
        // lies within 2,048 values of the floor (mx is the row's largest),
        // so that its bin is the exact top half; else by the top 11 bits.
        // Rows with full keys kept (at most one row per CU) stay on the
        // 11 + 5-bit form: their own select is 0.3 us faster relative, but
        // the next decode launch then measures 0.4 us slower.
        const uint32_t rel_base = !kFull && mx >= floor_top && mx - floor_top < 2048u ? floor_top : 0u;
        const uint32_t hist_shift = rel_base != 0u ? 0u : 5u;
        // The list in column order is chunk-major (chunk e of wave w covers
        // columns 2048e + 256w .. +255 at 512 threads): wave w's segment of
        // chunk e follows every segment of chunks before e and those of
        // waves before w in chunk e.  Per-lane counts of each chunk, three
        // 10-bit fields to a word (a wave's count per chunk is at most 256),
        // are scanned across the wave with DPP.
        // Bit i of chunk_bits(e, f): key 4e + i is listed (top half >= f).
        auto chunk_bits = [&](int e, uint32_t f) {
            const uint32_t a = top16[2 * e], b = top16[2 * e + 1];
            return (uint32_t)((a & 0xffffu) >= f) | ((uint32_t)((a >> 16) >= f) << 1) |
                   ((uint32_t)((b & 0xffffu) >= f) << 2) | ((uint32_t)((b >> 16) >= f) << 3);
        };
        uint32_t packed[kWords], incl[kWords];
#pragma unroll
        for (int w = 0; w < kWords; ++w) packed[w] = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e)
            packed[e / 12] += ((key_top(e) + 0x10000u - floor_top) >> 16) << (10 * ((e / 4) % 3));
#pragma unroll
        for (int w = 0; w < kWords; ++w) incl[w] = wave_inclusive_scan(packed[w]);
        if (lane == 63) {
#pragma unroll
            for (int e = 0; e < kChunks; ++e) seg_count[e * kWaves + wave] = (int)((incl[e / 3] >> (10 * (e % 3))) & 1023u);
        }
#pragma unroll
        for (int w = 0; w < kWords; ++w) incl[w] -= packed[w];  // exclusive from here on
        __syncthreads();
        // Lane c (< kChunks) of every wave: the chunk's total and this wave's
        // offset within it, then a scan over chunks.
        int tot = 0, pre = 0;
        if (lane < kChunks) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const int sc = seg_count[lane * kWaves + w];
                tot += sc;
                pre += w < wave ? sc : 0;
            }
        }
        const int tot_incl = (int)wave_inclusive_scan((uint32_t)tot);
        const int seg_off = tot_incl - tot + pre;
        const int listed = __builtin_amdgcn_readlane(tot_incl, 63);
        int need = 0;
        if (listed <= kListCap) {
            // The keys >= floor in column order (top halves), counted by
            // their top 11 bits.  Each lane visits only its listed keys of a
            // chunk (a few percent of the cells on score rows), by their
            // bits; the bits are formed again, against a copy of the floor
            // the compiler cannot prove equal, rather than kept from the
            // count above (one register per chunk).
            const uint32_t floor_top2 = __builtin_amdgcn_readfirstlane(floor_top);
#pragma unroll
            for (int e = 0; e < kChunks; ++e) {
                int w = __builtin_amdgcn_readlane(seg_off, e) + (int)((incl[e / 3] >> (10 * (e % 3))) & 1023u);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t t = key_top(4 * e + i);
                    const bool in = t >= floor_top2;
                    if (in) {
                        list_key[w] = kFull ? full[4 * e + i] : t << 16;
                        list_col[w] = chunk_col(e) + i;
                        atomicAdd(&hist_list[(t - rel_base) >> hist_shift], 1);
                    }
                    w += in;
                }
            }
            __syncthreads();
            if (tid < 64) {
                const uint32_t T =
                    wave_list_select<kFull>(list_key, list_col, listed, p.k, hist_list, sh.hist, tied_idx, x, &need,
                                            rel_base);
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
    // The candidate count from LDS rather than a register kept live (and
    // spilled) through the select.
    const int picked = min(s_num_cand, p.k);
    for (int i = picked + tid; i < p.k; i += THREADS) out[i] = -1;
}

// One row x[0 .. num_cols) by a 1024-thread workgroup, re-read from memory
// in each phase: column c owned by thread c % 1024; picks are placed slot by
// slot.  Used for rows longer than the register-resident limit, and by the
// fused path's fallback on rows it rescored into scratch.
__device__ __forceinline__ void streaming_select(const float *x, int num_cols, int32_t *out, int k) {
    constexpr int kThreads = 1024;
    constexpr int kWaves = kThreads / 64;
    __shared__ SelectShared sh;
    __shared__ int s_cnt[2][kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int slots = (num_cols + kThreads - 1) / kThreads;
    auto key_at = [&](int e) {
        const int i = e * kThreads + tid;
        return i < num_cols ? order_key(x[i]) : 0u;
    };

    int cand = 0;
    for (int e = 0; e < slots; ++e) cand += key_at(e) != 0u;
    int num_cand;
    block_exclusive_scan<kThreads>(cand, sh.wave_tmp, &num_cand);

    uint32_t T = 0u;
    int need = 0;
    if (num_cand > k) {
        const ListView no_list{nullptr, nullptr, 0};
        const RowView mem{x, num_cols, slots, 0};
        T = radix_threshold<1, kFromMemory, kThreads>(no_list, mem, k, 1u, sh, &need);
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
    const int picked = min(num_cand, k);
    for (int i = picked + tid; i < k; i += kThreads) out[i] = -1;
}

__global__ __launch_bounds__(1024) void topk_streaming_kernel(TopkParams p) {
    const int64_t row = blockIdx.x;
    streaming_select(p.logits + row * p.logits_stride, p.num_cols, p.out + row * p.out_stride, p.k);
}

// ---- Fused prefill top-k: the per-row floor and the final select. ----
//
// The fused path never writes the score matrix.  A first pass over the
// scores keeps, per row, the maximum of each group of G = kFusedGroupKeys
// keys.  The k-th largest group maximum is the floor F: at least k keys of
// the row are >= F, so every key of the row's top k is >= F; and keys > F
// can lie only in the fewer than k groups whose maximum is > F (at most
// G (k-1) keys).  Of the keys
// equal to F only the lowest columns can be picked, so each column chunk
// keeps at most its first k of them.  A second pass writes those candidates,
// per (row, column chunk) segment in column order, and the select below
// takes the exact top k of the concatenated segments (column order), which
// is the top k of the row.

// F per row as a score key: the k-th largest group maximum, or 0 (every
// visible key is a candidate) when fewer than k groups hold a visible key.
// One wave per row, an exact radix select over the keys' bits below the
// ones every visible group maximum shares: those are known from the row's
// OR and AND, so the first 11-bit histogram spreads over the row's own range
// (the top bits of similar scores fall in a few bins, whose LDS atomics
// would serialise).  Then each column chunk's room in the row's candidate
// pool: G per group whose maximum is above F (every key in it may be), plus
// the keys equal to F it may keep, at most k and at most G per group whose
// maximum is >= F, and never more than the chunk's columns.  These sum to at
// most min(G (k - 1) + chunks * k, columns), the pool's size.
__global__ __launch_bounds__(256) void topk_floor_kernel(FusedTopkParams p) {
    __shared__ __attribute__((aligned(16))) int hist[4][2048];
    __shared__ int groups_gt[4][kFusedMaxSegs], groups_eq[4][kFusedMaxSegs];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: row, g and g_rsrc are scalar
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= p.num_rows) return;  // wave-uniform; this wave works alone below
    const float *g = p.gmax + row * p.gmax_stride;
    int *h = hist[wave];
    // Rows of up to 64 * kFloorRegs groups keep their keys in registers
    // (lane l: groups l, l + 64, ...), loaded all at once; longer rows are
    // read from memory in each pass.
    constexpr int kFloorRegs = 64;
    const bool in_regs = p.gmax_stride <= 64 * kFloorRegs;
    // Unconditional loads through a buffer resource bounded by the row (a
    // load past its end returns 0, and none are made when the row is read
    // from memory instead), so all of them are in flight at once; lanes past
    // the row's end then drop theirs.
    const __amdgpu_buffer_rsrc_t g_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(g), 0, in_regs ? p.gmax_stride * 4 : 0, kBufferWord3);
    uint32_t rk[kFloorRegs];
#pragma unroll
    for (int j = 0; j < kFloorRegs; ++j) rk[j] = __builtin_amdgcn_raw_buffer_load_b32(g_rsrc, lane * 4, 256 * j, 0);
#pragma unroll
    for (int j = 0; j < kFloorRegs; ++j)
        rk[j] = lane < p.gmax_stride - 64 * j ? order_key(__uint_as_float(rk[j])) : 0u;
    // Count, OR and AND of the visible keys (key 0 is never picked).
    uint32_t kor = 0u, kand = ~0u;
    int nz = 0;
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kFloorRegs; ++j) {
            const uint32_t key = rk[j];
            kor |= key;
            kand &= key != 0u ? key : ~0u;
            nz += key != 0u;
        }
    } else {
        for (int i = lane; i < p.gmax_stride; i += 64) {
            const uint32_t key = order_key(g[i]);
            kor |= key;
            kand &= key != 0u ? key : ~0u;
            nz += key != 0u;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        kor |= (uint32_t)__shfl_xor((int)kor, o);
        kand &= (uint32_t)__shfl_xor((int)kand, o);
        nz += __shfl_xor(nz, o);
    }
    // Fewer than k visible group maxima: no floor (every visible key is a
    // candidate).  Otherwise the low `bits` bits are still open.
    const bool found = __builtin_amdgcn_readfirstlane(nz) >= p.k;
    const uint32_t diff = __builtin_amdgcn_readfirstlane(kor ^ kand);
    int bits = diff == 0u ? 0 : 32 - __builtin_clz(diff);
    uint32_t mask = bits == 32 ? 0u : ~0u << bits;
    uint32_t prefix = __builtin_amdgcn_readfirstlane(kand) & mask;
    int kk = p.k;
    // One wave: its LDS operations take effect in issue order.
#pragma unroll 1
    while (found && bits > 0) {
        const int w = bits < 11 ? bits : 11;
        const int shift = bits - w;
        const uint32_t digit = (1u << w) - 1u;
        // wave_find_bin scans all 2048 bins: clear them all.
#pragma unroll
        for (int b = 0; b < 2048 / 256; ++b) reinterpret_cast<int4 *>(h)[lane + 64 * b] = int4{0, 0, 0, 0};
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kFloorRegs; ++j) {
                const uint32_t key = rk[j];
                if (key != 0u && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & digit], 1);
            }
        } else {
            for (int i = lane; i < p.gmax_stride; i += 64) {
                const uint32_t key = order_key(g[i]);
                if (key != 0u && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & digit], 1);
            }
        }
        int above;
        const int bin = wave_find_bin<2048>(h, kk, &above);  // >= 0: at least kk keys match the prefix
        kk -= above;
        prefix |= (uint32_t)bin << shift;
        mask |= digit << shift;
        bits = shift;
    }
    const uint32_t T = found ? prefix : 0u;
    if (lane == 0) p.floor_key[row] = T;
    int *cgt = groups_gt[wave], *ceq = groups_eq[wave];
    for (int sg = lane; sg < p.segs; sg += 64) {
        cgt[sg] = 0;
        ceq[sg] = 0;
    }
    if (in_regs) {
        // Segments hold a multiple of 32 groups (chunks are multiples of 256
        // columns), so lanes 0-31 and 32-63 of register j each lie in one
        // segment: counted by ballots, summed in scalar registers and
        // written once per segment (segments come in increasing order).
        // The segment of group i is a multiply-high, exact while
        // i * groups_per_seg < 2^32 (here both are at most 4,096).
        const uint32_t seg_magic = 0xFFFFFFFFu / (uint32_t)p.groups_per_seg + 1u;
        int cur = 0, agt = 0, aeq = 0;
        auto add_half = [&](int sg, int ng, int ne) {
            if (sg != cur) {
                if (lane == 0) {
                    cgt[cur] = agt;
                    ceq[cur] = aeq;
                }
                cur = sg;
                agt = 0;
                aeq = 0;
            }
            agt += ng;
            aeq += ne;
        };
#pragma unroll
        for (int j = 0; j < kFloorRegs; ++j) {
            if (64 * j < p.gmax_stride) {  // keys past the row's end are 0: never counted
                const uint64_t mg = __ballot(rk[j] > T);
                const uint64_t me = __ballot(rk[j] == T && rk[j] != 0u);
                add_half((int)__umulhi((uint32_t)(64 * j), seg_magic), __popc((uint32_t)mg), __popc((uint32_t)me));
                add_half((int)__umulhi((uint32_t)(64 * j + 32), seg_magic), __popc((uint32_t)(mg >> 32)),
                         __popc((uint32_t)(me >> 32)));
            }
        }
        if (lane == 0) {
            cgt[cur] = agt;
            ceq[cur] = aeq;
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
        if (sg < p.segs) {
            // No more than the chunk's cells either, so a row's segments
            // never exceed its columns.
            constexpr int G = kFusedGroupKeys;
            const int seg_cols = min(G * p.groups_per_seg, p.out_cols - sg * G * p.groups_per_seg);
            room = min(G * cgt[sg] + min(p.k, G * (cgt[sg] + ceq[sg])), seg_cols);
        }
        const int incl = (int)wave_inclusive_scan((uint32_t)room);
        if (sg < p.segs) off[sg] = run + incl - room;
        run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) off[p.segs] = run;
}

// The exact top k of one row's candidates: larger keys first, equal keys to
// the lower column (the earlier position, segments being in column order);
// the picks are written in ascending column order, -1 padded.  Lists of up
// to kCap entries are staged in LDS and reuse the row select above;
// longer ones are read in place.  One workgroup per row.
template <int kCap>
__global__ __launch_bounds__(256) void topk_candidates_kernel(FusedTopkParams p) {
    constexpr int kThreads = 256;
    __shared__ SelectShared sh;
    __shared__ uint32_t lkey[kCap];
    __shared__ int lcol[kCap];
    __shared__ int seg_start[kFusedMaxSegs + 1];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    int32_t *out = p.out + row * p.out_stride;
    const int k = p.k;
    const int segs = p.segs;
    const int64_t rbase = row * (int64_t)p.pool_cap;
    // Entry e: the score's bits at 2e (a score >= +0: its key is them with
    // the sign bit set), its column at 2e + 1.
    const uint32_t *gcand = p.cand + 2 * rbase;
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
        for (int pos = tid; pos < k; pos += kThreads) out[pos] = pos < n ? (int32_t)gcand[2 * locate(pos) + 1] : -1;
        return;
    }
    const RowView none{nullptr, 0, 0, 0};
    if (n <= kCap) {
        // Every entry's 8-byte load in flight at once (positions past the
        // list read its last entry again and are dropped).
        constexpr int kPer = kCap / kThreads;
        u32x2 ent[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j * kThreads < n)  // uniform
                ent[j] = *reinterpret_cast<const u32x2 *>(gcand + 2 * locate(min(tid + kThreads * j, n - 1)));
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int pos = tid + kThreads * j;
            if (j * kThreads < n && pos < n) {
                lkey[pos] = ent[j][0] | 0x80000000u;
                lcol[pos] = (int32_t)ent[j][1];
            }
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
    // Long lists, read in place: the same radix select, then placement over
    // contiguous position slices.  Entries are read kBatch at a time with
    // their loads in flight together; a thread's positions only increase,
    // so its segment is tracked as it goes.
    constexpr int kBatch = 8;
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
    // Entry index of position pos (< n), at or after the last one asked for.
    auto entry_of = [&](int pos, int &sgi) {
        while (pos >= seg_start[sgi + 1]) ++sgi;
        return (int64_t)seg_base[sgi] + (pos - seg_start[sgi]);
    };
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < nb; b += kThreads) sh.hist[b] = 0;
        __syncthreads();
        int sgi = seg_of(min(tid, n - 1));
#pragma unroll 1
        for (int p0 = 0; p0 < n; p0 += kThreads * kBatch) {
            uint32_t kb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) kb[j] = gcand[2 * entry_of(min(p0 + tid + kThreads * j, n - 1), sgi)];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const uint32_t key = kb[j] | 0x80000000u;
                if (p0 + tid + kThreads * j < n && (key & mask) == prefix)
                    atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1);
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
    if (lo < hi) {
        int sgi = seg_of(lo);
#pragma unroll 1
        for (int b0 = lo; b0 < hi; b0 += kBatch) {
            uint32_t kb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) kb[j] = gcand[2 * entry_of(min(b0 + j, hi - 1), sgi)];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const uint32_t key = kb[j] | 0x80000000u;
                if (b0 + j < hi) {
                    gt += key > T;
                    eq += key == T;
                }
            }
        }
    }
    int gt_total, eq_total;
    int gt_before = block_exclusive_scan<kThreads>(gt, sh.wave_tmp, &gt_total);
    int eq_before = block_exclusive_scan<kThreads>(eq, sh.wave_tmp, &eq_total);
    if (lo < hi) {
        int sgi = seg_of(lo);
#pragma unroll 1
        for (int b0 = lo; b0 < hi; b0 += kBatch) {
            u32x2 eb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                eb[j] = *reinterpret_cast<const u32x2 *>(gcand + 2 * entry_of(min(b0 + j, hi - 1), sgi));
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j >= hi) break;
                const uint32_t key = eb[j][0] | 0x80000000u;
                const bool is_gt = key > T, is_eq = key == T;
                // Slots below k by construction (gt_total + need = k); checked
                // all the same, so an inconsistent pool cannot write past the row.
                const int at = is_gt ? gt_before + min(eq_before, need) : gt_before + eq_before;
                if ((is_gt || (is_eq && eq_before < need)) && at < k) out[at] = (int32_t)eb[j][1];
                gt_before += is_gt;
                eq_before += is_eq;
            }
        }
    }
}

// ---- Fused prefill top-k over score keys (rows of at most 32,768 columns). ----
//
// The prefill pass stores, per cell, the top 16 bits of the score's order
// key (2 bytes instead of the 4-byte score).  Picking on those prefixes is
// exact except among the cells whose prefix equals that of the k-th largest
// key: only there do the low 16 bits decide.  Those cells (a few dozen per
// row on score rows) are rescored with the prefill's own MFMA sequence (the
// same operands, instruction, feature order and epilogue, so the same bits)
// and ranked on their full keys.  Rows the in-register select cannot finish
// go to a fallback that rescores the whole row.

// Full order keys of 64 cells of prefill row `row`, one per lane: lane l's
// cell is key index key_idx (which every lane must hold in [0, num_keys)).
// The MFMA instruction (bf16 or fp16) and layout are the prefill kernel's:
// A lane (n, q4) holds head n % 4 of the row, features 32 ks + 8 q4 .. +7 in
// k-step ks, so every group of 4 result rows holds the 4 head dots; B lane
// (n, q4) of group g holds the same features of lane 16 g + n's key.  Lane
// l = 16 q4 + n takes group q4's result, which its own lane holds.
// q_lds: the row's four heads (4 x 128 elements, head-major) staged in LDS,
// or null to read them from memory.
template <bool kF16>
__device__ __forceinline__ uint32_t rescore_key(const Keys16TopkParams &p, int64_t row, int64_t key_idx,
                                                const uint16_t *q_lds = nullptr) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, q4 = lane >> 4;
    const uint16_t *qrow = q_lds ? q_lds + (n & 3) * 128 + 8 * q4
                                 : p.q + row * p.q_stride_row + (int64_t)(n & 3) * p.q_stride_head + 8 * q4;
    u32x4 a[4], b[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = load_u32x4(qrow + 32 * ks);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int lo = __shfl((int)(uint32_t)key_idx, 16 * g + n, 64);
        const int hi = __shfl((int)(uint32_t)((uint64_t)key_idx >> 32), 16 * g + n, 64);
        const int64_t kg = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
        const uint16_t *krow = p.kv + kg * p.k_stride + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[g][ks] = load_u32x4(krow + 32 * ks);
    }
    f32x4 acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[g] = mfma_qk<kF16>(a[ks], b[g][ks], acc[g]);
    }
    const f32x4 mine = q4 == 0 ? acc[0] : (q4 == 1 ? acc[1] : (q4 == 2 ? acc[2] : acc[3]));
    return order_key(head_sum_score(mine, p.scale));
}

// Wave 0's select over the listed keys (entries key16 << 16 | column, in
// column order; hist0 counts them by the top 11 bits of key16).  Returns
// T16 such that the picks are exactly the entries whose key16 is > T16,
// after rewriting the entries that share the k-th largest prefix: a picked
// one gets key16 0xffff, the others 0.  Returns -1 when the row needs the
// fallback (more than 64 entries share that prefix and only some are
// picked, or a rescored key disagrees with its stored prefix).  Requires
// more than k listed entries.
template <bool kF16>
__device__ __forceinline__ int wave_select_keys16(uint32_t *list, int n, int k, const int *hist0, int *hist,
                                                  int *tied_idx, const Keys16TopkParams &p, int64_t row,
                                                  int64_t start, const uint16_t *q_lds) {
    const int lane = threadIdx.x & 63;
    int above;
    int kk = k;
    const int b0 = wave_find_bin<2048>(hist0, kk, &above);
    kk -= above;
    // One wave: its LDS operations take effect in issue order.
    if (lane < 32) hist[lane] = 0;
#pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += 256) {
        uint32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = list[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + 64 * u + lane < n && (e[u] >> 21) == (uint32_t)b0) atomicAdd(&hist[(e[u] >> 16) & 31], 1);
    }
    const int b1 = wave_find_bin<32>(hist, kk, &above);
    kk -= above;
    const uint32_t top = ((uint32_t)b0 << 5) | (uint32_t)b1;
    const int tied = hist[b1];  // entries whose key16 is `top`
    if (kk == tied) return (int)top - 1;  // all of them are picked
    if (tied > 64) return -1;
    // Lane p takes the p-th tied entry in list (column) order.
    int base = 0;
#pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += 256) {
        uint32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = list[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + 64 * u + lane;
            const bool match = i < n && (e[u] >> 16) == top;
            const uint64_t m = __ballot(match);
            const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            tied_idx[match ? at : 64 + lane] = i;
            base += __popcll(m);
        }
    }
    const bool act = lane < tied;
    const int idx = tied_idx[act ? lane : 0];
    const uint32_t entry = list[idx];
    const int col = (int)(entry & 0xffffu);
    const uint32_t key = rescore_key<kF16>(p, row, start + col, q_lds);
    if (__ballot(act && (key >> 16) != top) != 0ull) return -1;
    // The kk-th largest of the tied keys (kk < tied), most significant bit
    // first over the low half; kr ends as the number of keys equal to T
    // that are picked (the lowest columns, i.e. the lowest lanes).
    uint32_t t = 0u, msk = 0u;
    int kr = kk;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t bb = 1u << bit;
        const int ones = __popcll(__ballot(act && (key & msk) == t && (key & bb) != 0u));
        if (kr <= ones) t |= bb;
        else kr -= ones;
        msk |= bb;
    }
    const uint32_t T = (top << 16) | t;
    const uint64_t eqm = __ballot(act && key == T);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const bool picked = act && (key > T || (key == T && __popcll(eqm & below) < kr));
    if (act) list[idx] = (picked ? 0xffff0000u : 0u) | (entry & 0xffffu);
    return (int)top;
}

// One row per workgroup of THREADS threads, E keys per thread (a multiple
// of 8): thread t holds the 8-key chunks t, t + THREADS, ..., as loaded (two
// keys per register), so each 16-byte load is part of one contiguous read
// of 16 * THREADS bytes.  The row buffer resource covers the row's padded
// width; the padding holds key 0, and loads past it return 0.  Floor from
// the maxima of the chunks (distinct cells), list of the keys >= floor in
// column order, one-wave select, placement from the list.
template <int E, int THREADS, int WPE, bool kF16>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(WPE)))
void topk_keys16_kernel(const uint16_t *keys, int64_t keys_stride, Keys16TopkParams p) {
    constexpr int kChunks = E / 8;
    constexpr int kWaves = THREADS / 64;
    constexpr int kListCap = 4096;
    static_assert(E % 8 == 0 && E <= 64 && THREADS % 64 == 0, "layout");
    __shared__ SelectShared sh;
    __shared__ int seg_count[kChunks * kWaves];
    __shared__ __attribute__((aligned(16))) int hist_list[2048];  // listed keys by their top 11 bits
    __shared__ uint32_t list[kListCap];
    __shared__ int tied_idx[128];
    __shared__ uint32_t s_floor;
    __shared__ uint32_t s_range[kWaves];  // per wave: largest chunk maximum << 16 | smallest nonzero one
    __shared__ int s_need, s_T;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[kHeads * kDim];  // the row's queries, for rescoring
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    // The row's queries (1 KB) are read ahead of its keys and staged in LDS,
    // so the rescoring of tied cells does not wait on them.
    u32x4 qv = zero_u32x4();
    if (tid < 64) qv = load_u32x4(p.q + row * p.q_stride_row + (int64_t)(tid >> 4) * p.q_stride_head + 8 * (tid & 15));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(keys + row * keys_stride), 0, (int)(keys_stride * 2), kBufferWord3);
    u32x4 w[kChunks];
#pragma unroll
    for (int e = 0; e < kChunks; ++e)
        w[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * (tid + THREADS * e), 0, kLoadNT));
    auto chunk_col = [&](int e) { return 8 * (tid + THREADS * e); };
    auto key_at = [&](int j) {  // key j (0 .. E-1) of this thread
        const uint32_t v = w[j / 8][(j % 8) / 2];
        return (j & 1) ? (v >> 16) : (v & 0xffffu);
    };
    for (int b = tid; b < 2048; b += THREADS) {
        sh.hist[b] = 0;
        hist_list[b] = 0;
    }
    if (tid < 64) *reinterpret_cast<u32x4 *>(&q_lds[8 * tid]) = qv;
    const int64_t start = p.row_k_start[row];
    int32_t *out = p.out + row * p.out_stride;

    // Floor: the k-th largest chunk maximum; at least k keys are >= it.  When
    // the maxima span fewer than 2,048 values (published per wave with the
    // cleared histograms), one histogram pass over maximum - smallest gives
    // it exactly; otherwise the lower edge of its 16-bit bin (top 11 bits,
    // then the next 5 among the maxima in that bin).  1 when fewer than k
    // chunks hold a candidate (every candidate is listed).
    uint32_t cmax[kChunks];
    uint32_t mx = 0u, mn = 0xffffu;
#pragma unroll
    for (int e = 0; e < kChunks; ++e) {
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(w[e][i] & 0xffffu, w[e][i] >> 16));
        cmax[e] = m;
        mx = max(mx, m);
        mn = min(mn, m != 0u ? m : 0xffffu);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    }
    if (lane == 0) s_range[wave] = (mx << 16) | mn;
    __syncthreads();
    mx = 0u;
    mn = 0xffffu;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        mx = max(mx, s_range[v] >> 16);
        mn = min(mn, s_range[v] & 0xffffu);
    }
    const bool one_pass = mn <= mx && mx - mn < 2048u;
#pragma unroll
    for (int e = 0; e < kChunks; ++e)
        if (cmax[e] != 0u) atomicAdd(&sh.hist[one_pass ? cmax[e] - mn : cmax[e] >> 5], 1);
    __syncthreads();
    if (tid < 64) {
        int above;
        const int bin = wave_find_bin<2048>(sh.hist, p.k, &above);
        if (lane == 0) {
            if (one_pass) s_floor = bin < 0 ? 1u : mn + (uint32_t)bin;
            else s_floor = bin <= 0 ? 1u : ((uint32_t)bin << 5);
            s_need = p.k - above;
        }
    }
    __syncthreads();
    if (!one_pass && s_floor > 1u) {  // uniform; hist_list is still all zero here
        const uint32_t b0 = s_floor >> 5;
#pragma unroll
        for (int e = 0; e < kChunks; ++e)
            if ((cmax[e] >> 5) == b0) atomicAdd(&hist_list[cmax[e] & 31], 1);
        __syncthreads();
        if (tid < 64) {
            int above;
            const int b1 = wave_find_bin<32>(hist_list, s_need, &above);
            if (lane == 0) s_floor |= (uint32_t)b1;
        }
        __syncthreads();
        if (tid < 32) hist_list[tid] = 0;
    }
    const uint32_t floor_top = s_floor;
    // Column order is chunk-major (chunk e of wave w covers columns
    // 8 (THREADS e + 64 w) .. +511): per-lane counts of each chunk (at most
    // 8), three 10-bit fields to a word, scanned across the wave with DPP.
    constexpr int kCntWords = (kChunks + 2) / 3;
    uint32_t packed[kCntWords], incl[kCntWords];
#pragma unroll
    for (int c = 0; c < kCntWords; ++c) packed[c] = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j)
        packed[j / 24] += ((key_at(j) + 0x10000u - floor_top) >> 16) << (10 * ((j / 8) % 3));
#pragma unroll
    for (int c = 0; c < kCntWords; ++c) incl[c] = wave_inclusive_scan(packed[c]);
    if (lane == 63) {
#pragma unroll
        for (int e = 0; e < kChunks; ++e) seg_count[e * kWaves + wave] = (int)((incl[e / 3] >> (10 * (e % 3))) & 1023u);
    }
    __syncthreads();
    int tot = 0, pre = 0;
    if (lane < kChunks) {
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const int sc = seg_count[lane * kWaves + v];
            tot += sc;
            pre += v < wave ? sc : 0;
        }
    }
    const int tot_incl = (int)wave_inclusive_scan((uint32_t)tot);
    const int seg_off = tot_incl - tot + pre;
    const int listed = __builtin_amdgcn_readlane(tot_incl, 63);
    int T16 = -1;
    if (listed <= kListCap) {
        const uint32_t floor_top2 = __builtin_amdgcn_readfirstlane(floor_top);
#pragma unroll
        for (int e = 0; e < kChunks; ++e) {
            int at = __builtin_amdgcn_readlane(seg_off, e) + (int)(((incl[e / 3] - packed[e / 3]) >> (10 * (e % 3))) & 1023u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t t = key_at(8 * e + i);
                const bool in = t >= floor_top2;
                if (in) {
                    list[at] = (t << 16) | (uint32_t)(chunk_col(e) + i);
                    atomicAdd(&hist_list[t >> 5], 1);
                }
                at += in;
            }
        }
        __syncthreads();
        if (listed <= p.k) {
            T16 = 0;  // every listed key is picked
        } else {
            if (tid < 64) {
                const int t = wave_select_keys16<kF16>(list, listed, p.k, hist_list, sh.hist, tied_idx, p, row, start, q_lds);
                if (lane == 0) s_T = t;
            }
            __syncthreads();
            T16 = s_T;
        }
    }
    if (T16 < 0) {  // uniform: the fallback writes this row
        if (tid == 0) p.hard_rows[atomicAdd(p.hard_count, 1)] = (int32_t)row;
        return;
    }
    // Picks: the entries with key16 > T16, in column order, from contiguous
    // slices of the list.
    const int per = (listed + THREADS - 1) / THREADS;
    const int lo = min(tid * per, listed), hi = min(lo + per, listed);
    int gt = 0;
#pragma unroll 1
    for (int i = lo; i < hi; ++i) gt += (int)(list[i] >> 16) > T16;
    int total;
    int before = block_exclusive_scan<THREADS>(gt, sh.wave_tmp, &total);
#pragma unroll 1
    for (int i = lo; i < hi; ++i) {
        const uint32_t e = list[i];
        if ((int)(e >> 16) > T16 && before < p.k) out[before++] = (int32_t)(e & 0xffffu);
    }
    for (int i = total + tid; i < p.k; i += THREADS) out[i] = -1;
}

// Rows the key select left: each workgroup takes hard rows blockIdx.x,
// blockIdx.x + gridDim.x, ..., rescores the whole row into its scratch row
// (-inf outside the row's keys, as the score kernel writes) and selects over
// it.  The rescoring is the prefill's arithmetic (rescore_key), so the scores
// and the picks are those of the score matrix.
template <bool kF16>
__global__ __launch_bounds__(1024) void topk_keys16_fallback_kernel(Keys16TopkParams p) {
    const int count = *p.hard_count;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float *x = p.scratch + (int64_t)blockIdx.x * p.scratch_stride;
    for (int i = blockIdx.x; i < count && p.num_keys > 0; i += gridDim.x) {
        const int64_t row = p.hard_rows[i];
        const int64_t start = p.row_k_start[row];
        const int64_t end = min((int64_t)p.row_k_end[row], p.num_keys);
        for (int c0 = 64 * wave; c0 < p.num_cols; c0 += 64 * 16) {  // wave-uniform
            const int c = c0 + lane;
            const int64_t kidx = start + c;
            const bool vis = c < p.num_cols && kidx >= 0 && kidx < end;
            // Lanes outside the row's keys rescore a key that exists (their
            // result is dropped); a hard row has at least one key.
            const int64_t safe = kidx < 0 ? 0 : (kidx >= p.num_keys ? p.num_keys - 1 : kidx);
            const uint32_t key = rescore_key<kF16>(p, row, safe);
            if (c < p.num_cols) {
                // The score back from its key: scores here are >= +0, +inf or
                // NaN (key 0, stored as NaN so that it is never picked).
                x[c] = !vis ? neg_inf() : (key == 0u ? __uint_as_float(0x7fc00000u) : __uint_as_float(key & 0x7fffffffu));
            }
        }
        __syncthreads();
        streaming_select(x, p.num_cols, p.out + row * p.out_stride, p.k);
        __syncthreads();
    }
}

template <int E, int THREADS, int WPE, bool kFull>
hipError_t launch_resident(const TopkParams &p, hipStream_t stream) {
    // 16-byte loads for rows 16-byte aligned with whole 4-column chunks.
    const int32_t vec_rows = p.vec && (p.num_cols & 3) == 0;
    return launch_kernel(topk_resident_kernel<E, THREADS, WPE, kFull>, dim3((unsigned)p.num_rows), dim3(THREADS),
                         stream, p.logits, p.logits_stride, p.num_cols, vec_rows, p);
}

// Columns per thread, rounded up to a multiple of 4 (16-byte loads), up to
// MAXE; the caller routes longer rows elsewhere.
template <int THREADS, int WPE, int MAXE, bool kFull = false, int E = 4>
hipError_t launch_config(const TopkParams &p, hipStream_t stream) {
    const int per = ((p.num_cols + THREADS - 1) / THREADS + 3) / 4 * 4;
    if (per <= E || E == MAXE) return launch_resident<E, THREADS, WPE, kFull>(p, stream);
    if constexpr (E + 4 <= MAXE) return launch_config<THREADS, WPE, MAXE, kFull, E + 4>(p, stream);
    return hipErrorInvalidValue;  // not reached
}

}  // namespace

hipError_t launch_topk_floor(const FusedTopkParams &p, hipStream_t stream) {
    return launch_kernel(topk_floor_kernel, dim3((unsigned)((p.num_rows + 3) / 4)), dim3(256), stream, p);
}

hipError_t launch_topk_candidates(const FusedTopkParams &p, hipStream_t stream) {
    // Pools of at most 4,096 entries (short rows, where most cells are
    // candidates) always fit the larger LDS list; otherwise the smaller list
    // keeps more rows per CU, and longer lists are read in place.
    if (p.pool_cap <= 4096)
        return launch_kernel(topk_candidates_kernel<4096>, dim3((unsigned)p.num_rows), dim3(256), stream, p);
    return launch_kernel(topk_candidates_kernel<2048>, dim3((unsigned)p.num_rows), dim3(256), stream, p);
}

hipError_t launch_topk(const TopkParams &p, hipStream_t stream, int num_cus) {
    // At most one row per CU: the latency of one row is the whole cost, so
    // 1024-thread rows (registers for four waves per SIMD), up to 64 columns
    // per thread (fewer than 2^16 per row, which the packed counts need);
    // up to 56 per thread the full keys also stay in registers, so the
    // select re-reads nothing.
    // Many rows: 512-thread rows, four per CU (registers for eight waves per
    // SIMD), up to 56 columns per thread; longer rows, 1024-thread rows two
    // per CU.  Rows longer than these shapes hold are streamed.
    const bool few = p.num_rows <= (num_cus > 0 ? num_cus : 256);
    if (few && p.num_cols <= 1024 * 56) return launch_config<1024, 4, 56, true>(p, stream);  // full keys kept
    if (few && p.num_cols < 65536) return launch_config<1024, 4, 64>(p, stream);
    if (p.num_cols > 32768)
        return launch_kernel(topk_streaming_kernel, dim3((unsigned)p.num_rows), dim3(1024), stream, p);
    if (p.num_cols <= 512 * 56) return launch_config<512, 8, 56>(p, stream);
    return launch_config<1024, 8, 32>(p, stream);
}

template <int E>
hipError_t launch_keys16(const Keys16TopkParams &p, hipStream_t stream) {
    if (p.num_cols > 512 * E) {
        if constexpr (E + 8 <= 64) return launch_keys16<E + 8>(p, stream);
        return hipErrorInvalidValue;
    }
    if (p.f16)
        return launch_kernel(topk_keys16_kernel<E, 512, 8, true>, dim3((unsigned)p.num_rows), dim3(512), stream,
                             p.keys, p.keys_stride, p);
    return launch_kernel(topk_keys16_kernel<E, 512, 8, false>, dim3((unsigned)p.num_rows), dim3(512), stream, p.keys,
                         p.keys_stride, p);
}

hipError_t launch_topk_keys16(const Keys16TopkParams &p, hipStream_t stream) {
    if (p.num_cols > kKeys16MaxCols) return hipErrorInvalidValue;
    return launch_keys16<8>(p, stream);
}

hipError_t launch_topk_keys16_fallback(const Keys16TopkParams &p, hipStream_t stream) {
    if (p.f16)
        return launch_kernel(topk_keys16_fallback_kernel<true>, dim3((unsigned)p.scratch_rows), dim3(1024), stream, p);
    return launch_kernel(topk_keys16_fallback_kernel<false>, dim3((unsigned)p.scratch_rows), dim3(1024), stream, p);
}

}  // namespace qsa
