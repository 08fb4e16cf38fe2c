// Per-token QSA metadata on gfx950 (vLLM page qsa_cache.py,
// _logical_positions and _build_qsa_metadata_kernel; PR 54513 "Main
// changes"): the request of each query token, its logical position
// seq_len - query_len + (t - query_start), and the number of complete
// 4-token blocks it may see, max(0, min((pos+1)/cr, seq_len/cr)).
// One thread per token; the request is found by binary search over
// query_start_loc.  Threads below num_reqs also write comp_lens.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

__global__ __launch_bounds__(kThreads) void metadata_kernel(MetaParams p) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p.comp_lens && t < p.num_reqs)
        p.comp_lens[t] = (int32_t)floor_div(p.seq_lens[t], p.compress_ratio);
    if (t >= p.num_tokens) return;

    int req = -1;
    if (p.num_reqs > 0 && t >= p.query_start_loc[0] && t < p.query_start_loc[p.num_reqs]) {
        // Last request whose start is <= t.
        int lo = 0, hi = p.num_reqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.query_start_loc[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        req = lo;
    }
    int64_t pos = -1;
    int32_t vis = 0;
    if (req >= 0) {
        const int64_t qs = p.query_start_loc[req];
        const int64_t qlen = (int64_t)p.query_start_loc[req + 1] - qs;
        const int64_t seq = p.seq_lens[req];
        pos = seq - qlen + (t - qs);
        int64_t v = floor_div(pos + 1, p.compress_ratio);
        const int64_t by_len = floor_div(seq, p.compress_ratio);
        v = v < by_len ? v : by_len;
        vis = (int32_t)(v < 0 ? 0 : v);
    }
    if (p.token_to_req) p.token_to_req[t] = req < 0 ? 0 : req;
    if (p.positions) p.positions[t] = pos;
    if (p.visible) p.visible[t] = vis;
    if (p.key_offsets) {
        // Padding tokens take request 0's offset and an empty interval.
        const int32_t start = p.num_reqs > 0 ? p.key_offsets[req < 0 ? 0 : req] : 0;
        p.row_k_start[t] = start;
        p.row_k_end[t] = start + vis;
    }
}

// Last request whose query start is <= t, or -1 for a padding token.
__device__ __forceinline__ int token_request(const int32_t *qsl, int num_reqs, int64_t t) {
    if (num_reqs <= 0 || t < qsl[0] || t >= qsl[num_reqs]) return -1;
    int lo = 0, hi = num_reqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Compressed-cache slot of each token (vLLM qsa_cache.py,
// compressed_qsa_slot_mapping and the compress_ratio != 1 slot branch of
// _build_qsa_metadata_kernel): a token at logical position pos writes the
// compressed key of its group when pos >= 0 and (pos+1) % cr == 0; that key's
// compressed position cp = pos / cr sits in logical block cp / block_size of
// the request's block-table row, at row cp % block_size.  -1 when no group
// closes, the logical block is past the table, its entry is negative, the
// token's main-cache slot is negative, or the token is padding.
__global__ __launch_bounds__(kThreads) void cache_slots_kernel(CacheMetaParams p) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= p.num_tokens) return;
    int64_t slot = -1;
    const int req = token_request(p.query_start_loc, p.num_reqs, t);
    if (req >= 0) {
        const int64_t qs = p.query_start_loc[req];
        const int64_t pos = (int64_t)p.seq_lens[req] - ((int64_t)p.query_start_loc[req + 1] - qs) + (t - qs);
        if (pos >= 0 && (pos + 1) % p.compress_ratio == 0) {
            const int64_t cp = pos / p.compress_ratio;
            const int64_t logical_block = cp / p.storage_block_size;
            if (logical_block < p.block_table_cols) {
                const int64_t block = p.block_table[(int64_t)req * p.block_table_stride + logical_block];
                const bool main_ok = !p.common_slot_mapping || p.common_slot_mapping[t] >= 0;
                if (block >= 0 && main_ok) slot = block * p.storage_block_size + cp % p.storage_block_size;
            }
        }
    }
    p.slot_mapping[t] = slot;
}

// Raw-key ring slot of each token (vLLM qsa_cache.py, the circular branch
// of _build_qsa_metadata_kernel; circular_qsa_slot_mapping): request r owns
// one ring of ring_size rows in block block_table[r][0], block 0 being the
// null block that is never written; a query token at logical position
// pos >= 0 among the last ring_size query tokens of its request writes row
// pos % ring_size.  -1 otherwise and for padding tokens.
__global__ __launch_bounds__(kThreads) void ring_slots_kernel(RingSlotParams p) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= p.num_tokens) return;
    int64_t slot = -1;
    const int req = token_request(p.query_start_loc, p.num_reqs, t);
    if (req >= 0 && p.block_table_cols > 0) {
        const int64_t qs = p.query_start_loc[req];
        const int64_t qe = p.query_start_loc[req + 1];
        const int64_t pos = (int64_t)p.seq_lens[req] - (qe - qs) + (t - qs);
        if (pos >= 0 && t + p.ring_size >= qe) {
            const int64_t block = p.block_table[(int64_t)req * p.block_table_stride];
            if (block > 0) slot = block * p.ring_size + pos % p.ring_size;
        }
    }
    p.slot_mapping[t] = slot;
}

// Work items of the compressed-cache writer (_build_qsa_metadata_kernel,
// k_work_metadata): a request with query tokens owns max(groups, 1) items,
// groups = seq_len/cr - (seq_len - query_len)/cr (floor division), numbered
// request by request; item w is (request, w - request's first item), and
// items past the last are (-1, -1).  Every block recomputes the per-request
// item offsets in LDS (a block-wide exclusive scan), so blocks need no
// grid-wide ordering, then binary-searches the owner of each of its items.
__global__ __launch_bounds__(kThreads) void k_work_kernel(CacheMetaParams p) {
    __shared__ int32_t first_item[kCacheMetaMaxReqs + 1];
    __shared__ int32_t wave_sum[kThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Thread tid sums the items of requests [tid*per, (tid+1)*per).
    const int per = (p.num_reqs + kThreads - 1) / kThreads;
    const int r0 = tid * per;
    int mine = 0;
    for (int r = r0; r < r0 + per && r < p.num_reqs; ++r) {
        const int64_t qlen = (int64_t)p.query_start_loc[r + 1] - p.query_start_loc[r];
        int count = 0;
        if (qlen > 0) {
            const int64_t groups = floor_div(p.seq_lens[r], p.compress_ratio) -
                                   floor_div((int64_t)p.seq_lens[r] - qlen, p.compress_ratio);
            count = groups > 1 ? (int)groups : 1;
        }
        first_item[r] = count;  // the count for now; turned into offsets below
        mine += count;
    }
    // Exclusive scan of the per-thread sums: within the wave, then across waves.
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_sum[w];
    int run = before + incl - mine;
    for (int r = r0; r < r0 + per && r < p.num_reqs; ++r) {
        const int count = first_item[r];
        first_item[r] = run;
        run += count;
    }
    if (tid == kThreads - 1) first_item[p.num_reqs] = run;  // total items
    __syncthreads();
    const int total = first_item[p.num_reqs];
    const int64_t w = (int64_t)blockIdx.x * kThreads + tid;
    if (w >= p.max_num_work) return;
    int req = -1, index = -1;
    if (w < total) {
        // Last request whose first item is <= w (requests with no items share
        // the next one's offset, so the last such request owns item w).
        int lo = 0, hi = p.num_reqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_item[mid] <= w) lo = mid;
            else hi = mid - 1;
        }
        req = lo;
        index = (int)(w - first_item[lo]);
    }
    p.k_work[2 * w] = req;
    p.k_work[2 * w + 1] = index;
}

// Compressed lengths and visible blocks of a uniform decode batch: thread
// per row r*dql + j at position seq_len - dql + j (the last dql tokens of
// the context), 4 tokens per compressed block.
__global__ __launch_bounds__(kThreads) void decode_visible_kernel(DecodeVisibleParams p) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p.comp_lens && i < p.num_reqs) p.comp_lens[i] = (int32_t)floor_div(p.seq_lens[i], 4);
    if (!p.visible || i >= (int64_t)p.num_reqs * p.dql) return;
    const int r = (int)(i / p.dql), j = (int)(i % p.dql);
    const int64_t seq = p.seq_lens[r];
    const int64_t pos = seq - p.dql + j;
    int64_t v = floor_div(pos + 1, 4);
    const int64_t by_len = floor_div(seq, 4);
    v = v < by_len ? v : by_len;
    p.visible[i] = (int32_t)(v < 0 ? 0 : v);
}

}  // namespace

hipError_t launch_cache_slots(const CacheMetaParams &p, hipStream_t stream) {
    return launch_kernel(cache_slots_kernel, dim3((unsigned)((p.num_tokens + kThreads - 1) / kThreads)),
                         dim3(kThreads), stream, p);
}

hipError_t launch_ring_slots(const RingSlotParams &p, hipStream_t stream) {
    return launch_kernel(ring_slots_kernel, dim3((unsigned)((p.num_tokens + kThreads - 1) / kThreads)),
                         dim3(kThreads), stream, p);
}

hipError_t launch_k_work(const CacheMetaParams &p, hipStream_t stream) {
    return launch_kernel(k_work_kernel, dim3((unsigned)((p.max_num_work + kThreads - 1) / kThreads)),
                         dim3(kThreads), stream, p);
}

hipError_t launch_decode_visible(const DecodeVisibleParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.num_reqs * p.dql;
    const int64_t n = rows > p.num_reqs ? rows : p.num_reqs;
    return launch_kernel(decode_visible_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads),
                         stream, p);
}

hipError_t launch_metadata(const MetaParams &p, hipStream_t stream) {
    const int64_t n = p.num_tokens > p.num_reqs ? p.num_tokens : p.num_reqs;
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    return launch_kernel(metadata_kernel, grid, dim3(kThreads), stream, p);
}

}  // namespace qsa
