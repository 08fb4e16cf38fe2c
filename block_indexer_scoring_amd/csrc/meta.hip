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

}  // namespace

hipError_t launch_metadata(const MetaParams &p, hipStream_t stream) {
    const int64_t n = p.num_tokens > p.num_reqs ? p.num_tokens : p.num_reqs;
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    return launch_kernel(metadata_kernel, grid, dim3(kThreads), stream, p);
}

}  // namespace qsa
