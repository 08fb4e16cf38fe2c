// Paged compressed keys gathered into contiguous rows, so that a prefill
// chunk can be scored straight from the compressed-key cache (the cache
// layout [pages, page_size, 1, dim] and page table with -1 entries of MATE
// "QSA (Qwen Sparse Attention)", section "MQA score"; the per-request key
// offsets of the packed prefill form).  Row key_offsets[r] + c of the output
// receives request r's compressed key c (c < key_counts[r]): row c %
// page_size of page page_table[r][c / page_size].  A missing page (negative
// or out-of-range id, or a slot past the table) gives a zero row;
// destinations outside [0, k_out_rows) are skipped.
//
// The copy is HBM-bound: one wavefront moves 64 key rows.  A key row
// (256 bytes of 2-byte elements, or 128 bytes of e4m3 codes) is spread over
// 16 (or 8) lanes, 16 bytes each, so every load and store instruction moves
// whole rows; all of a wave's loads are issued before its first store.  When
// the page size is a multiple of 64, a wave's 64 keys lie on one page, read
// once as a uniform (scalar) load instead of once per lane: that removes a
// dependent per-lane load from every key's path (32 -> 24 us on 105 MB).
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerWave = 64;

template <int ROW_BYTES, bool kOnePage>
__global__ __launch_bounds__(kWaves * 64) void gather_keys_kernel(GatherParams p) {
    constexpr int kLanesPerRow = ROW_BYTES / 16;
    constexpr int kRowsPerOp = 64 / kLanesPerRow;
    constexpr int kOps = kKeysPerWave / kRowsPerOp;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunks = ((int64_t)p.max_keys + kKeysPerWave * kWaves - 1) / (kKeysPerWave * kWaves);
    const int r = (int)(blockIdx.x / chunks);
    const int c0 = (int)(blockIdx.x % chunks) * kKeysPerWave * kWaves + wave * kKeysPerWave;
    int count = p.key_counts[r];
    count = count < 0 ? 0 : (count > p.max_keys ? p.max_keys : count);
    if (c0 >= count) return;
    const int64_t offset = p.key_offsets[r];
    const int part = lane % kLanesPerRow;  // 16-byte part of the row

    // kOnePage: the page of keys c0 .. c0+63 (page_size % 64 == 0).
    int span_page = -1;
    if (kOnePage) {
        const int slot = c0 / p.page_size;
        span_page = slot < p.page_table_cols ? load_uniform(p.page_table + (int64_t)r * p.page_table_stride + slot) : -1;
    }
    u32x4 v[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        const int c = c0 + i * kRowsPerOp + lane / kLanesPerRow;
        v[i] = zero_u32x4();
        if (c < count) {
            int page = span_page;
            if (!kOnePage) {
                const int slot = c / p.page_size;
                page = slot < p.page_table_cols ? p.page_table[(int64_t)r * p.page_table_stride + slot] : -1;
            }
            if (page >= 0 && page < p.num_pages)
                v[i] = load_u32x4(p.k_cache + ((int64_t)page * p.page_size + c % p.page_size) * ROW_BYTES + 16 * part);
        }
    }
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        const int c = c0 + i * kRowsPerOp + lane / kLanesPerRow;
        const int64_t row = offset + c;
        if (c < count && row >= 0 && row < p.k_out_rows)
            *reinterpret_cast<u32x4 *>(p.k_out + row * p.k_out_stride_bytes + 16 * part) = v[i];
    }
}

}  // namespace

hipError_t launch_gather_keys(const GatherParams &p, hipStream_t stream) {
    const int64_t chunks = ((int64_t)p.max_keys + kKeysPerWave * kWaves - 1) / (kKeysPerWave * kWaves);
    const dim3 grid((unsigned)(chunks * p.num_reqs));
    const bool one_page = p.page_size % kKeysPerWave == 0;
    if (p.row_bytes == 128) {
        if (one_page) return launch_kernel(gather_keys_kernel<128, true>, grid, dim3(kWaves * 64), stream, p);
        return launch_kernel(gather_keys_kernel<128, false>, grid, dim3(kWaves * 64), stream, p);
    }
    if (one_page) return launch_kernel(gather_keys_kernel<256, true>, grid, dim3(kWaves * 64), stream, p);
    return launch_kernel(gather_keys_kernel<256, false>, grid, dim3(kWaves * 64), stream, p);
}

}  // namespace qsa
