// Paged compressed keys gathered into contiguous rows, so that a prefill
// chunk can be scored straight from the compressed-key cache (the cache
// layout [pages, page_size, 1, dim] and page table with -1 entries of MATE
// "QSA (Qwen Sparse Attention)", section "MQA score"; the per-request key
// offsets of the packed prefill form).  Row key_offsets[r] + c of the output
// receives request r's compressed key c (c < key_counts[r]): row c %
// page_size of page page_table[r][c / page_size].  A missing page (negative
// or out-of-range id, or a slot past the table) gives a zero row;
// destinations outside [0, k_out_rows) are skipped.  Rows are copied as
// they are, or e4m3 codes are widened exactly to bf16 or fp16 values on the
// way (the same conversion as the e4m3 decode path): with the cache scale
// folded into the score multiplier, the 16-bit prefill then scores an e4m3
// cache exactly as the e4m3 decode does.
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

// IN_ROW / OUT_ROW: bytes per key row read / written; WIDEN: 0 copy, 1 e4m3
// -> bf16, 2 e4m3 -> fp16 (OUT_ROW = 2 * IN_ROW).
template <int IN_ROW, int OUT_ROW, int WIDEN, bool kOnePage>
__global__ __launch_bounds__(kWaves * 64) void gather_keys_kernel(GatherParams p) {
    static_assert(WIDEN == 0 ? IN_ROW == OUT_ROW : 2 * IN_ROW == OUT_ROW, "row sizes");
    constexpr int kLanesPerRow = OUT_ROW / 16;
    constexpr int kInBytes = IN_ROW / kLanesPerRow;  // bytes each lane reads per row: 16, or 8 when widening
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
            if (page >= 0 && page < p.num_pages) {
                const uint8_t *src = p.k_cache + ((int64_t)page * p.page_size + c % p.page_size) * IN_ROW + kInBytes * part;
                if constexpr (WIDEN == 0) {
                    v[i] = load_u32x4(src);
                } else {
                    const uint2 w = *reinterpret_cast<const uint2 *>(src);
                    v[i][0] = w.x;
                    v[i][1] = w.y;
                }
            }
        }
    }
    if constexpr (WIDEN != 0) {
        // Code 0 (and the zero row of a missing page) widens to +0.
#pragma unroll
        for (int i = 0; i < kOps; ++i) v[i] = e4m3x8_to_16bit<WIDEN == 2>(v[i][0], v[i][1]);
    }
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        const int c = c0 + i * kRowsPerOp + lane / kLanesPerRow;
        const int64_t row = offset + c;
        if (c < count && row >= 0 && row < p.k_out_rows)
            *reinterpret_cast<u32x4 *>(p.k_out + row * p.k_out_stride_bytes + 16 * part) = v[i];
    }
}

// Key rows written to cache rows: the compressed-key cache
// (QSACompressedKeyCache: one normed key per complete group, bf16 or e4m3)
// and the raw-key ring (QSAKeyStateCache: raw bf16 keys, optionally followed
// by the three int64 MRoPE positions), at the slots of the cache metadata.
// Row t of the keys goes to cache row slots[t] when 0 <= slots[t] <
// num_slots.  An e4m3 cache takes each bf16 value divided by the scale in
// fp32, rounded to the nearest e4m3 value with ties to even and saturated
// at 448 (qsa_prepare's _to_dst_dtype; the keys are bf16 already).  Half a
// wavefront moves one row: 32 lanes of 4 elements (8 bytes in; 8 bytes out,
// or 4 e4m3 bytes), lanes 0..2 also the positions.
constexpr int kWriteThreads = 256;

template <bool kFp8, bool kPositions>
__global__ __launch_bounds__(kWriteThreads) void write_keys_kernel(WriteKeysParams p) {
    const int64_t t = ((int64_t)blockIdx.x * kWriteThreads + threadIdx.x) / 32;
    const int l = threadIdx.x & 31;
    if (t >= p.num_tokens) return;
    const int64_t s = p.slots[t];
    if (s < 0 || s >= p.num_slots) return;
    const uint2 v = *reinterpret_cast<const uint2 *>(p.keys + t * p.key_stride + 4 * l);
    if constexpr (kFp8) {
        const float f[4] = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                            __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= e4m3_rne_sat(f[i] / p.scale) << (8 * i);
        *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.cache) + s * p.row_stride + 4 * l) = w;
    } else {
        uint16_t *row = static_cast<uint16_t *>(p.cache) + s * p.row_stride;
        *reinterpret_cast<uint2 *>(row + 4 * l) = v;
        if (kPositions && l < 3)
            *reinterpret_cast<int64_t *>(row + kDim + 4 * l) = p.positions[l * p.pos_stride_axis + t * p.pos_stride_token];
    }
}

}  // namespace

hipError_t launch_gather_keys(const GatherParams &p, hipStream_t stream) {
    const int64_t chunks = ((int64_t)p.max_keys + kKeysPerWave * kWaves - 1) / (kKeysPerWave * kWaves);
    const dim3 grid((unsigned)(chunks * p.num_reqs));
    const dim3 block(kWaves * 64);
    const bool one_page = p.page_size % kKeysPerWave == 0;
    if (p.widen == 1) {
        if (one_page) return launch_kernel(gather_keys_kernel<128, 256, 1, true>, grid, block, stream, p);
        return launch_kernel(gather_keys_kernel<128, 256, 1, false>, grid, block, stream, p);
    }
    if (p.widen == 2) {
        if (one_page) return launch_kernel(gather_keys_kernel<128, 256, 2, true>, grid, block, stream, p);
        return launch_kernel(gather_keys_kernel<128, 256, 2, false>, grid, block, stream, p);
    }
    if (p.row_bytes == 128) {
        if (one_page) return launch_kernel(gather_keys_kernel<128, 128, 0, true>, grid, block, stream, p);
        return launch_kernel(gather_keys_kernel<128, 128, 0, false>, grid, block, stream, p);
    }
    if (one_page) return launch_kernel(gather_keys_kernel<256, 256, 0, true>, grid, block, stream, p);
    return launch_kernel(gather_keys_kernel<256, 256, 0, false>, grid, block, stream, p);
}

hipError_t launch_write_keys(const WriteKeysParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(((int64_t)p.num_tokens * 32 + kWriteThreads - 1) / kWriteThreads));
    const dim3 block(kWriteThreads);
    if (p.fp8) return launch_kernel(write_keys_kernel<true, false>, grid, block, stream, p);
    if (p.positions) return launch_kernel(write_keys_kernel<false, true>, grid, block, stream, p);
    return launch_kernel(write_keys_kernel<false, false>, grid, block, stream, p);
}

}  // namespace qsa
