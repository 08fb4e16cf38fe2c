// Internal launch interface between the C ABI layer (qsa_api.cpp) and the
// HIP kernels.  Everything here has already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <hip/hip_ext.h>

namespace qsa {

// Element formats (the values of QSA_DTYPE_* in qsa.h).
constexpr int kFmtBf16 = 0, kFmtFp16 = 1, kFmtFp8E4m3 = 2;

struct DecodeParams {
    const uint16_t *q;          // bf16 or fp16 bits
    int64_t q_stride_req, q_stride_row, q_stride_head;
    const uint16_t *k;          // [num_pages][page_size][128] elements: 16-bit, or 1-byte e4m3 codes
    int64_t num_pages;
    int32_t page_size;
    const int32_t *page_table;
    int64_t page_table_stride;
    int32_t page_table_cols;
    const int32_t *comp_lens;
    const int32_t *visible;     // may be null
    int32_t num_reqs, dql;
    float scale;
    float *out;
    int64_t out_stride;
    int32_t out_cols;
    int32_t spans;              // ceil(out_cols / decode_span_keys())
    int32_t q_vec;              // Q may be read with 16-byte loads
    int32_t out_vec;            // out rows may be written with 16-byte stores
    int32_t q_f16;              // Q (and 16-bit keys) are fp16, not bf16
    int32_t k_fp8;              // keys are e4m3 codes (scale already holds the cache scale)
};

struct PrefillParams {
    const uint16_t *q;
    int64_t q_stride_row, q_stride_head;
    const uint16_t *k;
    int64_t k_stride, num_keys;
    const int32_t *row_k_start, *row_k_end;
    int32_t num_rows;
    float scale;
    float *out;
    int64_t out_stride;
    int32_t out_cols;
    int32_t col_chunk;          // output columns per workgroup (multiple of 64)
    int32_t row_blocks, col_chunks;
    int32_t out_vec;
    int32_t exact_stores;       // out_vec, and a row block's output spans < 2^31 bytes
    int32_t f16;                // Q and K are fp16, not bf16 (scores launch only)
    int32_t rotate;             // exact_stores, and some row does not start on a 128-byte line
    // Fused top-k passes (qsa_mqa_prefill_topk); unused by the score kernel.
    int32_t topk;
    float *gmax;                // [rows][gmax_stride] maxima of 16-key groups
    int32_t gmax_stride;        // groups per row: 16 * ceil(out_cols / 256)
    const uint32_t *floor_key;  // [rows] per-row floor (score key)
    const int32_t *seg_off;     // [rows][col_chunks + 1] segment offsets in the row's pool
    uint32_t *cand_key;         // [rows][pool_cap] candidate score keys
    int32_t *cand_col;          // [rows][pool_cap] candidate columns
    int32_t *cand_cnt;          // [rows][col_chunks] candidates per segment
    int32_t pool_cap;
};

struct TopkParams {
    const float *logits;
    int64_t logits_stride;
    int32_t num_rows, num_cols, k;
    int32_t *out;
    int64_t out_stride;
    int32_t vec;                // logits rows may be read with 16-byte loads
};

// Fused prefill top-k: floor and final select (see topk.hip).
constexpr int kFusedMaxK = 2048;
constexpr int kFusedMaxSegs = 256;   // column chunks per row
struct FusedTopkParams {
    int32_t num_rows, k;
    const float *gmax;
    int32_t gmax_stride;        // groups per row
    uint32_t *floor_key;        // [rows] the floor as a score key
    int32_t *seg_off;           // [rows][segs + 1] segment offsets in the row's pool
    const uint32_t *cand_key;   // [rows][pool_cap]
    const int32_t *cand_col;    // [rows][pool_cap]
    const int32_t *cand_cnt;    // [rows][segs]
    int32_t segs;               // column chunks
    int32_t groups_per_seg;     // groups per column chunk
    int32_t pool_cap;
    int32_t *out;
    int64_t out_stride;
};

struct MetaParams {
    const int32_t *query_start_loc, *seq_lens, *key_offsets;
    int32_t num_reqs, num_tokens, compress_ratio;
    int32_t *token_to_req;
    int64_t *positions;
    int32_t *visible, *comp_lens, *row_k_start, *row_k_end;
};

struct CacheMetaParams {
    const int32_t *query_start_loc, *seq_lens;
    int32_t num_reqs, num_tokens, compress_ratio;
    const int32_t *block_table;
    int64_t block_table_stride;
    int32_t block_table_cols, storage_block_size;
    const int64_t *common_slot_mapping;  // may be null
    int64_t *slot_mapping;               // [num_tokens] or null
    int32_t *k_work;                     // [max_num_work][2] or null
    int32_t max_num_work;
};
constexpr int kCacheMetaMaxReqs = 8192;  // requests one work-item block scans in LDS

struct GatherParams {
    const uint8_t *k_cache;              // [num_pages][page_size][row_bytes]
    int32_t row_bytes;                   // 256 (2-byte elements) or 128 (e4m3)
    int64_t num_pages;
    int32_t page_size;
    const int32_t *page_table;
    int64_t page_table_stride;
    int32_t page_table_cols;
    const int32_t *key_counts, *key_offsets;
    int32_t num_reqs;
    int32_t max_keys;                    // bound on key_counts (grid size)
    uint8_t *k_out;
    int64_t k_out_stride_bytes, k_out_rows;
    int32_t widen;                       // 0: copy rows; 1 / 2: e4m3 codes -> bf16 / fp16 values
};

struct PrepareQParams {
    const uint16_t *q;                   // bf16 [num_tokens][num_heads][128], token stride q_stride_token
    int64_t q_stride_token;
    int32_t num_tokens, num_heads;
    const int64_t *positions;            // positions[a * pos_stride_axis + t * pos_stride_token]
    int64_t pos_stride_axis, pos_stride_token;
    const void *cos_sin;                 // [cos_sin_rows][64]: 32 cos, 32 sin
    int64_t cos_sin_rows;
    const void *weight;                  // [128]
    float eps;
    int32_t mrope, mrope_h, mrope_w;     // interleaved MRoPE section (h, w) when mrope != 0
    void *out;                           // [num_tokens][num_heads][128] at the element strides below
    int64_t out_stride_token, out_stride_head;
    float out_scale;                     // e4m3 output: bf16 value / out_scale
    int32_t table_f32, weight_f32, out_fp8;
};

// Timing events attached to every launch from the calling thread (both null
// unless the caller armed them through the C ABI).
struct LaunchEvents {
    hipEvent_t start, stop;
};
LaunchEvents launch_events();

// Launches kernel(p) on stream with the calling thread's timing events.
template <typename P>
hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream, P p) {
    const LaunchEvents ev = launch_events();
    void *args[] = {&p};
    return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, stream,
                              ev.start, ev.stop, 0);
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);
int decode_span_keys();
int prefill_col_chunk(int64_t num_rows, int32_t out_cols, int64_t k_stride, int num_cus);
int64_t prefill_max_k_stride();  // larger key strides overflow the kernel's 32-bit key offsets
int prefill_rows_per_block();
hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_group_max(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_candidates(const PrefillParams &p, hipStream_t stream);
hipError_t launch_topk(const TopkParams &p, hipStream_t stream, int num_cus);
hipError_t launch_topk_floor(const FusedTopkParams &p, hipStream_t stream);
hipError_t launch_topk_candidates(const FusedTopkParams &p, hipStream_t stream);
hipError_t launch_metadata(const MetaParams &p, hipStream_t stream);
hipError_t launch_cache_slots(const CacheMetaParams &p, hipStream_t stream);  // p.slot_mapping set
hipError_t launch_k_work(const CacheMetaParams &p, hipStream_t stream);       // p.k_work set
hipError_t launch_gather_keys(const GatherParams &p, hipStream_t stream);
hipError_t launch_prepare_q(const PrepareQParams &p, hipStream_t stream);

}  // namespace qsa
