// C ABI of the QSA MQA indexer: argument checks (host arguments only, never
// device contents), error text, and dispatch to the gfx950 kernels.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "qsa.h"
#include "qsa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local qsa::LaunchEvents g_launch_events{nullptr, nullptr};

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return QSA_OK;
}

int device_status(const char *what, hipError_t err) {
    if (err != hipSuccess)
        return fail(QSA_ERR_DEVICE, "%s: kernel launch failed: %s", what, hipGetErrorString(err));
    return ok();
}

// Compute units of the current device (cached per device; 0 if unknown).
int current_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Fused prefill top-k workspace: per row the maxima of 8-key groups, the
// floor key, the offsets of the column chunks' segments in the row's
// candidate pool, a candidate count per chunk, and the pool (8-byte entries:
// the score's bits, column).  The pool holds every key above the floor (at most 8 (k - 1))
// and at most k keys equal to it per chunk, and no chunk more than its
// columns, so it never overflows; the floor kernel sizes each segment from
// the group maxima.
constexpr int64_t kFusedMaxKStride = (int64_t)1 << 14;
struct FusedLayout {
    int chunk;
    int64_t col_chunks, groups, pool_cap;
    int64_t off_gmax, off_floor, off_segoff, off_cnt, off_cand, total;
};
FusedLayout fused_layout(int32_t num_rows, int32_t out_cols, int32_t topk, int num_cus) {
    FusedLayout L{};
    // Column chunks on 256-column group boundaries, as few as still give one
    // workgroup per CU (row blocks x chunks), so both passes run in one round
    // of workgroups.  The layout depends on the sizes and the CU count only,
    // so the same layout serves every call.
    const int64_t row_blocks = ((int64_t)num_rows + qsa::prefill_rows_per_block() - 1) / qsa::prefill_rows_per_block();
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    const int64_t want = row_blocks > 0 && row_blocks < cus ? cus / row_blocks : 1;
    // At most 32,512 columns, so a chunk's key offsets stay 32-bit at the
    // largest key stride accepted.
    const int64_t max_chunk = (((int64_t)1 << 30) / (64 * kFusedMaxKStride * 2) - 1) * 64 / 256 * 256;
    const int64_t chunk = ((((int64_t)out_cols + want - 1) / want) + 255) / 256 * 256;
    L.chunk = (int)(chunk < 256 ? 256 : (chunk > max_chunk ? max_chunk : chunk));
    L.col_chunks = out_cols > 0 ? ((int64_t)out_cols + L.chunk - 1) / L.chunk : 0;
    if (L.col_chunks > qsa::kFusedMaxSegs) {  // wide rows: fewer, wider chunks
        L.chunk = (int)((((int64_t)out_cols + qsa::kFusedMaxSegs - 1) / qsa::kFusedMaxSegs + 255) / 256 * 256);
        L.col_chunks = ((int64_t)out_cols + L.chunk - 1) / L.chunk;
    }
    constexpr int64_t kGroupRowCols = 64 * qsa::kFusedGroupTiles;  // columns of 16 groups
    L.groups = 16 * (((int64_t)out_cols + kGroupRowCols - 1) / kGroupRowCols);
    // Each segment's room is also capped by its chunk's columns, so a row
    // never needs more than its columns.
    L.pool_cap = qsa::kFusedGroupKeys * (int64_t)(topk - 1) + L.col_chunks * topk;
    if (L.pool_cap > out_cols) L.pool_cap = out_cols;
    auto seg = [](int64_t b) { return (b + 255) / 256 * 256; };
    int64_t o = 0;
    L.off_gmax = o; o += seg((int64_t)num_rows * L.groups * 4);
    L.off_floor = o; o += seg((int64_t)num_rows * 4);
    L.off_segoff = o; o += seg((int64_t)num_rows * (L.col_chunks + 1) * 4);
    L.off_cnt = o; o += seg((int64_t)num_rows * L.col_chunks * 4);
    L.off_cand = o; o += seg((int64_t)num_rows * L.pool_cap * 8);
    L.total = o;
    return L;
}

// Workspace of the score-key path (rows of 1 .. kKeys16MaxCols columns):
// the cells' 16-bit key prefixes on rows padded to 64 columns, the count and
// list of rows left to the fallback, and one fp32 scratch row per fallback
// workgroup.
struct Keys16Layout {
    int64_t stride, off_keys, off_count, off_hard, off_scratch, total;
};
Keys16Layout keys16_layout(int32_t num_rows, int32_t out_cols) {
    Keys16Layout L{};
    auto seg = [](int64_t b) { return (b + 255) / 256 * 256; };
    L.stride = ((int64_t)out_cols + 63) / 64 * 64;
    int64_t o = 0;
    L.off_keys = o; o += seg((int64_t)num_rows * L.stride * 2);
    L.off_count = o; o += 256;
    L.off_hard = o; o += seg((int64_t)num_rows * 4);
    L.off_scratch = o; o += seg((int64_t)qsa::kKeys16FallbackGroups * L.stride * 4);
    L.total = o;
    return L;
}
bool use_keys16(int32_t out_cols) { return out_cols > 0 && out_cols <= qsa::kKeys16MaxCols; }

// Vector-load layout rule: 16-byte aligned base, and every axis with more
// than one element has a positive stride that is a multiple of 8 bf16.
bool axis_ok(int64_t size, int64_t stride) { return size <= 1 || (stride > 0 && stride % 8 == 0); }

int check_heads(const char *fn, int32_t num_heads, int32_t head_dim) {
    if (num_heads != 4 || head_dim != 128)
        return fail(QSA_ERR_UNSUPPORTED, "%s: only (num_heads, head_dim) = (4, 128) is supported, got (%d, %d)",
                    fn, num_heads, head_dim);
    return QSA_OK;
}

int check_scale(const char *fn, float scale) {
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: scale must be finite and > 0, got %g", fn, (double)scale);
    return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char *qsa_last_error(void) { return g_last_error.c_str(); }

int qsa_set_launch_events(void *start_event, void *stop_event) {
    g_launch_events = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
    return QSA_OK;
}

int qsa_split_batch(const int32_t *query_start_loc, int32_t num_reqs, int32_t decode_threshold,
                    int32_t *order, int32_t *counts) {
    const char *fn = "qsa_split_batch";
    if (!query_start_loc || !counts) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL query_start_loc or counts", fn);
    if (num_reqs < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: num_reqs < 0", fn);
    if (decode_threshold < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: decode_threshold < 1", fn);
    for (int32_t r = 0; r < num_reqs; ++r)
        if (query_start_loc[r + 1] < query_start_loc[r])
            return fail(QSA_ERR_INVALID_ARGUMENT, "%s: query_start_loc decreases at request %d", fn, r);
    // DQL: length of the first request whose length is in [1, threshold].
    int32_t dql = 0;
    for (int32_t r = 0; r < num_reqs && dql == 0; ++r) {
        const int32_t len = query_start_loc[r + 1] - query_start_loc[r];
        if (len >= 1 && len <= decode_threshold) dql = len;
    }
    auto is_decode = [&](int32_t r) {
        return dql > 0 && query_start_loc[r + 1] - query_start_loc[r] == dql;
    };
    int64_t num_decodes = 0, decode_tokens = 0, prefill_tokens = 0;
    if (order) {
        int32_t at = 0;
        for (int32_t r = 0; r < num_reqs; ++r)
            if (is_decode(r)) order[at++] = r;
        num_decodes = at;
        for (int32_t r = 0; r < num_reqs; ++r)
            if (!is_decode(r)) order[at++] = r;
    } else {
        while (num_decodes < num_reqs && is_decode((int32_t)num_decodes)) ++num_decodes;
    }
    const int64_t total = num_reqs > 0 ? (int64_t)query_start_loc[num_reqs] - query_start_loc[0] : 0;
    decode_tokens = num_decodes * dql;
    prefill_tokens = total - decode_tokens;
    counts[0] = (int32_t)num_decodes;
    counts[1] = (int32_t)decode_tokens;
    counts[2] = num_reqs - (int32_t)num_decodes;
    counts[3] = (int32_t)prefill_tokens;
    counts[4] = num_decodes > 0 ? dql : 0;
    return ok();
}

int qsa_build_metadata(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                       int32_t num_tokens, int32_t compress_ratio, const int32_t *key_offsets,
                       int32_t *token_to_req, int64_t *positions, int32_t *visible,
                       int32_t *comp_lens, int32_t *row_k_start, int32_t *row_k_end, void *stream) {
    const char *fn = "qsa_build_metadata";
    if (num_reqs < 0 || num_tokens < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (compress_ratio < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: compress_ratio < 1", fn);
    if (!query_start_loc) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL query_start_loc", fn);
    if (num_reqs > 0 && !seq_lens) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL seq_lens", fn);
    if (key_offsets && (!row_k_start || !row_k_end))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: key_offsets needs row_k_start and row_k_end", fn);
    if (!key_offsets && (row_k_start || row_k_end))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: row_k_start/row_k_end need key_offsets", fn);
    if (num_tokens == 0 && (num_reqs == 0 || !comp_lens)) return ok();
    qsa::MetaParams p{query_start_loc, seq_lens, key_offsets, num_reqs, num_tokens, compress_ratio,
                      token_to_req, positions, visible, comp_lens, row_k_start, row_k_end};
    return device_status(fn, qsa::launch_metadata(p, static_cast<hipStream_t>(stream)));
}

int qsa_decode_visible_blocks(const int32_t *seq_lens, int32_t num_reqs, int32_t dql, int32_t *comp_lens_out,
                              int32_t *visible_out, void *stream) {
    const char *fn = "qsa_decode_visible_blocks";
    if (num_reqs < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: num_reqs < 0", fn);
    if (dql < 1 || dql > 16) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: dql must be in [1, 16], got %d", fn, dql);
    if (num_reqs == 0 || (!comp_lens_out && !visible_out)) return ok();
    if (!seq_lens) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL seq_lens", fn);
    if ((int64_t)num_reqs * dql >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    qsa::DecodeVisibleParams p{seq_lens, num_reqs, dql, comp_lens_out, visible_out};
    return device_status(fn, qsa::launch_decode_visible(p, static_cast<hipStream_t>(stream)));
}

int qsa_build_cache_metadata(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                             int32_t num_tokens, int32_t compress_ratio, const int32_t *block_table,
                             int64_t block_table_stride, int32_t block_table_cols, int32_t storage_block_size,
                             const int64_t *common_slot_mapping, int64_t *slot_mapping, int32_t *k_work,
                             int32_t max_num_work, void *stream) {
    const char *fn = "qsa_build_cache_metadata";
    if (num_reqs < 0 || num_tokens < 0 || max_num_work < 0 || block_table_cols < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (compress_ratio < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: compress_ratio < 1", fn);
    if (storage_block_size < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: storage_block_size < 1", fn);
    if (num_reqs > 1 && block_table_cols > 0 && block_table_stride < block_table_cols)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: block_table_stride < block_table_cols", fn);
    const bool slots = slot_mapping && num_tokens > 0;
    const bool work = k_work && max_num_work > 0;
    if (!slots && !work) return ok();
    if (!query_start_loc) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL query_start_loc", fn);
    if (num_reqs > 0 && !seq_lens) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL seq_lens", fn);
    if (slots && num_reqs > 0 && block_table_cols > 0 && !block_table)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL block_table", fn);
    if (work && num_reqs > qsa::kCacheMetaMaxReqs)
        return fail(QSA_ERR_UNSUPPORTED, "%s: work items for more than %d requests", fn, qsa::kCacheMetaMaxReqs);
    qsa::CacheMetaParams p{};
    p.query_start_loc = query_start_loc;
    p.seq_lens = seq_lens;
    p.num_reqs = num_reqs;
    p.num_tokens = num_tokens;
    p.compress_ratio = compress_ratio;
    p.block_table = block_table;
    p.block_table_stride = block_table_stride;
    p.block_table_cols = block_table ? block_table_cols : 0;
    p.storage_block_size = storage_block_size;
    p.common_slot_mapping = common_slot_mapping;
    p.slot_mapping = slots ? slot_mapping : nullptr;
    p.k_work = work ? k_work : nullptr;
    p.max_num_work = max_num_work;
    // Up to two launches; armed timing events span them (start on the first,
    // stop on the last).
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const qsa::LaunchEvents ev = g_launch_events;
    hipError_t err = hipSuccess;
    if (slots) {
        g_launch_events = {ev.start, work ? nullptr : ev.stop};
        err = qsa::launch_cache_slots(p, st);
    }
    if (work && err == hipSuccess) {
        g_launch_events = {slots ? nullptr : ev.start, ev.stop};
        err = qsa::launch_k_work(p, st);
    }
    g_launch_events = ev;
    return device_status(fn, err);
}

int qsa_build_ring_slots(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                         int32_t num_tokens, const int32_t *block_table, int64_t block_table_stride,
                         int32_t block_table_cols, int32_t ring_size, int64_t *slot_mapping, void *stream) {
    const char *fn = "qsa_build_ring_slots";
    if (num_reqs < 0 || num_tokens < 0 || block_table_cols < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (ring_size < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: ring_size < 1", fn);
    if (num_reqs > 1 && block_table_cols > 0 && block_table_stride < block_table_cols)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: block_table_stride < block_table_cols", fn);
    if (num_tokens == 0) return ok();
    if (!query_start_loc || !slot_mapping) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL query_start_loc or slot_mapping", fn);
    if (num_reqs > 0 && !seq_lens) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL seq_lens", fn);
    if (num_reqs > 0 && block_table_cols > 0 && !block_table)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL block_table", fn);
    qsa::RingSlotParams p{query_start_loc, seq_lens, num_reqs, num_tokens, block_table, block_table_stride,
                          block_table ? block_table_cols : 0, ring_size, slot_mapping};
    return device_status(fn, qsa::launch_ring_slots(p, static_cast<hipStream_t>(stream)));
}

int qsa_write_keys(const void *keys, int64_t key_stride, int32_t num_tokens, const int64_t *slots, void *cache,
                   int32_t cache_dtype, int64_t row_stride, int64_t num_slots, float scale, const int64_t *positions,
                   int64_t pos_stride_axis, int64_t pos_stride_token, void *stream) {
    const char *fn = "qsa_write_keys";
    if (cache_dtype != QSA_DTYPE_BF16 && cache_dtype != QSA_DTYPE_FP8_E4M3)
        return fail(QSA_ERR_UNSUPPORTED, "%s: cache format %d is not bf16 or e4m3", fn, cache_dtype);
    const bool fp8 = cache_dtype == QSA_DTYPE_FP8_E4M3;
    if (num_tokens < 0 || num_slots < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (fp8 && !(std::isfinite(scale) && scale > 0.0f))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: scale must be finite and > 0 for an e4m3 cache", fn);
    if (positions && fp8) return fail(QSA_ERR_UNSUPPORTED, "%s: positions go with a bf16 cache only", fn);
    const int64_t min_row = positions ? 128 + 12 : 128;
    if (row_stride < min_row)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: row_stride %lld below the %lld elements a row needs", fn,
                    (long long)row_stride, (long long)min_row);
    if (num_tokens > 1 && key_stride < 128) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: key_stride < 128", fn);
    if (num_tokens == 0 || num_slots == 0) return ok();
    if (!keys || !slots || !cache) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL keys, slots or cache", fn);
    if (!aligned(keys, 8) || (num_tokens > 1 && key_stride % 4 != 0) || !aligned(cache, 8) || row_stride % 4 != 0 ||
        !aligned(slots, 8) || (positions && !aligned(positions, 8)))
        return fail(QSA_ERR_LAYOUT, "%s: keys, slots, cache and positions must be 8-byte aligned and the key and "
                                    "cache row strides multiples of 4 elements (8-byte moves)", fn);
    if (num_slots > ((int64_t)1 << 50) / row_stride) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cache too large", fn);
    if ((int64_t)num_tokens * 32 >= INT32_MAX) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    qsa::WriteKeysParams p{};
    p.keys = static_cast<const uint16_t *>(keys);
    p.key_stride = num_tokens > 1 ? key_stride : 128;
    p.num_tokens = num_tokens;
    p.slots = slots;
    p.cache = cache;
    p.row_stride = row_stride;
    p.num_slots = num_slots;
    p.fp8 = fp8;
    p.scale = scale;
    p.positions = positions;
    p.pos_stride_axis = pos_stride_axis;
    p.pos_stride_token = pos_stride_token;
    return device_status(fn, qsa::launch_write_keys(p, static_cast<hipStream_t>(stream)));
}

int qsa_gather_keys(const void *k_cache, int32_t k_dtype, int64_t num_pages, int32_t page_size,
                    const int32_t *page_table, int64_t page_table_stride, int32_t page_table_cols,
                    const int32_t *key_counts, const int32_t *key_offsets, int32_t num_reqs, int32_t max_keys,
                    void *k_out, int32_t out_dtype, int64_t k_out_stride, int64_t k_out_rows, void *stream) {
    const char *fn = "qsa_gather_keys";
    if (k_dtype != QSA_DTYPE_BF16 && k_dtype != QSA_DTYPE_FP16 && k_dtype != QSA_DTYPE_FP8_E4M3)
        return fail(QSA_ERR_UNSUPPORTED, "%s: key format %d", fn, k_dtype);
    const bool widen = k_dtype == QSA_DTYPE_FP8_E4M3 && (out_dtype == QSA_DTYPE_BF16 || out_dtype == QSA_DTYPE_FP16);
    if (out_dtype != k_dtype && !widen)
        return fail(QSA_ERR_UNSUPPORTED, "%s: output format %d: the key format, or bf16/fp16 for e4m3 keys", fn,
                    out_dtype);
    if (num_reqs < 0 || num_pages < 0 || page_table_cols < 0 || max_keys < 0 || k_out_rows < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (page_size < 1 || page_size > (1 << 20))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_size must be in [1, 2^20], got %d", fn, page_size);
    if (max_keys > (1 << 30)) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: max_keys above 2^30", fn);
    const int64_t elem = out_dtype == QSA_DTYPE_FP8_E4M3 ? 1 : 2;  // output element bytes
    if (k_out_stride < 128) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: k_out_stride < 128", fn);
    if (num_reqs > 1 && page_table_stride < page_table_cols)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_table_stride < page_table_cols", fn);
    if (num_pages > ((int64_t)1 << 46) / page_size) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: key cache too large", fn);
    if (num_reqs == 0 || max_keys == 0 || k_out_rows == 0) return ok();
    if (!key_counts || !key_offsets || !k_out)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL key_counts, key_offsets or k_out", fn);
    if (num_pages > 0 && !k_cache) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL k_cache", fn);
    if (page_table_cols > 0 && !page_table) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL page_table", fn);
    if ((num_pages > 0 && !aligned(k_cache, 16)) || !aligned(k_out, 16) || (k_out_stride * elem) % 16 != 0)
        return fail(QSA_ERR_LAYOUT, "%s: k_cache, k_out and the k_out row stride must be 16-byte aligned "
                                    "(16-byte vector copies)", fn);
    const int64_t chunks = ((int64_t)max_keys + 255) / 256;
    if (chunks * num_reqs >= INT32_MAX) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    qsa::GatherParams p{};
    p.k_cache = static_cast<const uint8_t *>(k_cache);
    p.row_bytes = k_dtype == QSA_DTYPE_FP8_E4M3 ? 128 : 256;
    p.widen = widen ? (out_dtype == QSA_DTYPE_FP16 ? 2 : 1) : 0;
    p.num_pages = num_pages;
    p.page_size = page_size;
    p.page_table = page_table;
    p.page_table_stride = page_table_stride;
    p.page_table_cols = page_table ? page_table_cols : 0;
    p.key_counts = key_counts;
    p.key_offsets = key_offsets;
    p.num_reqs = num_reqs;
    p.max_keys = max_keys;
    p.k_out = static_cast<uint8_t *>(k_out);
    p.k_out_stride_bytes = k_out_stride * elem;
    p.k_out_rows = k_out_rows;
    return device_status(fn, qsa::launch_gather_keys(p, static_cast<hipStream_t>(stream)));
}

int qsa_prepare_q(const void *q, int64_t q_stride_token, int32_t num_tokens, int32_t num_heads,
                  const int64_t *positions, int64_t pos_stride_axis, int64_t pos_stride_token,
                  const void *cos_sin, int32_t cos_sin_dtype, int64_t cos_sin_rows, const void *norm_weight,
                  int32_t weight_dtype, float eps, const int32_t *mrope_section, void *q_out,
                  int32_t out_dtype, float out_scale, int64_t out_stride_token, int64_t out_stride_head,
                  void *stream) {
    const char *fn = "qsa_prepare_q";
    if (cos_sin_dtype != QSA_DTYPE_BF16 && cos_sin_dtype != QSA_DTYPE_FP32)
        return fail(QSA_ERR_UNSUPPORTED, "%s: cos/sin table format %d is not bf16 or fp32", fn, cos_sin_dtype);
    if (weight_dtype != QSA_DTYPE_BF16 && weight_dtype != QSA_DTYPE_FP32)
        return fail(QSA_ERR_UNSUPPORTED, "%s: norm weight format %d is not bf16 or fp32", fn, weight_dtype);
    if (out_dtype != QSA_DTYPE_BF16 && out_dtype != QSA_DTYPE_FP8_E4M3)
        return fail(QSA_ERR_UNSUPPORTED, "%s: output format %d is not bf16 or e4m3", fn, out_dtype);
    if (num_tokens < 0 || cos_sin_rows < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (num_heads < 1 || num_heads > 1024)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: num_heads must be in [1, 1024], got %d", fn, num_heads);
    if (!std::isfinite(eps)) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: eps must be finite", fn);
    if (out_dtype == QSA_DTYPE_FP8_E4M3 && !(std::isfinite(out_scale) && out_scale > 0.0f))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: out_scale must be finite and > 0 for e4m3 output", fn);
    int32_t sec_h = 0, sec_w = 0;
    if (mrope_section) {
        const int32_t a = mrope_section[0], b = mrope_section[1], c = mrope_section[2];
        if (a < 0 || b < 0 || c < 0 || (int64_t)a + b + c != 32)
            return fail(QSA_ERR_INVALID_ARGUMENT, "%s: MRoPE section (%d, %d, %d) must be >= 0 and sum to 32", fn,
                        a, b, c);
        sec_h = b;
        sec_w = c;
    }
    if (num_tokens > 1 && q_stride_token < (int64_t)num_heads * 128)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: q_stride_token < num_heads * 128", fn);
    if (num_tokens == 0) return ok();
    if (!q || !positions || (!cos_sin && cos_sin_rows > 0) || !norm_weight || !q_out)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL q, positions, cos_sin, norm_weight or q_out", fn);
    if ((int64_t)num_tokens * num_heads >= ((int64_t)1 << 31))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    if (cos_sin_rows > (int64_t)INT32_MAX / (cos_sin_dtype == QSA_DTYPE_FP32 ? 256 : 128))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cos/sin table above 2^31 bytes", fn);
    const int out_align = out_dtype == QSA_DTYPE_FP8_E4M3 ? 8 : 16;
    if (!aligned(q, 16) || q_stride_token % 8 != 0 || !aligned(cos_sin, 16) || !aligned(norm_weight, 16) ||
        !aligned(positions, 8) || !aligned(q_out, out_align) || out_stride_token % 8 != 0 ||
        out_stride_head % 8 != 0)
        return fail(QSA_ERR_LAYOUT, "%s: q, cos_sin and norm_weight must be 16-byte aligned, q_out %d-byte "
                                    "aligned, and the q and q_out strides multiples of 8 elements",
                    fn, out_align);
    qsa::PrepareQParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_stride_token = q_stride_token;
    p.num_tokens = num_tokens;
    p.num_heads = num_heads;
    p.positions = positions;
    p.pos_stride_axis = mrope_section ? pos_stride_axis : 0;
    p.pos_stride_token = pos_stride_token;
    p.cos_sin = cos_sin;
    p.cos_sin_rows = cos_sin_rows;
    p.weight = norm_weight;
    p.eps = eps;
    p.mrope = mrope_section ? 1 : 0;
    p.mrope_h = sec_h;
    p.mrope_w = sec_w;
    p.out = q_out;
    p.out_stride_token = out_stride_token;
    p.out_stride_head = out_stride_head;
    p.out_scale = out_scale;
    p.table_f32 = cos_sin_dtype == QSA_DTYPE_FP32;
    p.weight_f32 = weight_dtype == QSA_DTYPE_FP32;
    p.out_fp8 = out_dtype == QSA_DTYPE_FP8_E4M3;
    return device_status(fn, qsa::launch_prepare_q(p, static_cast<hipStream_t>(stream)));
}

// Query format must be bf16 or fp16; keys share it or are e4m3 codes with a
// positive finite cache scale.
static int check_formats(const char *fn, int32_t q_dtype, int32_t k_dtype, float k_scale) {
    if (q_dtype != QSA_DTYPE_BF16 && q_dtype != QSA_DTYPE_FP16)
        return fail(QSA_ERR_UNSUPPORTED, "%s: query format %d is not QSA_DTYPE_BF16 or QSA_DTYPE_FP16", fn,
                    q_dtype);
    if (k_dtype != q_dtype && k_dtype != QSA_DTYPE_FP8_E4M3)
        return fail(QSA_ERR_UNSUPPORTED, "%s: key format %d: keys are the query's format or QSA_DTYPE_FP8_E4M3",
                    fn, k_dtype);
    if (k_dtype == QSA_DTYPE_FP8_E4M3 && !(std::isfinite(k_scale) && k_scale > 0.0f))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: k_scale must be finite and > 0 for fp8 keys", fn);
    return QSA_OK;
}

// plan: null for the mapped launch (tasks from comp_lens), else a task table
// of plan_bytes bytes from qsa_build_decode_plan (comp_lens unused).
// static_plan: build the task table from comp_lens into the library's own
// device array, then run the planned launch (no plan argument).
static int decode_impl(const char *fn, const void *q, int32_t q_dtype, int64_t q_stride_req,
                       int64_t q_stride_row, int64_t q_stride_head, const void *k_cache, int32_t k_dtype,
                       float k_scale, int64_t num_pages, int32_t page_size, const int32_t *page_table,
                       int64_t page_table_stride, int32_t page_table_cols, const int32_t *comp_lens,
                       const int32_t *visible, int32_t num_reqs, int32_t dql, int32_t num_heads,
                       int32_t head_dim, float scale, float *out, int64_t out_stride, int32_t out_cols,
                       void *stream, const void *plan = nullptr, int64_t plan_bytes = 0,
                       bool static_plan = false) {
    int rc;
    if ((rc = check_heads(fn, num_heads, head_dim))) return rc;
    if ((rc = check_scale(fn, scale))) return rc;
    if ((rc = check_formats(fn, q_dtype, k_dtype, k_scale))) return rc;
    const bool k_fp8 = k_dtype == QSA_DTYPE_FP8_E4M3;
    // The cache scale multiplies each key element; it leaves the ReLU and
    // head sum as a positive factor, so it joins the score multiplier.
    const float mult = k_fp8 ? scale * k_scale : scale;
    if (!(std::isfinite(mult) && mult > 0.0f))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: scale * k_scale is not a finite positive fp32", fn);
    if (num_reqs < 0 || out_cols < 0 || num_pages < 0 || page_table_cols < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (dql < 1 || dql > 16) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: dql must be in [1, 16], got %d", fn, dql);
    if (page_size < 1 || page_size > (1 << 20))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_size must be in [1, 2^20], got %d", fn, page_size);
    if (out_stride < out_cols) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: out_stride < out_cols", fn);
    if (num_reqs > 1 && page_table_stride < page_table_cols)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_table_stride < page_table_cols", fn);
    if (num_pages > ((int64_t)1 << 46) / page_size)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: key cache too large", fn);
    if (num_reqs == 0 || out_cols == 0) return ok();
    if (!q || !out || (!plan && !comp_lens))
        return fail(QSA_ERR_INVALID_ARGUMENT, plan ? "%s: NULL q or out" : "%s: NULL q, comp_lens or out", fn);
    if (num_pages > 0 && !k_cache) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL k_cache", fn);
    if (page_table_cols > 0 && !page_table) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL page_table", fn);
    if (num_pages > 0 && !aligned(k_cache, 16))
        return fail(QSA_ERR_LAYOUT, "%s: k_cache must be 16-byte aligned (16-byte vector loads)", fn);
    if (!aligned(out, 4)) return fail(QSA_ERR_LAYOUT, "%s: out must be 4-byte aligned", fn);
    if (!aligned(q, 2)) return fail(QSA_ERR_LAYOUT, "%s: q must be 2-byte aligned", fn);
    const int64_t span_keys = qsa::decode_span_keys();
    const int64_t spans = ((int64_t)out_cols + span_keys - 1) / span_keys;
    if ((int64_t)num_reqs * dql > INT32_MAX || (int64_t)num_reqs * spans >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    const int64_t plan_need = (int64_t)num_reqs * spans * 16;
    if (plan) {
        if (!aligned(plan, 16)) return fail(QSA_ERR_LAYOUT, "%s: plan must be 16-byte aligned", fn);
        if (plan_bytes < plan_need)
            return fail(QSA_ERR_INVALID_ARGUMENT, "%s: plan of %lld bytes, %lld needed for %d requests x %d columns",
                        fn, (long long)plan_bytes, (long long)plan_need, num_reqs, out_cols);
    }

    qsa::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_stride_req = q_stride_req;
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.k = static_cast<const uint16_t *>(k_cache);
    p.num_pages = num_pages;
    p.page_size = page_size;
    p.page_table = page_table;
    p.page_table_stride = page_table_stride;
    p.page_table_cols = page_table_cols;
    p.comp_lens = comp_lens;
    p.visible = visible;
    p.num_reqs = num_reqs;
    p.dql = dql;
    p.scale = mult;
    p.out = out;
    p.out_stride = out_stride;
    p.out_cols = out_cols;
    p.spans = (int32_t)spans;
    p.q_vec = aligned(q, 16) && q_stride_req % 8 == 0 && q_stride_row % 8 == 0 && q_stride_head % 8 == 0;
    p.out_vec = aligned(out, 16) && out_stride % 4 == 0;
    p.q_f16 = q_dtype == QSA_DTYPE_FP16;
    p.k_fp8 = k_fp8;
    p.plan = static_cast<const int32_t *>(plan);
    p.plan_entries = plan ? (int64_t)num_reqs * spans : 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (!static_plan) return device_status(fn, qsa::launch_decode(p, st));

    // The task table goes to the library's device array: two launches, no
    // allocation.  Every entry the decode reads is written by the first.
    const int64_t entries = (int64_t)num_reqs * spans;
    if (entries > qsa::static_plan_entries())
        return fail(QSA_ERR_UNSUPPORTED,
                    "%s: %d requests x %d columns need %lld task entries; the library's table holds %lld "
                    "(use qsa_build_decode_plan with a caller-owned table)",
                    fn, num_reqs, out_cols, (long long)entries, (long long)qsa::static_plan_entries());
    if (num_reqs > qsa::kPlanMaxReqs)
        return fail(QSA_ERR_UNSUPPORTED, "%s: plans for more than %d requests", fn, qsa::kPlanMaxReqs);
    int32_t *table = nullptr;
    const hipError_t terr = qsa::static_plan_pointer(&table);
    if (terr != hipSuccess)
        return fail(QSA_ERR_DEVICE, "%s: the library's task table is not available: %s", fn, hipGetErrorString(terr));
    qsa::PlanParams pp{};
    pp.comp_lens = comp_lens;
    pp.page_table = page_table;
    pp.page_table_stride = page_table_stride;
    pp.page_table_cols = page_table ? page_table_cols : 0;
    pp.num_pages = num_pages;
    pp.page_size = page_size;
    pp.num_reqs = num_reqs;
    pp.spans = (int32_t)spans;
    pp.plan = table;
    pp.entries = entries;
    p.plan = table;
    p.plan_entries = entries;
    // Armed timing events span both launches.
    const qsa::LaunchEvents ev = g_launch_events;
    g_launch_events = {ev.start, nullptr};
    hipError_t err = qsa::launch_decode_plan(pp, st);
    g_launch_events = {nullptr, ev.stop};
    if (err == hipSuccess) err = qsa::launch_decode(p, st);
    g_launch_events = ev;
    return device_status(fn, err);
}

int qsa_decode_plan_bytes(int32_t num_reqs, int32_t out_cols, int64_t *bytes) {
    const char *fn = "qsa_decode_plan_bytes";
    if (!bytes) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL bytes", fn);
    if (num_reqs < 0 || out_cols < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    const int64_t span_keys = qsa::decode_span_keys();
    *bytes = (int64_t)num_reqs * (((int64_t)out_cols + span_keys - 1) / span_keys) * 16;
    return ok();
}

int qsa_build_decode_plan(const int32_t *comp_lens, const int32_t *page_table, int64_t page_table_stride,
                          int32_t page_table_cols, int64_t num_pages, int32_t page_size, int32_t num_reqs,
                          int32_t out_cols, void *plan, int64_t plan_bytes, void *stream) {
    const char *fn = "qsa_build_decode_plan";
    if (num_reqs < 0 || out_cols < 0 || num_pages < 0 || page_table_cols < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (page_size < 1 || page_size > (1 << 20))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_size must be in [1, 2^20], got %d", fn, page_size);
    if (num_reqs > 1 && page_table_stride < page_table_cols)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: page_table_stride < page_table_cols", fn);
    if (num_reqs > qsa::kPlanMaxReqs)
        return fail(QSA_ERR_UNSUPPORTED, "%s: plans for more than %d requests", fn, qsa::kPlanMaxReqs);
    const int64_t span_keys = qsa::decode_span_keys();
    const int64_t spans = ((int64_t)out_cols + span_keys - 1) / span_keys;
    if ((int64_t)num_reqs * spans >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    const int64_t need = (int64_t)num_reqs * spans * 16;
    if (need == 0) return ok();
    if (!comp_lens || !plan) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL comp_lens or plan", fn);
    if (page_table_cols > 0 && !page_table) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL page_table", fn);
    if (!aligned(plan, 16)) return fail(QSA_ERR_LAYOUT, "%s: plan must be 16-byte aligned", fn);
    if (plan_bytes < need)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: plan of %lld bytes, %lld needed", fn, (long long)plan_bytes,
                    (long long)need);
    qsa::PlanParams p{};
    p.comp_lens = comp_lens;
    p.page_table = page_table;
    p.page_table_stride = page_table_stride;
    p.page_table_cols = page_table ? page_table_cols : 0;
    p.num_pages = num_pages;
    p.page_size = page_size;
    p.num_reqs = num_reqs;
    p.spans = (int32_t)spans;
    p.plan = static_cast<int32_t *>(plan);
    p.entries = (int64_t)num_reqs * spans;
    return device_status(fn, qsa::launch_decode_plan(p, static_cast<hipStream_t>(stream)));
}

int qsa_mqa_decode_static_plan(const void *q, int32_t q_dtype, int64_t q_stride_req, int64_t q_stride_row,
                               int64_t q_stride_head, const void *k_cache, int32_t k_dtype, float k_scale,
                               int64_t num_pages, int32_t page_size, const int32_t *page_table,
                               int64_t page_table_stride, int32_t page_table_cols, const int32_t *comp_lens,
                               const int32_t *visible, int32_t num_reqs, int32_t dql, int32_t num_heads,
                               int32_t head_dim, float scale, float *out, int64_t out_stride, int32_t out_cols,
                               void *stream) {
    return decode_impl("qsa_mqa_decode_static_plan", q, q_dtype, q_stride_req, q_stride_row, q_stride_head, k_cache,
                       k_dtype, k_scale, num_pages, page_size, page_table, page_table_stride, page_table_cols,
                       comp_lens, visible, num_reqs, dql, num_heads, head_dim, scale, out, out_stride, out_cols,
                       stream, nullptr, 0, true);
}

int qsa_mqa_decode_planned(const void *plan, int64_t plan_bytes, const void *q, int32_t q_dtype,
                           int64_t q_stride_req, int64_t q_stride_row, int64_t q_stride_head, const void *k_cache,
                           int32_t k_dtype, float k_scale, int64_t num_pages, int32_t page_size,
                           const int32_t *page_table, int64_t page_table_stride, int32_t page_table_cols,
                           const int32_t *visible, int32_t num_reqs, int32_t dql, int32_t num_heads,
                           int32_t head_dim, float scale, float *out, int64_t out_stride, int32_t out_cols,
                           void *stream) {
    const char *fn = "qsa_mqa_decode_planned";
    if (!plan && num_reqs > 0 && out_cols > 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL plan", fn);
    return decode_impl(fn, q, q_dtype, q_stride_req, q_stride_row, q_stride_head, k_cache, k_dtype, k_scale,
                       num_pages, page_size, page_table, page_table_stride, page_table_cols, nullptr, visible,
                       num_reqs, dql, num_heads, head_dim, scale, out, out_stride, out_cols, stream, plan,
                       plan_bytes);
}

int qsa_mqa_decode(const void *q, int64_t q_stride_req, int64_t q_stride_row, int64_t q_stride_head,
                   const void *k_cache, int64_t num_pages, int32_t page_size, const int32_t *page_table,
                   int64_t page_table_stride, int32_t page_table_cols, const int32_t *comp_lens,
                   const int32_t *visible, int32_t num_reqs, int32_t dql, int32_t num_heads,
                   int32_t head_dim, float scale, float *out, int64_t out_stride, int32_t out_cols,
                   void *stream) {
    return decode_impl("qsa_mqa_decode", q, QSA_DTYPE_BF16, q_stride_req, q_stride_row, q_stride_head, k_cache,
                       QSA_DTYPE_BF16, 1.0f, num_pages, page_size, page_table, page_table_stride,
                       page_table_cols, comp_lens, visible, num_reqs, dql, num_heads, head_dim, scale, out,
                       out_stride, out_cols, stream);
}

int qsa_mqa_decode_typed(const void *q, int32_t q_dtype, int64_t q_stride_req, int64_t q_stride_row,
                         int64_t q_stride_head, const void *k_cache, int32_t k_dtype, float k_scale,
                         int64_t num_pages, int32_t page_size, const int32_t *page_table,
                         int64_t page_table_stride, int32_t page_table_cols, const int32_t *comp_lens,
                         const int32_t *visible, int32_t num_reqs, int32_t dql, int32_t num_heads,
                         int32_t head_dim, float scale, float *out, int64_t out_stride, int32_t out_cols,
                         void *stream) {
    return decode_impl("qsa_mqa_decode_typed", q, q_dtype, q_stride_req, q_stride_row, q_stride_head, k_cache,
                       k_dtype, k_scale, num_pages, page_size, page_table, page_table_stride, page_table_cols,
                       comp_lens, visible, num_reqs, dql, num_heads, head_dim, scale, out, out_stride, out_cols,
                       stream);
}

static int prefill_impl(const char *fn, const void *q, int64_t q_stride_row, int64_t q_stride_head,
                        const void *k, int64_t k_stride, int64_t num_keys, int32_t dtype,
                        const int32_t *row_k_start, const int32_t *row_k_end, int32_t num_rows,
                        int32_t num_heads, int32_t head_dim, float scale, float *out, int64_t out_stride,
                        int32_t out_cols, void *stream) {
    int rc;
    if ((rc = check_heads(fn, num_heads, head_dim))) return rc;
    if ((rc = check_scale(fn, scale))) return rc;
    if (dtype != QSA_DTYPE_BF16 && dtype != QSA_DTYPE_FP16)
        return fail(QSA_ERR_UNSUPPORTED, "%s: format %d is not QSA_DTYPE_BF16 or QSA_DTYPE_FP16", fn, dtype);
    if (num_rows < 0 || out_cols < 0 || num_keys < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (out_stride < out_cols) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: out_stride < out_cols", fn);
    if (num_rows == 0 || out_cols == 0) return ok();
    if (!q || !out || !row_k_start || !row_k_end)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL q, out, row_k_start or row_k_end", fn);
    if (num_keys > 0 && !k) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL k", fn);
    if (!aligned(q, 16) || !axis_ok(num_rows, q_stride_row) || !axis_ok(4, q_stride_head) ||
        (num_keys > 0 && (!aligned(k, 16) || !axis_ok(num_keys, k_stride))))
        return fail(QSA_ERR_LAYOUT,
                    "%s: q and k need a 16-byte aligned base and positive strides that are multiples "
                    "of 8 elements on every axis longer than 1 (16-byte vector loads)", fn);
    if (!aligned(out, 4)) return fail(QSA_ERR_LAYOUT, "%s: out must be 4-byte aligned", fn);
    // The stride of a single key is never used; normalise it.
    if (num_keys <= 1) k_stride = 128;
    if (k_stride > qsa::prefill_max_k_stride())
        return fail(QSA_ERR_UNSUPPORTED, "%s: k_stride %lld exceeds %lld elements", fn, (long long)k_stride,
                    (long long)qsa::prefill_max_k_stride());

    const int bm = qsa::prefill_rows_per_block();
    const int chunk = qsa::prefill_col_chunk(num_rows, out_cols, k_stride, current_cu_count());
    const int64_t row_blocks = ((int64_t)num_rows + bm - 1) / bm;
    const int64_t col_chunks = ((int64_t)out_cols + chunk - 1) / chunk;
    if (row_blocks * col_chunks >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);

    qsa::PrefillParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.k = static_cast<const uint16_t *>(k);
    p.k_stride = k_stride;
    p.num_keys = num_keys;
    p.row_k_start = row_k_start;
    p.row_k_end = row_k_end;
    p.num_rows = num_rows;
    p.scale = scale;
    p.out = out;
    p.out_stride = out_stride;
    p.out_cols = out_cols;
    p.col_chunk = chunk;
    p.row_blocks = (int32_t)row_blocks;
    p.col_chunks = (int32_t)col_chunks;
    p.out_vec = aligned(out, 16) && out_stride % 4 == 0;
    p.exact_stores = p.out_vec && (int64_t)bm * out_stride * 4 < ((int64_t)1 << 31);
    p.f16 = dtype == QSA_DTYPE_FP16;
    // Rows that all start on a 128-byte line need no line-aligned layout.
    p.rotate = p.exact_stores && !(aligned(out, 128) && (out_stride * 4) % 128 == 0);
    return device_status(fn, qsa::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

int qsa_mqa_prefill(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                    int64_t k_stride, int64_t num_keys, const int32_t *row_k_start,
                    const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                    float scale, float *out, int64_t out_stride, int32_t out_cols, void *stream) {
    return prefill_impl("qsa_mqa_prefill", q, q_stride_row, q_stride_head, k, k_stride, num_keys, QSA_DTYPE_BF16,
                        row_k_start, row_k_end, num_rows, num_heads, head_dim, scale, out, out_stride, out_cols,
                        stream);
}

int qsa_mqa_prefill_typed(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                          int64_t k_stride, int64_t num_keys, int32_t dtype, const int32_t *row_k_start,
                          const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                          float scale, float *out, int64_t out_stride, int32_t out_cols, void *stream) {
    return prefill_impl("qsa_mqa_prefill_typed", q, q_stride_row, q_stride_head, k, k_stride, num_keys, dtype,
                        row_k_start, row_k_end, num_rows, num_heads, head_dim, scale, out, out_stride, out_cols,
                        stream);
}

int qsa_topk_blocks(const float *logits, int64_t logits_stride, int32_t num_rows, int32_t num_cols,
                    int32_t k, int32_t *out_idx, int64_t out_stride, void *stream) {
    const char *fn = "qsa_topk_blocks";
    if (num_rows < 0 || num_cols < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (k < 1 || k > (1 << 20)) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: k must be in [1, 2^20], got %d", fn, k);
    if (logits_stride < num_cols) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: logits_stride < num_cols", fn);
    if (out_stride < k) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: out_stride < k", fn);
    if (num_rows == 0) return ok();
    if (!out_idx || (num_cols > 0 && !logits))
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL logits or out_idx", fn);
    if (!aligned(logits, 4) || !aligned(out_idx, 4))
        return fail(QSA_ERR_LAYOUT, "%s: logits and out_idx must be 4-byte aligned", fn);
    qsa::TopkParams p{logits, logits_stride, num_rows, num_cols, k, out_idx, out_stride,
                      aligned(logits, 16) && logits_stride % 4 == 0};
    return device_status(fn, qsa::launch_topk(p, static_cast<hipStream_t>(stream), current_cu_count()));
}

int qsa_prefill_topk_workspace_bytes(int32_t num_rows, int32_t out_cols, int32_t topk, int64_t *bytes) {
    const char *fn = "qsa_prefill_topk_workspace_bytes";
    if (!bytes) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL bytes", fn);
    if (num_rows < 0 || out_cols < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (topk < 1 || topk > qsa::kFusedMaxK)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: topk must be in [1, %d], got %d", fn, qsa::kFusedMaxK, topk);
    *bytes = use_keys16(out_cols) ? keys16_layout(num_rows, out_cols).total
                                  : fused_layout(num_rows, out_cols, topk, current_cu_count()).total;
    return ok();
}

// qsa_mqa_prefill_topk on rows of 1 .. kKeys16MaxCols columns: the prefill
// pass storing the cells' 16-bit key prefixes, the select over them
// (rescoring the cells that tie the k-th largest prefix), and the fallback
// for rows that select leaves.  Arguments already checked by the caller:
// sizes, scale, topk, out_idx and the workspace's alignment.
static int prefill_topk_keys16(const char *fn, const void *q, int64_t q_stride_row, int64_t q_stride_head,
                               const void *k, int64_t k_stride, int64_t num_keys, bool f16, const int32_t *row_k_start,
                               const int32_t *row_k_end, int32_t num_rows, float scale, int32_t out_cols,
                               int32_t topk, int32_t *out_idx, int64_t out_stride, void *workspace,
                               int64_t workspace_bytes, void *stream, int cus) {
    const Keys16Layout L = keys16_layout(num_rows, out_cols);
    if (workspace_bytes < L.total)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace of %lld bytes, %lld needed", fn,
                    (long long)workspace_bytes, (long long)L.total);
    if (!q || !row_k_start || !row_k_end) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL q, row_k_start or row_k_end", fn);
    if (num_keys > 0 && !k) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL k", fn);
    if (!aligned(q, 16) || !axis_ok(num_rows, q_stride_row) || !axis_ok(4, q_stride_head) ||
        (num_keys > 0 && (!aligned(k, 16) || !axis_ok(num_keys, k_stride))))
        return fail(QSA_ERR_LAYOUT,
                    "%s: q and k need a 16-byte aligned base and positive strides that are multiples "
                    "of 8 elements on every axis longer than 1 (16-byte vector loads)", fn);
    if (num_keys <= 1) k_stride = 128;
    if (k_stride > qsa::prefill_max_k_stride())
        return fail(QSA_ERR_UNSUPPORTED, "%s: k_stride %lld exceeds %lld elements", fn, (long long)k_stride,
                    (long long)qsa::prefill_max_k_stride());
    const int bm = qsa::prefill_rows_per_block();
    const int chunk = qsa::prefill_col_chunk(num_rows, out_cols, k_stride, cus);
    const int64_t row_blocks = ((int64_t)num_rows + bm - 1) / bm;
    const int64_t col_chunks = ((int64_t)out_cols + chunk - 1) / chunk;
    if (row_blocks * col_chunks >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    char *ws = static_cast<char *>(workspace);

    qsa::PrefillParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.k = static_cast<const uint16_t *>(k);
    p.k_stride = k_stride;
    p.num_keys = num_keys;
    p.row_k_start = row_k_start;
    p.row_k_end = row_k_end;
    p.num_rows = num_rows;
    p.scale = scale;
    p.out_cols = out_cols;
    p.col_chunk = chunk;
    p.row_blocks = (int32_t)row_blocks;
    p.col_chunks = (int32_t)col_chunks;
    p.f16 = f16;
    p.keys16 = reinterpret_cast<uint16_t *>(ws + L.off_keys);
    p.keys_stride = L.stride;
    p.hard_count = reinterpret_cast<int32_t *>(ws + L.off_count);

    qsa::Keys16TopkParams t{};
    t.keys = p.keys16;
    t.keys_stride = L.stride;
    t.num_rows = num_rows;
    t.num_cols = out_cols;
    t.k = topk;
    t.out = out_idx;
    t.out_stride = out_stride;
    t.q = p.q;
    t.q_stride_row = q_stride_row;
    t.q_stride_head = q_stride_head;
    t.kv = p.k;
    t.k_stride = k_stride;
    t.num_keys = num_keys;
    t.row_k_start = row_k_start;
    t.row_k_end = row_k_end;
    t.scale = scale;
    t.f16 = f16;
    t.hard_count = p.hard_count;
    t.hard_rows = reinterpret_cast<int32_t *>(ws + L.off_hard);
    t.scratch = reinterpret_cast<float *>(ws + L.off_scratch);
    t.scratch_stride = L.stride;
    t.scratch_rows = qsa::kKeys16FallbackGroups;

    // Three launches; armed timing events span them.
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const qsa::LaunchEvents ev = g_launch_events;
    g_launch_events = {ev.start, nullptr};
    hipError_t err = qsa::launch_prefill_keys16(p, st);
    g_launch_events = {nullptr, nullptr};
    if (err == hipSuccess) err = qsa::launch_topk_keys16(t, st);
    g_launch_events = {nullptr, ev.stop};
    if (err == hipSuccess) err = qsa::launch_topk_keys16_fallback(t, st);
    g_launch_events = ev;
    return device_status(fn, err);
}

static int prefill_topk_impl(const char *fn, const void *q, int64_t q_stride_row, int64_t q_stride_head,
                             const void *k, int64_t k_stride, int64_t num_keys, int32_t dtype,
                             const int32_t *row_k_start, const int32_t *row_k_end, int32_t num_rows,
                             int32_t num_heads, int32_t head_dim, float scale, int32_t out_cols, int32_t topk,
                             int32_t *out_idx, int64_t out_stride, void *workspace, int64_t workspace_bytes,
                             void *stream) {
    int rc;
    if ((rc = check_heads(fn, num_heads, head_dim))) return rc;
    if ((rc = check_scale(fn, scale))) return rc;
    if (dtype != QSA_DTYPE_BF16 && dtype != QSA_DTYPE_FP16)
        return fail(QSA_ERR_UNSUPPORTED, "%s: format %d is not QSA_DTYPE_BF16 or QSA_DTYPE_FP16", fn, dtype);
    if (num_rows < 0 || out_cols < 0 || num_keys < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (topk < 1 || topk > qsa::kFusedMaxK)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: topk must be in [1, %d], got %d", fn, qsa::kFusedMaxK, topk);
    if (out_stride < topk) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: out_stride < topk", fn);
    if (num_rows == 0) return ok();
    if (!out_idx || !workspace) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL out_idx or workspace", fn);
    if (!aligned(out_idx, 4)) return fail(QSA_ERR_LAYOUT, "%s: out_idx must be 4-byte aligned", fn);
    if (!aligned(workspace, 256)) return fail(QSA_ERR_LAYOUT, "%s: workspace must be 256-byte aligned", fn);
    const int cus = current_cu_count();
    if (use_keys16(out_cols))
        return prefill_topk_keys16(fn, q, q_stride_row, q_stride_head, k, k_stride, num_keys, dtype == QSA_DTYPE_FP16,
                                   row_k_start, row_k_end, num_rows, scale, out_cols, topk, out_idx, out_stride,
                                   workspace, workspace_bytes, stream, cus);
    if (dtype != QSA_DTYPE_BF16 && out_cols > 0)
        return fail(QSA_ERR_UNSUPPORTED, "%s: fp16 rows wider than %d columns are not supported", fn,
                    qsa::kKeys16MaxCols);
    const FusedLayout L = fused_layout(num_rows, out_cols, topk, cus);
    if (workspace_bytes < L.total)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace of %lld bytes, %lld needed", fn,
                    (long long)workspace_bytes, (long long)L.total);
    char *ws = static_cast<char *>(workspace);
    qsa::FusedTopkParams fp{};
    fp.num_rows = num_rows;
    fp.k = topk;
    fp.gmax = reinterpret_cast<float *>(ws + L.off_gmax);
    fp.gmax_stride = (int32_t)L.groups;
    fp.floor_key = reinterpret_cast<uint32_t *>(ws + L.off_floor);
    fp.cand = reinterpret_cast<uint32_t *>(ws + L.off_cand);
    fp.cand_cnt = reinterpret_cast<int32_t *>(ws + L.off_cnt);
    fp.seg_off = reinterpret_cast<int32_t *>(ws + L.off_segoff);
    fp.segs = (int32_t)L.col_chunks;
    fp.groups_per_seg = L.chunk / qsa::kFusedGroupKeys;
    fp.out_cols = out_cols;
    fp.pool_cap = (int32_t)L.pool_cap;
    fp.out = out_idx;
    fp.out_stride = out_stride;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (out_cols == 0) {  // no columns: every row is -1
        fp.cand_cnt = nullptr;
        return device_status(fn, qsa::launch_topk_candidates(fp, st));
    }
    if (!q || !row_k_start || !row_k_end) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL q, row_k_start or row_k_end", fn);
    if (num_keys > 0 && !k) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL k", fn);
    if (!aligned(q, 16) || !axis_ok(num_rows, q_stride_row) || !axis_ok(4, q_stride_head) ||
        (num_keys > 0 && (!aligned(k, 16) || !axis_ok(num_keys, k_stride))))
        return fail(QSA_ERR_LAYOUT,
                    "%s: q and k need a 16-byte aligned base and positive strides that are multiples "
                    "of 8 elements on every axis longer than 1 (16-byte vector loads)", fn);
    if (num_keys <= 1) k_stride = 128;
    if (k_stride > kFusedMaxKStride)
        return fail(QSA_ERR_UNSUPPORTED, "%s: k_stride %lld exceeds %lld elements", fn, (long long)k_stride,
                    (long long)kFusedMaxKStride);
    if (((int64_t)L.chunk + 64) * k_stride * 2 > ((int64_t)1 << 30) ||  // 32-bit key offsets per chunk
        (int64_t)qsa::prefill_rows_per_block() * L.groups * 4 >= ((int64_t)1 << 31) ||  // and per workgroup's
        (int64_t)qsa::prefill_rows_per_block() * L.pool_cap * 8 >= ((int64_t)1 << 31))  // maxima and pools
        return fail(QSA_ERR_UNSUPPORTED, "%s: rows of %d columns are too wide", fn, out_cols);

    qsa::PrefillParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_stride_row = q_stride_row;
    p.q_stride_head = q_stride_head;
    p.k = static_cast<const uint16_t *>(k);
    p.k_stride = k_stride;
    p.num_keys = num_keys;
    p.row_k_start = row_k_start;
    p.row_k_end = row_k_end;
    p.num_rows = num_rows;
    p.scale = scale;
    p.out_cols = out_cols;
    p.col_chunk = L.chunk;
    p.row_blocks = (int32_t)((num_rows + qsa::prefill_rows_per_block() - 1) / qsa::prefill_rows_per_block());
    p.col_chunks = (int32_t)L.col_chunks;
    if ((int64_t)p.row_blocks * p.col_chunks >= INT32_MAX)
        return fail(QSA_ERR_INVALID_ARGUMENT, "%s: problem too large for one launch", fn);
    p.topk = topk;
    p.gmax = reinterpret_cast<float *>(ws + L.off_gmax);
    p.gmax_stride = fp.gmax_stride;
    p.floor_key = fp.floor_key;
    p.cand = reinterpret_cast<uint32_t *>(ws + L.off_cand);
    p.cand_cnt = reinterpret_cast<int32_t *>(ws + L.off_cnt);
    p.seg_off = fp.seg_off;
    p.pool_cap = fp.pool_cap;

    // Four launches; armed timing events span them (start on the first,
    // stop on the last).
    const qsa::LaunchEvents ev = g_launch_events;
    auto arm = [&](bool first, bool last) {
        g_launch_events = {first ? ev.start : nullptr, last ? ev.stop : nullptr};
    };
    arm(true, false);
    hipError_t err = qsa::launch_prefill_group_max(p, st);
    arm(false, false);
    if (err == hipSuccess) err = qsa::launch_topk_floor(fp, st);
    if (err == hipSuccess) err = qsa::launch_prefill_candidates(p, st);
    arm(false, true);
    if (err == hipSuccess) err = qsa::launch_topk_candidates(fp, st);
    g_launch_events = ev;
    return device_status(fn, err);
}

int qsa_mqa_prefill_topk(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                         int64_t k_stride, int64_t num_keys, const int32_t *row_k_start,
                         const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                         float scale, int32_t out_cols, int32_t topk, int32_t *out_idx, int64_t out_stride,
                         void *workspace, int64_t workspace_bytes, void *stream) {
    return prefill_topk_impl("qsa_mqa_prefill_topk", q, q_stride_row, q_stride_head, k, k_stride, num_keys,
                             QSA_DTYPE_BF16, row_k_start, row_k_end, num_rows, num_heads, head_dim, scale, out_cols,
                             topk, out_idx, out_stride, workspace, workspace_bytes, stream);
}

int qsa_mqa_prefill_topk_typed(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                               int64_t k_stride, int64_t num_keys, int32_t dtype, const int32_t *row_k_start,
                               const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                               float scale, int32_t out_cols, int32_t topk, int32_t *out_idx, int64_t out_stride,
                               void *workspace, int64_t workspace_bytes, void *stream) {
    return prefill_topk_impl("qsa_mqa_prefill_topk_typed", q, q_stride_row, q_stride_head, k, k_stride, num_keys,
                             dtype, row_k_start, row_k_end, num_rows, num_heads, head_dim, scale, out_cols, topk,
                             out_idx, out_stride, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace qsa {
LaunchEvents launch_events() { return g_launch_events; }
}  // namespace qsa
