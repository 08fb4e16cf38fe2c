/*
 * qsa.h -- C ABI of the MI355X (gfx950) QSA lightweight MQA indexer.
 *
 * The indexer scores compressed 4-token key blocks for every query row:
 *
 *   score(row, n) = scale * sum_{h<4} max(0, q[row][h][:] . k[n][:])
 *
 * with 4 query heads sharing one 128-wide compressed key head, scale normally
 * 1/sqrt(128), and -inf for every block the row may not see.  Definitions:
 * MATE API docs, page "QSA (Qwen Sparse Attention)", section "MQA score"
 * (score, paged decode form, packed prefill form, layout rules) and section
 * "Core Attention" (request-local int32 block indices, -1 padding); the
 * visibility rule is from the vLLM page "vllm/models/qwen4_exp/common/
 * qsa_cache.py" (_build_qsa_metadata_kernel) and vLLM PR 54513 "Separate
 * prefill and decode paths for QSA indexer" (section "Main changes").
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory (hipMalloc'd or from a
 *     framework allocator).  Host pointers are marked "host".  The library
 *     allocates nothing and keeps no device state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it; no call synchronizes.
 *   - Argument checks read only the host-side arguments, never device
 *     contents, so every call may be captured into a HIP graph.
 *   - Strides are in elements, not bytes.
 *   - Return value: QSA_OK, or an error code with a message available from
 *     qsa_last_error() on the calling thread.  Calls with nothing to compute
 *     (zero rows) return QSA_OK without launching.
 *   - Entry points are thread-safe; calls that write overlapping outputs on
 *     different streams race, as with any kernel.
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 11

enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARGUMENT = 1, /* a size, count, pointer or value is invalid   */
    QSA_ERR_UNSUPPORTED = 2,      /* heads/head_dim other than (4, 128)          */
    QSA_ERR_LAYOUT = 3,           /* alignment or stride rule of the vector loads */
    QSA_ERR_DEVICE = 4            /* the HIP runtime reported an error            */
};

/* Element formats of the typed entry points (qsa_mqa_decode_typed,
 * qsa_mqa_prefill_typed, qsa_gather_keys, qsa_prepare_q).
 *   QSA_DTYPE_BF16, QSA_DTYPE_FP16: 2-byte elements.  MATE "QSA (Qwen Sparse
 *     Attention)", section "MQA score": the query and the compressed key are
 *     BF16 or FP16.
 *   QSA_DTYPE_FP8_E4M3: 1-byte OCP e4m3 codes (bias 7; S.1111.111 is NaN;
 *     largest finite 448), keys only.  The vLLM QSA state backend allows an
 *     e4m3 compressed indexer cache; qsa_prepare's _to_dst_dtype writes it
 *     by rounding to bf16, dividing by the cache scale and converting.  Read
 *     here as the inverse: a key element is its e4m3 value times k_scale.
 *     NaN codes are outside the contract.
 *   QSA_DTYPE_FP32: 4-byte IEEE binary32 (qsa_prepare_q's cos/sin table and
 *     norm weight). */
enum qsa_dtype { QSA_DTYPE_BF16 = 0, QSA_DTYPE_FP16 = 1, QSA_DTYPE_FP8_E4M3 = 2, QSA_DTYPE_FP32 = 3 };

/* QSA_ABI_VERSION of the loaded library. */
int qsa_abi_version(void);

/* Text of the last error returned on this thread ("" if none). */
const char *qsa_last_error(void);

/* qsa_set_launch_events -- per-kernel timing hook (instrumentation; not an
 * operation of the indexer).
 *   While set, every kernel that this library launches from the calling
 *   thread is launched with hipExtLaunchKernel and these events: the runtime
 *   marks start_event when the kernel begins executing and stop_event when
 *   it ends, so hipEventElapsedTime(start, stop) is the kernel's own
 *   duration, without the dispatch latency that an event pair recorded on
 *   the stream around the call adds.  Each entry point below launches one
 *   kernel (none when it has nothing to compute), except
 *   qsa_build_cache_metadata (up to two), qsa_mqa_decode_static_plan (two)
 *   and qsa_mqa_prefill_topk / qsa_mqa_prefill_topk_typed (three, or four
 *   on rows wider than 32,768 columns):
 *   for those the start event marks the first kernel's begin and the stop
 *   event the last kernel's end.
 *   start_event, stop_event : hipEvent_t handles created by the caller (may
 *                             be NULL); owned by the caller, who must keep
 *                             them alive until the launches complete.
 *   Pass NULL, NULL to stop timing.  The setting is per calling thread.
 *   Returns QSA_OK. */
int qsa_set_launch_events(void *start_event, void *stop_event);

/* ------------------------------------------------------------------------
 * Per-step metadata (host and device helpers).
 *
 * qsa_split_batch -- decode/prefill split of one batch (host only).
 *   Source: vLLM page qsa_cache.py, QSAMetadataBuilder (decode threshold
 *   with speculative tokens counted as decode, decodes ordered first, one
 *   uniform decode query length).  Rule used here: a request is a decode when
 *   its query length L satisfies 1 <= L <= decode_threshold and L equals the
 *   decode query length DQL, the length of the first request (in batch order)
 *   with 1 <= L <= decode_threshold.  Empty requests are not decodes.
 *   query_start_loc : host int32 [num_reqs+1], non-decreasing, from 0.
 *   order           : host int32 [num_reqs] or NULL.  NULL: the batch is
 *                     taken as already ordered decodes-first and the decodes
 *                     are its longest qualifying prefix.  Non-NULL: receives
 *                     the stable order that puts every decode first, and the
 *                     counts describe the batch in that order.
 *   counts          : host int32 [5] receives num_decodes, num_decode_tokens,
 *                     num_prefills, num_prefill_tokens, DQL (0 if no decode).
 *   Errors: INVALID_ARGUMENT for NULL query_start_loc/counts, num_reqs < 0,
 *   decode_threshold < 1, or a decreasing query_start_loc.
 */
int qsa_split_batch(const int32_t *query_start_loc, int32_t num_reqs, int32_t decode_threshold,
                    int32_t *order, int32_t *counts);

/* qsa_build_metadata -- per-token metadata on the device.
 *   For query token t in [0, num_tokens): its request r (the one with
 *   query_start_loc[r] <= t < query_start_loc[r+1]), its logical position
 *   pos = seq_lens[r] - query_len[r] + (t - query_start_loc[r]) and its
 *   visible block count max(0, min((pos+1)/cr, seq_lens[r]/cr)) (floor
 *   division).  Tokens at or past query_start_loc[num_reqs] are padding:
 *   request 0, position -1, 0 visible blocks.  Also comp_lens[r] =
 *   seq_lens[r]/cr, and -- when key_offsets is given -- the prefill key
 *   interval of each token over packed keys: row_k_start[t] =
 *   key_offsets[r], row_k_end[t] = key_offsets[r] + visible[t].
 *   Source: vLLM page qsa_cache.py (_logical_positions,
 *   _build_qsa_metadata_kernel); PR 54513 "Main changes".
 *   query_start_loc : device int32 [num_reqs+1];  seq_lens : device int32 [num_reqs]
 *   key_offsets     : device int32 [num_reqs] or NULL
 *   token_to_req    : device int32 [num_tokens] or NULL
 *   positions       : device int64 [num_tokens] or NULL
 *   visible         : device int32 [num_tokens] or NULL
 *   comp_lens       : device int32 [num_reqs] or NULL
 *   row_k_start, row_k_end : device int32 [num_tokens]; required iff key_offsets
 *   Errors: INVALID_ARGUMENT for negative counts, compress_ratio < 1, NULL
 *   required pointers.
 */
int qsa_build_metadata(const int32_t *query_start_loc, const int32_t *seq_lens,
                       int32_t num_reqs, int32_t num_tokens, int32_t compress_ratio,
                       const int32_t *key_offsets, int32_t *token_to_req, int64_t *positions,
                       int32_t *visible, int32_t *comp_lens, int32_t *row_k_start,
                       int32_t *row_k_end, void *stream);

/* qsa_decode_visible_blocks -- compressed lengths and per-row visible
 * blocks of a uniform decode batch (device).
 *   Source: MATE "QSA (Qwen Sparse Attention)", sections "MQA score" and
 *   "Entrypoints" (decode scores over compressed context lengths); vLLM
 *   qsa_cache.py (_logical_positions, _build_qsa_metadata_kernel) for the
 *   positions and the visibility rule, with 4 tokens per compressed block.
 *   Every request is a decode of dql query tokens, the last dql tokens of its
 *   context: row r*dql + j sits at position pos = seq_lens[r] - dql + j and
 *   sees max(0, min((pos+1)/4, seq_lens[r]/4)) blocks (floor division);
 *   comp_lens[r] = seq_lens[r]/4.  The same values qsa_build_metadata gives
 *   for query_start_loc = 0, dql, 2*dql, ... (one kernel).
 *   seq_lens      : device int32 [num_reqs]
 *   comp_lens_out : device int32 [num_reqs] or NULL
 *   visible_out   : device int32 [num_reqs*dql] or NULL
 *   Errors: INVALID_ARGUMENT for num_reqs < 0, dql outside [1, 16] or a NULL
 *   seq_lens with requests to read.
 */
int qsa_decode_visible_blocks(const int32_t *seq_lens, int32_t num_reqs, int32_t dql,
                              int32_t *comp_lens_out, int32_t *visible_out, void *stream);

/* ------------------------------------------------------------------------
 * qsa_build_cache_metadata -- where each token's compressed key goes, and the
 * work items of the compressed-cache writer.
 *   Source: vLLM qsa_cache.py, compressed_qsa_slot_mapping and the slot
 *   mapping (compress_ratio != 1) and k_work_metadata parts of
 *   _build_qsa_metadata_kernel.
 *
 *   query_start_loc, seq_lens, num_reqs, num_tokens, compress_ratio: as
 *     qsa_build_metadata (positions pos = seq_len - query_len + (t - start)).
 *   block_table : device int32 [num_reqs][block_table_cols], row stride
 *     block_table_stride: the physical block of each logical block of
 *     storage_block_size compressed rows (-1 = none).
 *   common_slot_mapping : device int64 [num_tokens] (the main cache's slots)
 *     or NULL; a token whose entry is negative writes no compressed key.
 *   slot_mapping : device int64 [num_tokens] out, or NULL.  Token t writes
 *     the compressed key of its group when pos >= 0 and (pos+1) %
 *     compress_ratio == 0: cp = pos / compress_ratio, slot = block_table[r]
 *     [cp / storage_block_size] * storage_block_size + cp % storage_block_size.
 *     -1 when no group closes, the logical block is past the table, the
 *     entry is negative, the main-cache slot is negative, or t is padding.
 *   k_work : device int32 [max_num_work][2] out, or NULL.  A request with
 *     query tokens owns max(seq_len/cr - (seq_len - query_len)/cr, 1) items
 *     (floor division), numbered request by request; item w = (request,
 *     index within the request); items past the last are (-1, -1).
 *   Errors: INVALID_ARGUMENT for negative counts, compress_ratio or
 *   storage_block_size < 1, a short block_table_stride or a NULL pointer that
 *   has work to feed; UNSUPPORTED for work items over more than 8,192
 *   requests.  Two kernels (slots, work items) run on `stream`.
 */
int qsa_build_cache_metadata(const int32_t *query_start_loc, const int32_t *seq_lens,
                             int32_t num_reqs, int32_t num_tokens, int32_t compress_ratio,
                             const int32_t *block_table, int64_t block_table_stride,
                             int32_t block_table_cols, int32_t storage_block_size,
                             const int64_t *common_slot_mapping, int64_t *slot_mapping,
                             int32_t *k_work, int32_t max_num_work, void *stream);

/* ------------------------------------------------------------------------
 * Cache updates upstream of the scores: the raw-key ring (the compressor's
 * state) and the compressed-key cache.
 *
 * qsa_build_ring_slots -- the raw-key ring row each query token writes.
 *   Source: vLLM qsa_cache.py, the circular branch of
 *   _build_qsa_metadata_kernel and circular_qsa_slot_mapping; the ring's
 *   capacity in QSAKeyStateCache (compress_ratio plus the speculative
 *   tokens, rounded up to whole groups).
 *   Request r owns one ring of ring_size rows in block block_table[r][0];
 *   block 0 is the null block of dummy and padding requests and is never
 *   written.  A query token at logical position pos = seq_len - query_len +
 *   (t - query_start) >= 0 that is one of the last ring_size query tokens of
 *   its request writes slot block * ring_size + pos % ring_size; every other
 *   token (and padding past query_start_loc[num_reqs], and every token when
 *   the table has no columns) gets -1.
 *   query_start_loc : device int32 [num_reqs+1];  seq_lens : device int32 [num_reqs]
 *   block_table     : device int32 [num_reqs][block_table_cols], row stride
 *                     block_table_stride (only column 0 is read)
 *   slot_mapping    : device int64 [num_tokens] out
 *   Errors: INVALID_ARGUMENT for negative counts, ring_size < 1, a short
 *   block_table_stride or a NULL pointer that has work to feed.  One kernel.
 */
int qsa_build_ring_slots(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                         int32_t num_tokens, const int32_t *block_table, int64_t block_table_stride,
                         int32_t block_table_cols, int32_t ring_size, int64_t *slot_mapping,
                         void *stream);

/* qsa_write_keys -- key rows written to cache rows at given slots.
 *   Source: vLLM qsa_cache.py, QSACompressedKeyCache (one normed key per
 *   complete group, at the slots of compressed_qsa_slot_mapping /
 *   qsa_build_cache_metadata) and QSAKeyStateCache (raw bf16 keys,
 *   optionally followed by exact int64 MRoPE positions, at the ring slots);
 *   qsa_prepare's _to_dst_dtype for an fp8 cache (round to bf16, divide by
 *   the cache scale, convert to e4m3).  The keys themselves (the raw keys,
 *   or the compressed ones, whose 4 -> 1 compression is not on the pages)
 *   are the caller's.
 *   keys       : device bf16 [num_tokens][key_stride] (128 used per row),
 *                8-byte aligned, key_stride a multiple of 4.
 *   slots      : device int64 [num_tokens]: row t goes to cache row slots[t]
 *                when 0 <= slots[t] < num_slots; other tokens write nothing.
 *                Two tokens naming one slot race (unspecified winner).
 *   cache      : device rows of row_stride elements of cache_dtype, 8-byte
 *                aligned (a paged cache [pages][page_size][1][W] is
 *                pages * page_size rows of stride W); rows no token names
 *                are left as they are.
 *   cache_dtype: QSA_DTYPE_BF16 (the bits as they are) or
 *                QSA_DTYPE_FP8_E4M3 (each value divided by `scale` in fp32
 *                and rounded to the nearest e4m3 code, ties to even,
 *                saturating at 448; NaN gives 0x7F).
 *   row_stride : elements per cache row, a multiple of 4, at least 128
 *                (140 with positions).
 *   positions  : NULL, or (bf16 caches) device int64 [3 axes][num_tokens] at
 *                element a * pos_stride_axis + t * pos_stride_token: written
 *                after the key as three little-endian int64 from element 128
 *                of the row (QSAKeyStateCache's rope_position_offset), 8-byte
 *                aligned.
 *   Errors: UNSUPPORTED for another cache format or positions with an e4m3
 *   cache; INVALID_ARGUMENT for negative sizes, a short row or key stride,
 *   a bad scale (e4m3) or a NULL pointer that has work to feed; LAYOUT for
 *   misaligned pointers or strides.  One kernel.
 */
int qsa_write_keys(const void *keys, int64_t key_stride, int32_t num_tokens, const int64_t *slots,
                   void *cache, int32_t cache_dtype, int64_t row_stride, int64_t num_slots, float scale,
                   const int64_t *positions, int64_t pos_stride_axis, int64_t pos_stride_token,
                   void *stream);

/* ------------------------------------------------------------------------
 * qsa_gather_keys -- paged compressed keys gathered into contiguous rows,
 * so that qsa_mqa_prefill can score a chunk straight from the cache.
 *   Source: MATE "QSA (Qwen Sparse Attention)", section "MQA score" (paged
 *   keys [pages, page_size, 1, dim], page table with -1 entries; packed
 *   prefill keys with per-row intervals).
 *
 *   k_cache    : device [num_pages][page_size][1][128] elements of k_dtype
 *                (QSA_DTYPE_BF16, QSA_DTYPE_FP16: 256 bytes per key;
 *                QSA_DTYPE_FP8_E4M3: 128), contiguous, 16-byte aligned.
 *                The elements are copied as they are.
 *   page_table : device int32 [num_reqs][page_table_cols], row stride
 *                page_table_stride.
 *   key_counts, key_offsets : device int32 [num_reqs]: request r's keys
 *                0 .. key_counts[r]-1 (clamped to [0, max_keys]) go to rows
 *                key_offsets[r] .. of k_out, in order.
 *   max_keys   : host bound on key_counts (sizes the launch).
 *   out_dtype  : k_dtype (rows copied as they are), or for e4m3 keys
 *                QSA_DTYPE_BF16 / QSA_DTYPE_FP16: the codes' values widened
 *                exactly (no scale).  qsa_mqa_prefill over bf16 keys widened
 *                from an e4m3 cache, with scale * k_scale as its multiplier,
 *                then scores the cache as qsa_mqa_decode_typed does.
 *   k_out      : device [k_out_rows][k_out_stride] elements of out_dtype,
 *                16-byte aligned, row stride k_out_stride >= 128 with
 *                16-byte rows.  Key c of request r is row c % page_size of
 *                page page_table[r][c / page_size]; a missing page (id < 0,
 *                >= num_pages, or a slot past the table) gives a zero row.
 *                Rows outside [0, k_out_rows) are skipped; rows no request
 *                covers are left untouched.
 *   Errors: UNSUPPORTED for another k_dtype or out_dtype; INVALID_ARGUMENT for negative
 *   sizes, page_size outside [1, 1<<20], max_keys above 2^30, a short
 *   stride or a NULL pointer that has work to feed; LAYOUT for misaligned
 *   k_cache, k_out or rows.
 */
int qsa_gather_keys(const void *k_cache, int32_t k_dtype, int64_t num_pages, int32_t page_size,
                    const int32_t *page_table, int64_t page_table_stride, int32_t page_table_cols,
                    const int32_t *key_counts, const int32_t *key_offsets, int32_t num_reqs,
                    int32_t max_keys, void *k_out, int32_t out_dtype, int64_t k_out_stride,
                    int64_t k_out_rows, void *stream);

/* ------------------------------------------------------------------------
 * qsa_mqa_decode -- decode scores over the paged compressed-key cache.
 *   Source: MATE "QSA (Qwen Sparse Attention)", section "MQA score" (paged
 *   keys [pages, page_size, 1, dim], page table with -1 for unused entries,
 *   compressed context lengths, missing or out-of-range pages score -inf,
 *   broadcast Q accepted); visibility per row from vLLM qsa_cache.py.
 *
 *   q          : device bf16 [num_reqs][dql][4][128]; element strides
 *                q_stride_req, q_stride_row, q_stride_head (any value,
 *                including 0 for broadcast); unit feature stride.  No
 *                alignment rule: aligned Q uses 16-byte loads, other Q
 *                element loads.
 *   k_cache    : device bf16 [num_pages][page_size][1][128], contiguous,
 *                16-byte aligned.  Row p*page_size + i holds compressed key
 *                i of page p.
 *   page_table : device int32 [num_reqs][page_table_cols], row stride
 *                page_table_stride.  Entry -1 (or any id outside
 *                [0, num_pages)) = no page: those blocks score -inf.
 *   comp_lens  : device int32 [num_reqs]: complete 4-token blocks of each
 *                request (seq_len / 4).
 *   visible    : device int32 [num_reqs*dql] or NULL: blocks visible to row
 *                r*dql+j; values are clamped to [0, comp_lens[r]].  NULL:
 *                every row sees comp_lens[r] blocks.
 *   scale      : finite, > 0; multiplies the head sum (1/sqrt(128) normally).
 *   out        : device fp32 [num_reqs*dql][out_cols], row stride out_stride
 *                (>= out_cols), 4-byte aligned.  Column c = block c of the
 *                request.  Every cell is written: the score, or -inf when
 *                c >= visible, the page is missing, or c >= page_table_cols
 *                * page_size.
 *   Errors: UNSUPPORTED unless (num_heads, head_dim) == (4, 128);
 *   INVALID_ARGUMENT for negative sizes, dql outside [1, 16], page_size
 *   outside [1, 1<<20], out_stride < out_cols, a bad scale or a NULL pointer
 *   that has work to feed; LAYOUT for a misaligned k_cache or out.
 */
int qsa_mqa_decode(const void *q, int64_t q_stride_req, int64_t q_stride_row,
                   int64_t q_stride_head, const void *k_cache, int64_t num_pages,
                   int32_t page_size, const int32_t *page_table, int64_t page_table_stride,
                   int32_t page_table_cols, const int32_t *comp_lens, const int32_t *visible,
                   int32_t num_reqs, int32_t dql, int32_t num_heads, int32_t head_dim,
                   float scale, float *out, int64_t out_stride, int32_t out_cols,
                   void *stream);

/* ------------------------------------------------------------------------
 * qsa_mqa_prefill -- prefill scores over packed queries and shared keys.
 *   Source: MATE "QSA (Qwen Sparse Attention)", section "MQA score" (packed
 *   queries, shared keys, per-row key intervals; the vector-load layout
 *   rules for query and keys).
 *
 *   q          : device bf16 [num_rows][4][128], element strides
 *                q_stride_row, q_stride_head; unit feature stride.
 *   k          : device bf16 [num_keys][128], element row stride k_stride;
 *                unit feature stride.
 *   Layout rule (q and k): base 16-byte aligned; every axis with more than
 *   one element has a positive stride that is a multiple of 8 elements.
 *   row_k_start, row_k_end : device int32 [num_rows].  Column c of row t
 *                holds key row_k_start[t] + c; the cell is a score when that
 *                key lies in [0, num_keys) and below row_k_end[t], else -inf
 *                (an empty or reversed interval masks the whole row).
 *   out        : device fp32 [num_rows][out_cols], row stride out_stride
 *                (>= out_cols), 4-byte aligned; every cell is written.
 *   Errors: as qsa_mqa_decode, plus LAYOUT when q or k breaks the layout rule,
 *   and UNSUPPORTED for k_stride above 4,194,304 elements (the kernel's key
 *   offsets are 32-bit).
 */
int qsa_mqa_prefill(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                    int64_t k_stride, int64_t num_keys, const int32_t *row_k_start,
                    const int32_t *row_k_end, int32_t num_rows, int32_t num_heads,
                    int32_t head_dim, float scale, float *out, int64_t out_stride,
                    int32_t out_cols, void *stream);

/* ------------------------------------------------------------------------
 * qsa_mqa_decode_typed -- qsa_mqa_decode with typed queries and keys.
 *   Source: as qsa_mqa_decode; formats per enum qsa_dtype above.
 *
 *   q_dtype : QSA_DTYPE_BF16 or QSA_DTYPE_FP16 (2-byte elements; strides in
 *             elements as for qsa_mqa_decode).
 *   k_dtype : q_dtype (a [num_pages][page_size][1][128] cache of 2-byte
 *             elements), or QSA_DTYPE_FP8_E4M3 (the same shape in 1-byte
 *             codes: 128 bytes per key).  k_cache is 16-byte aligned.
 *   k_scale : fp8 keys only: the cache scale, finite and > 0; key element =
 *             e4m3 value * k_scale.  Ignored for 2-byte keys.
 *   The scores equal scale * k_scale * sum_h relu(q_h . code) for fp8 keys;
 *   scale * k_scale is formed once in fp32 and must be finite and > 0.
 *   Other arguments, output and errors as qsa_mqa_decode, plus UNSUPPORTED
 *   for other formats or 2-byte keys in a format other than the query's,
 *   and INVALID_ARGUMENT for a bad k_scale.
 */
int qsa_mqa_decode_typed(const void *q, int32_t q_dtype, int64_t q_stride_req,
                         int64_t q_stride_row, int64_t q_stride_head, const void *k_cache,
                         int32_t k_dtype, float k_scale, int64_t num_pages, int32_t page_size,
                         const int32_t *page_table, int64_t page_table_stride,
                         int32_t page_table_cols, const int32_t *comp_lens,
                         const int32_t *visible, int32_t num_reqs, int32_t dql,
                         int32_t num_heads, int32_t head_dim, float scale, float *out,
                         int64_t out_stride, int32_t out_cols, void *stream);

/* ------------------------------------------------------------------------
 * Planned decode: a task table built once per step, read by every decode
 * launch of that step (one per layer that runs the indexer).
 *   Source: as qsa_mqa_decode.  The vLLM metadata builder (qsa_cache.py,
 *   QSAMetadataBuilder.build and _build_qsa_metadata_kernel) likewise builds
 *   the step's indexer metadata once, from the compressed lengths and block
 *   tables, for all layers.  The scores are those of qsa_mqa_decode, bit for
 *   bit; the table only tells each wavefront its (request, 64-key span), the
 *   span's physical page and the request's compressed length, so that a
 *   wavefront starts its key loads after one table read.
 *
 * qsa_decode_plan_bytes -- size of the task table for num_reqs requests and
 *   out_cols output columns: num_reqs * ceil(out_cols / 64) entries of 16
 *   bytes.  bytes: host int64 out.  Errors: INVALID_ARGUMENT for a NULL
 *   bytes or negative sizes.
 *
 * qsa_build_decode_plan -- fill the task table (one kernel on `stream`).
 *   comp_lens, page_table, page_table_stride, page_table_cols, num_pages,
 *   page_size, num_reqs, out_cols: as qsa_mqa_decode.
 *   plan       : device buffer of plan_bytes >= qsa_decode_plan_bytes(...)
 *                bytes, 16-byte aligned, caller-owned.  Entry {r, span,
 *                page, comp}: the spans holding keys, request by request,
 *                then the spans past each request's keys in groups of 4
 *                (span | 1<<31), then unused entries (r = -1).  page is the
 *                span's physical page when page_size is a multiple of 64,
 *                else -1 (the decode then reads the page table per key).
 *   The table depends on comp_lens and the page table: build it again when
 *   either changes (normally once per step).
 *   Errors: INVALID_ARGUMENT for negative sizes, page_size outside
 *   [1, 1<<20], a short page_table_stride, a NULL pointer that has work to
 *   feed or a short plan; LAYOUT for a misaligned plan; UNSUPPORTED for more
 *   than 4,096 requests.
 *
 * qsa_mqa_decode_planned -- qsa_mqa_decode_typed driven by a task table.
 *   plan, plan_bytes : a table from qsa_build_decode_plan for the same
 *                num_reqs, out_cols, page_size, page table and compressed
 *                lengths (a table for other arguments gives wrong scores but
 *                never reads or writes outside the given buffers: entries
 *                out of range are ignored, pages out of range read as
 *                missing).
 *   q, q_dtype, strides, k_cache, k_dtype, k_scale, num_pages, page_size,
 *   page_table (used per key when page_size is not a multiple of 64; may be
 *   NULL otherwise), visible, num_reqs, dql, num_heads, head_dim, scale,
 *   out, out_stride, out_cols: as qsa_mqa_decode_typed.  The compressed
 *   lengths come from the table.
 *   Errors: as qsa_mqa_decode_typed, plus INVALID_ARGUMENT for a NULL plan
 *   or plan_bytes below the table's size, and LAYOUT for a misaligned plan.
 */
/* qsa_mqa_decode_static_plan -- the planned decode with the task table in
 * the library's own device memory, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It calls no allocating routine: the table lives in a
 * 4 MiB array (262,144 entries) that each device holds from the library's
 * first use on it until the process ends.
 *   Arguments, output and errors as qsa_mqa_decode_typed (comp_lens and
 *   the page table are read to build the table).  The call enqueues two
 *   kernels on stream: qsa_build_decode_plan into the library's table, then
 *   qsa_mqa_decode_planned from it; the scores equal qsa_mqa_decode_planned's
 *   with a table built by qsa_build_decode_plan, bit for bit.
 *   Limits: num_reqs * ceil(out_cols / 64) <= 262,144 and num_reqs <=
 *   4,096, else UNSUPPORTED (no launch).  DEVICE if the table's address
 *   cannot be obtained.
 *   Every call on one device shares that device's table: calls that overlap
 *   on one GPU (other streams, other threads) race and give wrong scores;
 *   calls in one stream are ordered and safe.  The table keeps the last
 *   call's contents, and nothing needs clearing: each call writes every
 *   entry it reads.
 */
int qsa_mqa_decode_static_plan(const void *q, int32_t q_dtype, int64_t q_stride_req,
                               int64_t q_stride_row, int64_t q_stride_head, const void *k_cache,
                               int32_t k_dtype, float k_scale, int64_t num_pages, int32_t page_size,
                               const int32_t *page_table, int64_t page_table_stride,
                               int32_t page_table_cols, const int32_t *comp_lens,
                               const int32_t *visible, int32_t num_reqs, int32_t dql,
                               int32_t num_heads, int32_t head_dim, float scale, float *out,
                               int64_t out_stride, int32_t out_cols, void *stream);

int qsa_decode_plan_bytes(int32_t num_reqs, int32_t out_cols, int64_t *bytes);

int qsa_build_decode_plan(const int32_t *comp_lens, const int32_t *page_table,
                          int64_t page_table_stride, int32_t page_table_cols, int64_t num_pages,
                          int32_t page_size, int32_t num_reqs, int32_t out_cols, void *plan,
                          int64_t plan_bytes, void *stream);

int qsa_mqa_decode_planned(const void *plan, int64_t plan_bytes, const void *q, int32_t q_dtype,
                           int64_t q_stride_req, int64_t q_stride_row, int64_t q_stride_head,
                           const void *k_cache, int32_t k_dtype, float k_scale, int64_t num_pages,
                           int32_t page_size, const int32_t *page_table,
                           int64_t page_table_stride, int32_t page_table_cols,
                           const int32_t *visible, int32_t num_reqs, int32_t dql,
                           int32_t num_heads, int32_t head_dim, float scale, float *out,
                           int64_t out_stride, int32_t out_cols, void *stream);

/* ------------------------------------------------------------------------
 * qsa_mqa_prefill_typed -- qsa_mqa_prefill with BF16 or FP16 queries and
 * keys (dtype QSA_DTYPE_BF16 or QSA_DTYPE_FP16; both share it).
 *   Source: MATE "QSA (Qwen Sparse Attention)", section "MQA score" (BF16
 *   or FP16 query and key; packed queries, per-row key intervals).
 *   Arguments, layout rule, output and errors as qsa_mqa_prefill (strides in
 *   elements), plus UNSUPPORTED for any other dtype.
 */
int qsa_mqa_prefill_typed(const void *q, int64_t q_stride_row, int64_t q_stride_head,
                          const void *k, int64_t k_stride, int64_t num_keys, int32_t dtype,
                          const int32_t *row_k_start, const int32_t *row_k_end,
                          int32_t num_rows, int32_t num_heads, int32_t head_dim, float scale,
                          float *out, int64_t out_stride, int32_t out_cols, void *stream);

/* ------------------------------------------------------------------------
 * qsa_topk_blocks -- per-row top-k block indices.
 *   Source: MATE "QSA (Qwen Sparse Attention)": the caller keeps the
 *   top-scoring blocks (intro) as request-local int32 indices padded with -1
 *   (section "Core Attention").  Rule used here: candidates are the cells
 *   greater than -inf (NaN is never a candidate); the k largest are kept,
 *   equal values (with -0 equal to +0) going to the lower column; the picks
 *   are written in ascending column order followed by -1 up to k.
 *
 *   logits  : device fp32 [num_rows][num_cols], row stride logits_stride
 *             (>= num_cols), 4-byte aligned.
 *   out_idx : device int32 [num_rows][k], row stride out_stride (>= k).
 *   Errors: INVALID_ARGUMENT for negative sizes, k < 1, k > 1<<20, strides
 *   below the row width or NULL pointers that have work to feed.
 */
int qsa_topk_blocks(const float *logits, int64_t logits_stride, int32_t num_rows,
                    int32_t num_cols, int32_t k, int32_t *out_idx, int64_t out_stride,
                    void *stream);

/* ------------------------------------------------------------------------
 * qsa_mqa_prefill_topk -- prefill scores and per-row top-k in one call,
 *   without writing the fp32 score matrix.
 *   Source: the two operations above (MATE "QSA (Qwen Sparse Attention)",
 *   sections "MQA score" and "Core Attention"), composed; keeping the
 *   logits workspace out of the prefill step is the motivation in the vLLM
 *   pull request "[Qwen3.8-Flash-Next] Separate prefill and decode paths
 *   for QSA indexer", section "Main changes" (chunked prefill bounds a
 *   512 MiB logits workspace).
 *   Result: out_idx equals qsa_topk_blocks(k = topk) applied to the
 *   out_cols-wide output of qsa_mqa_prefill with the same arguments, bit for
 *   bit (the same scores; ties to the lower column; ascending; -1 padded).
 *   q, k, row_k_start, row_k_end, num_rows, num_heads, head_dim, scale,
 *   out_cols : as qsa_mqa_prefill; k_stride at most 16,384 elements.
 *   topk       : 1 .. 2048.
 *   out_idx    : device int32 [num_rows][topk], row stride out_stride (>= topk).
 *   workspace  : device memory of at least qsa_prefill_topk_workspace_bytes
 *                bytes, 256-byte aligned, owned by the caller; its contents
 *                on entry do not matter and are clobbered.
 *   Rows of 1 .. 32,768 columns: the prefill pass stores the top 16 bits of
 *   each cell's order key (2 bytes per cell instead of the 4-byte score), a
 *   select picks on them and rescores, with the prefill's own MFMA sequence
 *   (hence the same bits), only the cells whose prefix ties that of the k-th
 *   largest key; rows it cannot finish (more than 4,096 keys at or above its
 *   floor, or more than 64 such ties) are rescored whole by a fallback.
 *   Workspace about num_rows * 2 * round_up(out_cols, 64) + 256 *
 *   round_up(out_cols, 64) bytes (half the fp32 score matrix).  Three
 *   kernels: the key pass, the select, the fallback (which returns at once
 *   when no row was left to it).
 *   Wider rows (and out_cols 0): a group-maximum pass over the scores, the
 *   per-row floor over the group maxima, a candidate pass over the scores
 *   and the final select (four kernels); workspace about
 *   num_rows * (8 * min(8 * (topk - 1) + chunks * topk, out_cols)
 *   + out_cols / 2) bytes, chunks being the column chunks per row, of which
 *   a call touches a few percent.
 *   The size depends on the sizes and the device's CU count only.  With
 *   timing events armed the start event marks the first kernel's begin and
 *   the stop event the last kernel's end.
 *   Errors: as qsa_mqa_prefill (UNSUPPORTED also, for rows wider than
 *   32,768 columns, for k_stride > 16,384 and for rows whose per-workgroup
 *   workspace offsets would pass 2^31 bytes),
 *   INVALID_ARGUMENT for topk outside [1, 2048], out_stride < topk, a NULL
 *   out_idx or workspace, or a workspace below the size needed; LAYOUT for a
 *   misaligned out_idx or workspace.
 */
int qsa_mqa_prefill_topk(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                         int64_t k_stride, int64_t num_keys, const int32_t *row_k_start,
                         const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                         float scale, int32_t out_cols, int32_t topk, int32_t *out_idx, int64_t out_stride,
                         void *workspace, int64_t workspace_bytes, void *stream);

/* qsa_mqa_prefill_topk_typed -- qsa_mqa_prefill_topk with BF16 or FP16
 *   queries and keys (dtype QSA_DTYPE_BF16 or QSA_DTYPE_FP16; both share it).
 *   Source: MATE "QSA (Qwen Sparse Attention)", section "MQA score" (BF16 or
 *   FP16 query and key), composed with the top-k as above.
 *   Result: equal to qsa_topk_blocks applied to the output of
 *   qsa_mqa_prefill_typed with the same arguments, bit for bit (fp16 rows
 *   are scored and rescored with the fp16 product).  Workspace, arguments
 *   and errors as qsa_mqa_prefill_topk, plus UNSUPPORTED for any other
 *   dtype and for FP16 rows wider than 32,768 columns.
 */
int qsa_mqa_prefill_topk_typed(const void *q, int64_t q_stride_row, int64_t q_stride_head, const void *k,
                               int64_t k_stride, int64_t num_keys, int32_t dtype, const int32_t *row_k_start,
                               const int32_t *row_k_end, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                               float scale, int32_t out_cols, int32_t topk, int32_t *out_idx, int64_t out_stride,
                               void *workspace, int64_t workspace_bytes, void *stream);

/* qsa_prefill_topk_workspace_bytes -- workspace size qsa_mqa_prefill_topk
 *   (and qsa_mqa_prefill_topk_typed)
 *   needs for these sizes on the current device (host only; the column
 *   split depends on the device's compute-unit count).
 *   Errors: INVALID_ARGUMENT for a NULL bytes, negative sizes or topk
 *   outside [1, 2048].
 */
int qsa_prefill_topk_workspace_bytes(int32_t num_rows, int32_t out_cols, int32_t topk, int64_t *bytes);

/* ------------------------------------------------------------------------
 * qsa_prepare_q -- the indexer's query heads normalized and rotated.
 *   Source: vLLM "vllm.models.qwen4_exp.amd.ops.qsa_prepare", functions
 *   _norm_rope (Gemma RMSNorm with weight + 1, then NeoX rotary embedding of
 *   the first 64 features, optionally interleaved MRoPE), _store_rotated and
 *   _to_dst_dtype (round to bf16; for an fp8 destination divide by the scale
 *   and convert); supports_fused_pre_indexer (head dim 128, rotary dim 64,
 *   NeoX style, MRoPE section summing to 32).  The compression of the keys
 *   that the same page's kernel performs is not covered.
 *
 *   For head x of a token (128 bf16 features), in fp32:
 *     rrms = 1/sqrt(sum(x^2)/128 + eps),  y_d = (x_d * rrms) * (w_d + 1),
 *   y rounded to cos_sin_dtype; then for pair j < 32, in cos_sin_dtype with
 *   one rounding per operation and no fused multiply-add,
 *     out_j = y_j c_j - y_{j+32} s_j,  out_{j+32} = y_{j+32} c_j + y_j s_j;
 *   features 64..127 are y.  The sum of squares is the fp32 rounding of the
 *   exact sum and rrms the fp32 rounding of 1/sqrt (the page leaves the
 *   order and the reciprocal square root's accuracy open).
 *
 *   q          : device bf16 [num_tokens][num_heads][128]; token stride
 *                q_stride_token elements (>= num_heads*128 when
 *                num_tokens > 1, a multiple of 8), heads contiguous, 16-byte
 *                aligned.
 *   positions  : device int64; token t's position on axis a (0 temporal,
 *                1 height, 2 width) at positions[a*pos_stride_axis +
 *                t*pos_stride_token].  Without MRoPE only axis 0 is read.
 *   cos_sin    : device [cos_sin_rows][64] of cos_sin_dtype (QSA_DTYPE_BF16
 *                or QSA_DTYPE_FP32), contiguous, 16-byte aligned (may be NULL
 *                when cos_sin_rows is 0): row p holds cos of pairs 0..31,
 *                then their sin; only rows that positions name are read.  A position outside
 *                [0, cos_sin_rows) is the caller's error: the pairs that use
 *                it come out NaN (the other features are unaffected).
 *   norm_weight: device [128] of weight_dtype (QSA_DTYPE_BF16 or
 *                QSA_DTYPE_FP32), 16-byte aligned; the gain is weight + 1.
 *   eps        : finite, added to the mean square.
 *   mrope_section : host int32[3] (t, h, w), each >= 0, summing to 32, or
 *                NULL for plain rotary.  Pair j reads the height position
 *                when j % 3 == 1 and j < 3h, the width position when
 *                j % 3 == 2 and j < 3w, else the temporal one; every axis
 *                reads the same table.  (The page adds the three masked
 *                reads to zero, so a -0 entry reads as +0; so does this.)
 *   q_out      : device [num_tokens][num_heads][128] of out_dtype at element
 *                strides out_stride_token, out_stride_head (multiples of 8),
 *                unit feature stride, 16-byte (bf16) or 8-byte (e4m3)
 *                aligned; must not overlap q.  QSA_DTYPE_BF16: the result
 *                rounded to bf16 (ties to even).  QSA_DTYPE_FP8_E4M3: that
 *                bf16 value divided by out_scale (finite, > 0) in fp32, then
 *                the nearest finite e4m3 value (ties to the even code, so
 *                magnitudes above 448 give 448; NaN gives 0x7F).
 *   Errors: INVALID_ARGUMENT for negative counts, num_heads outside
 *   [1, 1024], num_tokens * num_heads >= 2^31, a table of 2^31 bytes or
 *   more, a bad section, eps or out_scale, a short q stride or a NULL
 *   pointer that has work to feed; UNSUPPORTED for other dtypes; LAYOUT for
 *   misaligned pointers or strides.  One kernel runs on `stream`.
 */
int qsa_prepare_q(const void *q, int64_t q_stride_token, int32_t num_tokens, int32_t num_heads,
                  const int64_t *positions, int64_t pos_stride_axis, int64_t pos_stride_token,
                  const void *cos_sin, int32_t cos_sin_dtype, int64_t cos_sin_rows, const void *norm_weight,
                  int32_t weight_dtype, float eps, const int32_t *mrope_section, void *q_out,
                  int32_t out_dtype, float out_scale, int64_t out_stride_token, int64_t out_stride_head,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
