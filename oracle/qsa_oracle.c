/*
 * Plain CPU oracle for the QSA lightweight MQA indexer (block scoring).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library; it is written from the definitions on the pages, slowly and
 * plainly, so that a reader can check every line against them.
 *
 * Arithmetic: bf16 inputs are widened exactly to double, every dot product
 * and the head sum are accumulated in double, and the scaled result is
 * rounded once to fp32.
 *
 * Sources (page title, section):
 *   [MATE-QSA]  "QSA (Qwen Sparse Attention)" (MATE API docs), intro and
 *               section "MQA score": score = sum over the 4 query heads of
 *               ReLU(q_h . k), times 1/sqrt(128); incomplete/future blocks
 *               masked; paged keys [pages, page_size, 1, dim] with a page
 *               table whose unused entries may be -1 and whose missing or
 *               out-of-range pages score -inf; packed prefill queries with
 *               per-row key intervals; "scale" is a multiplier.
 *               Section "Core Attention": selected block indices are
 *               request-local int32, padded with -1, at most 512 per row.
 *   [QSA-CACHE] "vLLM/vllm/models/qwen4_exp/common/qsa_cache.py",
 *               functions _logical_positions, _build_qsa_metadata_kernel,
 *               _build_qsa_metadata_torch and QSAMetadataBuilder.build:
 *               logical position of a query token, visible_blocks =
 *               max(0, min((pos+1)//cr, seq_len//cr)), decode/prefill split
 *               with a uniform decode query length.
 *   [PR-54513]  "[Qwen3.8-Flash-Next] Separate prefill and decode paths for
 *               QSA indexer" (vLLM PR 54513), section "Main changes":
 *               visible_blocks = (logical_position + 1) // compress_ratio
 *               moves into the per-step metadata.
 *   [QSA-CACHE] QSAStateBackend: the compressed indexer cache may hold fp8
 *               e4m3 entries.
 *   [QSA-PREP]  "vllm/models/qwen4_exp/amd/ops/qsa_prepare.py", _to_dst_dtype:
 *               a value bound for an fp8 cache is rounded to bf16, divided
 *               by the cache's scale, then converted to fp8.
 *   [MATE-QSA]  "MQA score": query and compressed key are BF16 or FP16.
 *   [QSA-PREP]  _norm_rope: Gemma RMSNorm (weight + 1) in fp32, the result
 *               rounded to the cos/sin table's type, then NeoX rotation of
 *               the first half of the rotary slice with per-axis (MRoPE)
 *               table rows; _store_rotated: the first 64 features are the
 *               rotated ones; _to_dst_dtype: round to bf16 (then / scale
 *               and fp8 for an fp8 destination).  supports_fused_pre_indexer:
 *               head dim 128, rotary dim 64, NeoX style, interleaved MRoPE
 *               whose section sums to 32.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - scale multiplies the head sum (equal to scaling before ReLU for
 *     scale > 0);  ReLU(x) = x > 0 ? x : +0.0, so unmasked cells are >= +0.
 *   - decode row (r, j) sees min(max(visible[r*dql+j], 0), comp_len[r])
 *     blocks; with no visible array it sees comp_len[r].
 *   - prefill column c of row t holds key row_k_start[t] + c; it is valid
 *     iff that key lies in [0, num_keys) and below row_k_end[t].
 *   - an fp8 key element stands for its e4m3 value times the cache's scale
 *     (the inverse of the division on the write side); the scale applies
 *     to fp8 keys only.  fp8 is the OCP e4m3 format (the "fp8_e4m3" cache
 *     dtype).  NaN codes are outside the contract.
 *   - top-k keeps the k largest cells that are > -inf (NaN excluded),
 *     breaks ties toward the lower column, compares with IEEE ordering
 *     (-0 == +0), emits the picks in ascending column order and pads -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QSA_ORACLE_HEADS 4
#define QSA_ORACLE_DIM 128

/* bf16 bit pattern -> double.  A bf16 value is the upper half of an IEEE
 * binary32 value, so the widening is exact. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16 bit pattern -> double: sign, 5-bit exponent with bias
 * 15, 10-bit fraction.  Exponent 0 holds zero and the subnormals (fraction
 * times 2^-24); exponent 31 holds infinities (fraction 0) and NaN.  Exact. */
static double fp16_bits_to_double(uint16_t bits)
{
    int sign = bits >> 15;
    int exponent = (bits >> 10) & 31;
    int fraction = bits & 1023;
    double v;
    if (exponent == 0)
        v = ldexp((double)fraction, -24);
    else if (exponent == 31)
        v = fraction ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fraction), exponent - 25);  /* 2^(e-15) * (1 + f/1024) */
    return sign ? -v : v;
}

/* OCP 8-bit floating point E4M3 bit pattern -> double: sign, 4-bit exponent
 * with bias 7, 3-bit fraction.  Exponent 0 holds zero and the subnormals
 * (fraction times 2^-9); S.1111.111 is NaN; there are no infinities (the
 * largest finite magnitude is 448).  Exact. */
static double e4m3_bits_to_double(uint8_t bits)
{
    int sign = bits >> 7;
    int exponent = (bits >> 3) & 15;
    int fraction = bits & 7;
    double v;
    if (exponent == 15 && fraction == 7)
        v = NAN;
    else if (exponent == 0)
        v = ldexp((double)fraction, -9);
    else
        v = ldexp((double)(8 + fraction), exponent - 10);  /* 2^(e-7) * (1 + f/8) */
    return sign ? -v : v;
}

/* Element formats of the typed entry points. */
#define ORACLE_BF16 0
#define ORACLE_FP16 1
#define ORACLE_FP8_E4M3 2
#define ORACLE_FP32 3

/* Element `index` of an array of `format` elements, widened exactly. */
static double element(const void *base, int64_t index, int format)
{
    if (format == ORACLE_FP8_E4M3) return e4m3_bits_to_double(((const uint8_t *)base)[index]);
    if (format == ORACLE_FP32) return (double)((const float *)base)[index];
    uint16_t bits = ((const uint16_t *)base)[index];
    return format == ORACLE_FP16 ? fp16_bits_to_double(bits) : bf16_bits_to_double(bits);
}

static float neg_inf(void) { return -INFINITY; }

/* Python-style floor division for the metadata formulas (C '/' truncates). */
static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
    return q;
}

/* One score cell [MATE-QSA, "MQA score"]:
 *   scale * sum_h max(0, sum_d q[h][d] * k[d]),
 * with query element q[q_off + h*q_stride_head + d] in q_format and key
 * element k[k_off + d] in k_format; an fp8 key element counts as its value
 * times k_scale.  Accumulated in double, rounded once to fp32. */
static float score_cell_typed(const void *q, int64_t q_off, int64_t q_stride_head, int q_format,
                              const void *k, int64_t k_off, int k_format, double k_scale,
                              float scale)
{
    double head_sum = 0.0;
    for (int h = 0; h < QSA_ORACLE_HEADS; ++h) {
        double dot = 0.0;
        for (int d = 0; d < QSA_ORACLE_DIM; ++d) {
            double kv = element(k, k_off + d, k_format);
            if (k_format == ORACLE_FP8_E4M3) kv *= k_scale;
            dot += element(q, q_off + h * q_stride_head + d, q_format) * kv;
        }
        head_sum += (dot > 0.0) ? dot : 0.0;
    }
    return (float)(head_sum * (double)scale);
}

/* ---------------------------------------------------------------------- */
/* Per-step metadata [QSA-CACHE _logical_positions / metadata kernels].     */

/* For every query token t in [0, num_tokens):
 *   request r = the one whose [qsl[r], qsl[r+1]) holds t (linear scan),
 *   pos = seq_len[r] - query_len[r] + (t - qsl[r]),
 *   visible = max(0, min(floor((pos+1)/cr), floor(seq_len[r]/cr))).
 * Tokens past qsl[num_reqs] are padding: request 0, position -1,
 * visible 0 (the padding rule of the metadata kernel). */
void oracle_token_metadata(const int32_t *query_start_loc, const int32_t *seq_lens,
                           int32_t num_reqs, int32_t num_tokens, int32_t compress_ratio,
                           int32_t *token_to_req, int64_t *positions, int32_t *visible)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int32_t req = -1;
        for (int32_t r = 0; r < num_reqs; ++r)
            if (query_start_loc[r] <= t && t < query_start_loc[r + 1]) { req = r; break; }
        if (req < 0) {
            if (token_to_req) token_to_req[t] = 0;
            if (positions) positions[t] = -1;
            if (visible) visible[t] = 0;
            continue;
        }
        int64_t query_len = (int64_t)query_start_loc[req + 1] - query_start_loc[req];
        int64_t pos = (int64_t)seq_lens[req] - query_len + (t - query_start_loc[req]);
        int64_t by_pos = floor_div(pos + 1, compress_ratio);
        int64_t by_len = floor_div(seq_lens[req], compress_ratio);
        int64_t v = by_pos < by_len ? by_pos : by_len;
        if (v < 0) v = 0;
        if (token_to_req) token_to_req[t] = req;
        if (positions) positions[t] = pos;
        if (visible) visible[t] = (int32_t)v;
    }
}

/* Number of complete compressed blocks per request: floor(seq_len / cr). */
void oracle_comp_lens(const int32_t *seq_lens, int32_t num_reqs, int32_t compress_ratio,
                      int32_t *comp_lens)
{
    for (int32_t r = 0; r < num_reqs; ++r)
        comp_lens[r] = (int32_t)floor_div(seq_lens[r], compress_ratio);
}

/* Prefill key intervals for packed keys: request r's compressed keys start
 * at key_offsets[r]; token t may read keys [start, start + visible[t]). */
void oracle_prefill_intervals(const int32_t *token_to_req, const int32_t *visible,
                              const int32_t *key_offsets, int32_t num_tokens,
                              int32_t *row_k_start, int32_t *row_k_end)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int32_t start = key_offsets[token_to_req[t]];
        row_k_start[t] = start;
        row_k_end[t] = start + visible[t];
    }
}

/* ---------------------------------------------------------------------- */
/* Typed inputs: BF16 or FP16 queries and keys [MATE-QSA "MQA score"], and   */
/* fp8 e4m3 keys scaled by the cache's scale [QSA-CACHE, QSA-PREP].          */

/* Decode over paged compressed keys [MATE-QSA "MQA score", paged form].
 * Rows [row_begin, row_end) of the [num_reqs*dql, out_cols] output; row
 * `row` is written at out + (row - row_begin) * out_stride.  Row index =
 * r*dql + j.  Query elements in q_format, key elements in k_format; strides
 * in elements; k_cache is [num_pages][page_size][1][128] elements,
 * contiguous. */
void oracle_decode_typed(const void *q, int q_format, int64_t q_stride_req, int64_t q_stride_row,
                         int64_t q_stride_head, const void *k_cache, int k_format, double k_scale,
                         int64_t num_pages, int32_t page_size, const int32_t *page_table,
                         int64_t page_table_stride, int32_t page_table_cols,
                         const int32_t *comp_lens, const int32_t *visible, int32_t num_reqs,
                         int32_t dql, float scale, float *out, int64_t out_stride,
                         int32_t out_cols, int32_t row_begin, int32_t row_end)
{
    (void)num_reqs;
    for (int32_t row = row_begin; row < row_end; ++row) {
        int32_t r = row / dql;
        int32_t j = row % dql;
        int64_t seen = visible ? (int64_t)visible[row] : (int64_t)comp_lens[r];
        if (seen > comp_lens[r]) seen = comp_lens[r];
        if (seen < 0) seen = 0;
        int64_t q_off = r * q_stride_req + j * q_stride_row;
        for (int32_t c = 0; c < out_cols; ++c) {
            float value = neg_inf();
            if (c < seen) {
                int64_t slot = c / page_size;
                if (slot < page_table_cols) {
                    int64_t page = page_table[r * page_table_stride + slot];
                    if (page >= 0 && page < num_pages) {
                        int64_t k_off = (page * page_size + (c % page_size)) * QSA_ORACLE_DIM;
                        value = score_cell_typed(q, q_off, q_stride_head, q_format, k_cache, k_off,
                                                 k_format, k_scale, scale);
                    }
                }
            }
            out[(int64_t)(row - row_begin) * out_stride + c] = value;
        }
    }
}

/* Prefill over packed queries and shared keys [MATE-QSA "MQA score"].
 * Rows [row_begin, row_end) of the [num_rows, out_cols] output; row t is
 * written at out + (t - row_begin) * out_stride.  Column c of row t scores
 * key n = row_k_start[t] + c when 0 <= n < num_keys and n < row_k_end[t];
 * every other cell is -inf.  Element formats and strides as in
 * oracle_decode_typed. */
void oracle_prefill_typed(const void *q, int q_format, int64_t q_stride_row, int64_t q_stride_head,
                          const void *k, int k_format, double k_scale, int64_t k_stride,
                          int64_t num_keys, const int32_t *row_k_start, const int32_t *row_k_end,
                          int32_t num_rows, float scale, float *out, int64_t out_stride,
                          int32_t out_cols, int32_t row_begin, int32_t row_end)
{
    (void)num_rows;
    for (int32_t t = row_begin; t < row_end; ++t) {
        for (int32_t c = 0; c < out_cols; ++c) {
            int64_t n = (int64_t)row_k_start[t] + c;
            float value = neg_inf();
            if (n >= 0 && n < num_keys && n < row_k_end[t])
                value = score_cell_typed(q, (int64_t)t * q_stride_row, q_stride_head, q_format, k,
                                         n * k_stride, k_format, k_scale, scale);
            out[(int64_t)(t - row_begin) * out_stride + c] = value;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* BF16 queries and keys (the canonical inputs).                            */

/* oracle_decode_typed with bf16 queries and keys. */
void oracle_decode(const uint16_t *q, int64_t q_stride_req, int64_t q_stride_row,
                   int64_t q_stride_head, const uint16_t *k_cache, int64_t num_pages,
                   int32_t page_size, const int32_t *page_table, int64_t page_table_stride,
                   int32_t page_table_cols, const int32_t *comp_lens, const int32_t *visible,
                   int32_t num_reqs, int32_t dql, float scale, float *out,
                   int64_t out_stride, int32_t out_cols, int32_t row_begin, int32_t row_end)
{
    oracle_decode_typed(q, ORACLE_BF16, q_stride_req, q_stride_row, q_stride_head, k_cache,
                        ORACLE_BF16, 1.0, num_pages, page_size, page_table, page_table_stride,
                        page_table_cols, comp_lens, visible, num_reqs, dql, scale, out, out_stride,
                        out_cols, row_begin, row_end);
}

/* oracle_prefill_typed with bf16 queries and keys. */
void oracle_prefill(const uint16_t *q, int64_t q_stride_row, int64_t q_stride_head,
                    const uint16_t *k, int64_t k_stride, int64_t num_keys,
                    const int32_t *row_k_start, const int32_t *row_k_end, int32_t num_rows,
                    float scale, float *out, int64_t out_stride, int32_t out_cols,
                    int32_t row_begin, int32_t row_end)
{
    oracle_prefill_typed(q, ORACLE_BF16, q_stride_row, q_stride_head, k, ORACLE_BF16, 1.0, k_stride,
                         num_keys, row_k_start, row_k_end, num_rows, scale, out, out_stride, out_cols,
                         row_begin, row_end);
}

/* ---------------------------------------------------------------------- */
/* Compressed-cache metadata [CACHE compressed_qsa_slot_mapping and the      */
/* slot and k_work parts of _build_qsa_metadata_kernel].                    */

/* Slot of the compressed key each query token writes.  Token t of request r
 * (query_start_loc[r] <= t < query_start_loc[r+1]) at logical position pos
 * closes a group of compress_ratio tokens when pos >= 0 and (pos+1) % cr ==
 * 0; its compressed position cp = pos / cr lies in logical block
 * cp / storage_block_size of the request's block-table row, at row
 * cp % storage_block_size, so slot = block * storage_block_size +
 * cp % storage_block_size.  -1 when the token closes no group, the logical
 * block is past the table's columns, the block entry is negative, the
 * token's main-cache slot (common_slot_mapping, when given) is negative, or
 * the token is padding (past query_start_loc[num_reqs]). */
void oracle_cache_slots(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                        int32_t num_tokens, int32_t compress_ratio, const int32_t *block_table,
                        int64_t block_table_stride, int32_t block_table_cols,
                        int32_t storage_block_size, const int64_t *common_slot_mapping,
                        int64_t *slot_mapping)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = -1;
        for (int32_t r = 0; r < num_reqs; ++r) {
            if (t < query_start_loc[r] || t >= query_start_loc[r + 1]) continue;
            int64_t query_len = (int64_t)query_start_loc[r + 1] - query_start_loc[r];
            int64_t pos = (int64_t)seq_lens[r] - query_len + (t - query_start_loc[r]);
            if (pos < 0 || (pos + 1) % compress_ratio != 0) break;
            int64_t cp = pos / compress_ratio;
            int64_t logical_block = cp / storage_block_size;
            if (logical_block >= block_table_cols) break;
            int64_t block = block_table[r * block_table_stride + logical_block];
            if (block < 0) break;
            if (common_slot_mapping && common_slot_mapping[t] < 0) break;
            slot = block * storage_block_size + cp % storage_block_size;
            break;
        }
        slot_mapping[t] = slot;
    }
}

/* Work items of the compressed-cache writer.  A request with query tokens
 * owns max(seq_len//cr - (seq_len - query_len)//cr, 1) items: one per group
 * its chunk completes, and at least one (which also commits the raw-key
 * suffix); a request without query tokens owns none.  Items are numbered
 * request by request; item w holds (request, index within the request),
 * and every item past the last holds (-1, -1).  k_work is [max_num_work][2]. */
void oracle_k_work(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                   int32_t compress_ratio, int32_t *k_work, int32_t max_num_work)
{
    int64_t w = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        int64_t query_len = (int64_t)query_start_loc[r + 1] - query_start_loc[r];
        if (query_len <= 0) continue;
        int64_t groups = floor_div(seq_lens[r], compress_ratio) -
                         floor_div((int64_t)seq_lens[r] - query_len, compress_ratio);
        int64_t count = groups > 1 ? groups : 1;
        for (int64_t i = 0; i < count; ++i, ++w) {
            if (w < max_num_work) {
                k_work[2 * w] = r;
                k_work[2 * w + 1] = (int32_t)i;
            }
        }
    }
    for (; w < max_num_work; ++w) {
        k_work[2 * w] = -1;
        k_work[2 * w + 1] = -1;
    }
}

/* ---------------------------------------------------------------------- */
/* Raw-key ring and key-cache writes [QSA-CACHE: the circular branch of      */
/* _build_qsa_metadata_kernel and circular_qsa_slot_mapping; the caches      */
/* QSAKeyStateCache and QSACompressedKeyCache; QSA-PREP _to_dst_dtype].       */

static uint8_t float_to_e4m3_bits(float f);  /* defined with the query preparation below */

/* Ring slot of each query token.  Request r owns one ring of ring_size rows
 * in block block_table[r][0]; block 0 is the null block, owned by dummy and
 * padding requests, and is never written.  Token t of request r at logical
 * position pos >= 0 writes row pos % ring_size of the ring when it is one
 * of the last ring_size query tokens of its request (t + ring_size >= the
 * request's query end): slot = block * ring_size + pos % ring_size.  -1 for
 * every other token, for padding tokens and when the table has no
 * columns. */
void oracle_ring_slots(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                       int32_t num_tokens, const int32_t *block_table, int64_t block_table_stride,
                       int32_t block_table_cols, int32_t ring_size, int64_t *slot_mapping)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = -1;
        for (int32_t r = 0; r < num_reqs; ++r) {
            if (t < query_start_loc[r] || t >= query_start_loc[r + 1]) continue;
            int64_t query_end = query_start_loc[r + 1];
            int64_t query_len = query_end - query_start_loc[r];
            int64_t pos = (int64_t)seq_lens[r] - query_len + (t - query_start_loc[r]);
            if (pos < 0) break;
            if ((int64_t)t + ring_size < query_end) break;
            if (block_table_cols <= 0) break;
            int64_t block = block_table[r * block_table_stride];
            if (block <= 0) break;
            slot = block * ring_size + pos % ring_size;
            break;
        }
        slot_mapping[t] = slot;
    }
}

/* Key rows written to cache rows.  Row t of keys (128 bf16 elements, rows
 * key_stride elements apart) goes to cache row slots[t] when 0 <= slots[t]
 * < num_slots; cache rows are row_stride elements of the cache's format
 * apart, and rows no token writes are left as they are.  Cache format
 * ORACLE_BF16: the bits as they are.  ORACLE_FP8_E4M3: each value divided
 * by scale in fp32, then the nearest e4m3 code [_to_dst_dtype: round to
 * bf16, which the keys already are, divide by the scale, convert].
 * positions (bf16 caches only): NULL, or int64 positions of three axes
 * (element a * pos_stride_axis + t * pos_stride_token) that follow the key
 * in the row as three little-endian int64 from element 128
 * [QSAKeyStateCache: raw bf16 key, then exact int64 MRoPE positions]. */
void oracle_write_keys(const uint16_t *keys, int64_t key_stride, int32_t num_tokens, const int64_t *slots,
                       void *cache, int cache_format, int64_t row_stride, int64_t num_slots, float scale,
                       const int64_t *positions, int64_t pos_stride_axis, int64_t pos_stride_token)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        const uint16_t *src = keys + (int64_t)t * key_stride;
        if (cache_format == ORACLE_FP8_E4M3) {
            uint8_t *dst = (uint8_t *)cache + s * row_stride;
            for (int d = 0; d < QSA_ORACLE_DIM; ++d)
                dst[d] = float_to_e4m3_bits((float)bf16_bits_to_double(src[d]) / scale);
        } else {
            uint16_t *dst = (uint16_t *)cache + s * row_stride;
            for (int d = 0; d < QSA_ORACLE_DIM; ++d) dst[d] = src[d];
            if (positions) {
                for (int a = 0; a < 3; ++a) {
                    int64_t v = positions[a * pos_stride_axis + (int64_t)t * pos_stride_token];
                    memcpy(dst + QSA_ORACLE_DIM + 4 * a, &v, sizeof v);
                }
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Top-k block selection [MATE-QSA intro: the caller keeps the best blocks;  */
/* "Core Attention": request-local int32 indices, -1 padding].              */

typedef struct {
    float value;
    int32_t col;
} oracle_cand;

/* Larger value first; equal values (IEEE, so -0 == +0) by lower column. */
static int by_score_then_col(const void *a, const void *b)
{
    const oracle_cand *x = (const oracle_cand *)a, *y = (const oracle_cand *)b;
    if (x->value > y->value) return -1;
    if (x->value < y->value) return 1;
    return (x->col > y->col) - (x->col < y->col);
}

static int by_col(const void *a, const void *b)
{
    const oracle_cand *x = (const oracle_cand *)a, *y = (const oracle_cand *)b;
    return (x->col > y->col) - (x->col < y->col);
}

/* Rows [row_begin, row_end) of logits (row t at logits + t*logits_stride):
 * out_idx + (t - row_begin)*out_stride receives the picked columns in
 * ascending order, then -1.  Returns 0, or -1 when memory runs out. */
int oracle_topk(const float *logits, int64_t logits_stride, int32_t num_cols, int32_t k,
                int32_t *out_idx, int64_t out_stride, int32_t row_begin, int32_t row_end)
{
    oracle_cand *cand = (oracle_cand *)malloc(sizeof(oracle_cand) * (size_t)(num_cols > 0 ? num_cols : 1));
    if (!cand) return -1;
    for (int32_t t = row_begin; t < row_end; ++t) {
        const float *row = logits + (int64_t)t * logits_stride;
        int32_t n = 0;
        for (int32_t c = 0; c < num_cols; ++c)
            if (row[c] > neg_inf()) { /* false for -inf and for NaN */
                cand[n].value = row[c];
                cand[n].col = c;
                ++n;
            }
        qsort(cand, (size_t)n, sizeof(oracle_cand), by_score_then_col);
        int32_t keep = n < k ? n : k;
        qsort(cand, (size_t)keep, sizeof(oracle_cand), by_col);
        int32_t *dst = out_idx + (int64_t)(t - row_begin) * out_stride;
        for (int32_t i = 0; i < k; ++i) dst[i] = i < keep ? cand[i].col : -1;
    }
    free(cand);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Query preparation [QSA-PREP _norm_rope, _store_rotated, _to_dst_dtype].   */
/*                                                                          */
/* Readings where the page leaves a detail open:                            */
/*   - the sum of squares is the fp32 rounding of the exact sum (it is      */
/*     accumulated here in double); the page sums in fp32 in an unstated    */
/*     order, which can differ from this by a few fp32 ulps;                */
/*   - rrms is the fp32 rounding of 1/sqrt(mean + eps);                     */
/*   - arithmetic in the table's type rounds once per operation, with no    */
/*     fused multiply-add (bf16 operations computed in fp32 and rounded     */
/*     once are exact bf16 operations: 24 >= 2*8 + 2 bits);                 */
/*   - under MRoPE the page adds the three masked table reads to a zero     */
/*     start, which returns the selected entry except that -0 becomes +0;   */
/*   - fp8 is OCP e4m3: the nearest finite value, ties to the even code, so */
/*     magnitudes above 448 (and infinities) give 448; NaN gives 0x7F;      */
/*   - a position outside the table's rows is the caller's error: the       */
/*     pairs that use it read NaN for cos and sin.                          */
/* ------------------------------------------------------------------------ */

#define PREP_DIM 128
#define PREP_PAIRS 32 /* rotary dim 64: 32 (cos, sin) pairs, NeoX halves */

/* fp32 -> bf16 bit pattern, nearest with ties to even; NaN -> 0x7FC0. */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f)) return 0x7FC0;
    uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

static float bf16_round(float f) { return (float)bf16_bits_to_double(float_to_bf16_bits(f)); }

/* Rounds an fp32 result to the rotation type (bf16 or fp32). */
static float in_type(float v, int format) { return format == ORACLE_BF16 ? bf16_round(v) : v; }

/* fp32 -> e4m3 code: the nearest finite value, ties to the even code. */
static uint8_t float_to_e4m3_bits(float f)
{
    if (isnan(f)) return 0x7F;
    double a = fabs((double)f);
    if (a > 448.0) a = 448.0;
    int best = 0;
    double best_err = a;
    for (int code = 1; code <= 0x7E; ++code) {
        double err = fabs(e4m3_bits_to_double((uint8_t)code) - a);
        if (err < best_err || (err == best_err && (code & 1) == 0)) {
            best = code;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(f) ? 0x80 : 0));
}

void oracle_round_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_bits(x[i]);
}

void oracle_round_e4m3(const float *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_e4m3_bits(x[i]);
}

/* Interleaved MRoPE: the axis (0 temporal, 1 height, 2 width) of rotary
 * pair j under section (t, h, w).  The page writes j <= 3h; j % 3 == 1
 * never holds at j == 3h, so it is the same set. */
static int mrope_axis(int j, const int32_t *section)
{
    if (j % 3 == 1 && j < 3 * section[1]) return 1;
    if (j % 3 == 2 && j < 3 * section[2]) return 2;
    return 0;
}

/* Tokens [token_begin, token_end): q holds num_heads heads of 128 bf16
 * features per token (head h of token t at q + t*q_stride_token + h*128).
 * positions[a*pos_stride_axis + t*pos_stride_token] is token t's position
 * on axis a (pos_stride_axis 0 for one position per token).  cos_sin has
 * cos_sin_rows rows of 32 cos then 32 sin in rot_format (bf16 or fp32),
 * the weight 128 entries in weight_format (bf16 or fp32).  mrope_section
 * is NULL (plain rotary) or (t, h, w).  Output element (t, h, d) lands at
 * t*out_stride_token + h*out_stride_head + d as bf16, or as e4m3 of the
 * bf16 value divided by out_scale. */
void oracle_prepare_q(const uint16_t *q, int64_t q_stride_token, int32_t num_heads, const int64_t *positions,
                      int64_t pos_stride_axis, int64_t pos_stride_token, const void *cos_sin, int rot_format,
                      int64_t cos_sin_rows, const void *weight, int weight_format, float eps,
                      const int32_t *mrope_section, void *out, int out_format, float out_scale,
                      int64_t out_stride_token, int64_t out_stride_head, int32_t token_begin, int32_t token_end)
{
    for (int32_t t = token_begin; t < token_end; ++t) {
        int64_t pos[3];
        for (int a = 0; a < 3; ++a) pos[a] = positions[a * pos_stride_axis + (int64_t)t * pos_stride_token];
        for (int32_t h = 0; h < num_heads; ++h) {
            const uint16_t *xb = q + (int64_t)t * q_stride_token + (int64_t)h * PREP_DIM;
            float x[PREP_DIM], y[PREP_DIM], o[PREP_DIM];
            double sum_sq = 0.0;
            for (int d = 0; d < PREP_DIM; ++d) {
                x[d] = (float)bf16_bits_to_double(xb[d]);
                sum_sq += (double)(x[d] * x[d]);
            }
            float mean_eps = (float)sum_sq / (float)PREP_DIM + eps;
            float rrms = (float)(1.0 / sqrt((double)mean_eps));
            for (int d = 0; d < PREP_DIM; ++d) {
                float gain = (float)element(weight, d, weight_format) + 1.0f;
                y[d] = in_type((x[d] * rrms) * gain, rot_format);
            }
            for (int j = 0; j < PREP_PAIRS; ++j) {
                int64_t p = pos[mrope_section ? mrope_axis(j, mrope_section) : 0];
                float c = NAN, s = NAN;
                if (p >= 0 && p < cos_sin_rows) {
                    c = (float)element(cos_sin, p * 2 * PREP_PAIRS + j, rot_format);
                    s = (float)element(cos_sin, p * 2 * PREP_PAIRS + PREP_PAIRS + j, rot_format);
                    if (mrope_section) {
                        c = in_type(0.0f + c, rot_format);
                        s = in_type(0.0f + s, rot_format);
                    }
                }
                float lo = y[j], hi = y[j + PREP_PAIRS];
                o[j] = in_type(in_type(lo * c, rot_format) - in_type(hi * s, rot_format), rot_format);
                o[j + PREP_PAIRS] = in_type(in_type(hi * c, rot_format) + in_type(lo * s, rot_format), rot_format);
            }
            for (int d = 2 * PREP_PAIRS; d < PREP_DIM; ++d) o[d] = y[d];
            for (int d = 0; d < PREP_DIM; ++d) {
                uint16_t v = float_to_bf16_bits(o[d]);
                int64_t at = (int64_t)t * out_stride_token + (int64_t)h * out_stride_head + d;
                if (out_format == ORACLE_FP8_E4M3)
                    ((uint8_t *)out)[at] = float_to_e4m3_bits((float)bf16_bits_to_double(v) / out_scale);
                else
                    ((uint16_t *)out)[at] = v;
            }
        }
    }
}
