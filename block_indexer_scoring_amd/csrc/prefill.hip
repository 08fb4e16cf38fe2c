// Prefill scores for the QSA MQA indexer on gfx950.
//
// Definition (MATE "QSA (Qwen Sparse Attention)", section "MQA score",
// packed form): row t scores key n = row_k_start[t] + c in output column c
// as scale * sum_h relu(q[t][h] . k[n]) when 0 <= n < num_keys and
// n < row_k_end[t]; every other cell is -inf.
//
// The scores are one dense contraction [rows*4 heads x 128] x [128 x keys]
// followed by a per-(row, key) epilogue, run on the matrix cores with
// v_mfma_f32_16x16x32_bf16:
//   - A workgroup of 8 wavefronts owns kBM = 128 query rows (16 per wave)
//     and a chunk of output columns; one workgroup fills a CU (two waves
//     per SIMD).  Each wavefront keeps its 16 rows x 4 heads of Q in
//     registers as MFMA A fragments for the whole chunk (m = 4*row + head).
//   - Key tiles of 64 keys (16 KB) are staged in LDS by buffer loads that
//     write LDS directly, two tiles per buffer and two buffers: the loads of
//     the next pair are in flight while the current pair is multiplied (one
//     workgroup barrier per 128 keys), and all 8 waves reuse each staged
//     tile.  The buffer resource spans exactly the existing keys, so keys
//     outside [0, num_keys) arrive as zeros with no per-key edge path.  LDS
//     rows are XOR-swizzled in 16-byte units so the B-fragment reads are
//     free of bank conflicts.
//   - In the MFMA result a lane holds the 4 heads of one (row, key), so
//     ReLU, head sum and scale run in-lane; tile key c + 4n + g sits in
//     column n of group g, giving each lane 4 consecutive keys for one
//     16-byte store.  A wave works through its tile in 4-row slices, and
//     the epilogue and store of each slice run while the matrix cores
//     multiply the next (software pipeline, instruction groups interleaved
//     MFMA / VALU), so the vector ALU work hides under MFMA time.  Only
//     tiles that cross a row's interval end (or start) evaluate the mask.
//   - Stores and key loads share the in-order vector-memory counter; every
//     slice's scores leave as exactly one buffer store, so the wait for a
//     key buffer can leave the most recent stores in flight.
//   - Workgroups are numbered so that those on one XCD (launch order is
//     round-robin over the 8 XCDs) share a column chunk: each XCD's L2
//     then holds one chunk's keys rather than all of them.
//   - Tiles past the last key any row of the workgroup may see are not
//     multiplied: they are written as -inf only (causal tile skip).
// Rows of one workgroup normally share row_k_start (packed requests); rows
// with different starts are handled in one pass per distinct start.
#include <climits>

#include "qsa_device.h"
#include "qsa_internal.h"


namespace qsa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 64;                     // keys per LDS tile
constexpr int kTileElems = kBN * kDim;      // bf16 elements per tile
constexpr int kBlocksPerWave = kBN / 4 / kWaves;  // 1 KB LDS blocks staged per wave per tile
constexpr int kTilesPerStage = 2;                // key tiles per LDS buffer
constexpr int kStoresInFlight = 4;               // stores a key-buffer wait leaves outstanding
constexpr int kXcds = 8;                         // XCDs that launch order cycles through

// LDS element offset of 16-byte chunk `chunk` (0..15) of tile key `key`.
__device__ __forceinline__ int lds_offset(int key, int chunk) {
    return key * kDim + ((chunk ^ ((key >> 2) & 15)) << 3);
}

__device__ __forceinline__ int clamp_cols(int64_t v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : (int)v);
}

__device__ __forceinline__ int wave_min(int v) {
    v = min(v, __shfl_xor(v, 16, 64));
    v = min(v, __shfl_xor(v, 32, 64));
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void store4(float *dst, bool vec, int col, int c_end, float a, float b,
                                       float c, float d) {
    if (vec && col + 3 < c_end) {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{a, b, c, d};
    } else {
        if (col < c_end) dst[0] = a;
        if (col + 1 < c_end) dst[1] = b;
        if (col + 2 < c_end) dst[2] = c;
        if (col + 3 < c_end) dst[3] = d;
    }
}

// Fourth word of a raw buffer resource (32-bit data format) on gfx9-class GPUs.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of the score stores: non-temporal (the "nt" bit).  The
// scores are written once and not read back by this kernel; with whole
// 128-byte lines per store (line-aligned stores below) streaming them
// measured faster than the default policy.
constexpr int kStoreNT = 2;

// What the kernel does with each slice of scores:
//   kModeScores       store them (plain stores);
//   kModeScoresExact  store them as exactly one buffer store per lane (the
//                     output rows of a workgroup span less than 2 GiB), so
//                     the number of vector-memory ops after each key
//                     prefetch is fixed on every path;
//   kModeGroupMax     (fused top-k, first pass) keep the maximum of each
//                     8-key group of a row: the keys 4n .. 4n+3 of two
//                     consecutive tiles that lane n holds;
//   kModeCandidates   (fused top-k, second pass) append the cells at or
//                     above the row's floor to the row's candidate list;
//   kModeKeys16       (fused top-k) store the top 16 bits of each cell's
//                     order key (2 bytes per cell, 0 outside a row's keys),
//                     as exactly one 8-byte buffer store per lane and slice,
//                     every row written out to its 64-column padded end.
constexpr int kModeScores = 0, kModeScoresExact = 1, kModeGroupMax = 2, kModeCandidates = 3, kModeKeys16 = 4;
constexpr int kGroupTiles = kFusedGroupTiles;  // tiles per group in kModeGroupMax (16 groups per row of them)

// Inclusive prefix sum within each 16-lane row of a wavefront (DPP
// row_shr 1, 2, 4, 8 with zero fill).
__device__ __forceinline__ uint32_t row16_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    return x;
}

// kF16: Q and K are fp16 rather than bf16 (the same layout and staging; only
// the MFMA's operand type differs).  kRotate (kModeScoresExact only): the
// line-aligned store layout below, for outputs whose rows do not all start
// on a 128-byte line; with aligned rows the plain layout is the same stores
// without the carried cells.
template <int kMode, bool kF16, bool kRotate>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillParams p) {
    constexpr bool kExact = kMode == kModeScoresExact;
    static_assert(!kRotate || kExact, "line-aligned layout is for exact score stores");
    constexpr bool kFused = kMode == kModeGroupMax || kMode == kModeCandidates;
    constexpr bool kKeys = kMode == kModeKeys16;
    // Two separate LDS objects (not one [2][...] array), so the compiler can
    // tell the buffer being read from the one being filled and does not wait
    // for the prefetch before reading the current tile.
    __shared__ __attribute__((aligned(16))) uint16_t ktile0[kTilesPerStage * kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t ktile1[kTilesPerStage * kTileElems];
    __shared__ int s_start[kBM];
    __shared__ int s_end[kBM];  // min(row_k_end, num_keys)
    __shared__ int s_done[kBM];
    __shared__ int s_cur, s_lim;
    // kModeCandidates, per row of the workgroup: the floor as a float, and
    // the segment's start (an entry index in the workgroup's pools) and size.
    __shared__ float c_floor[kFused ? kBM : 1];
    __shared__ int c_sbase[kFused ? kBM : 1], c_segn[kFused ? kBM : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int q4 = lane >> 4;
    // Workgroup i runs on XCD i % 8.  Renumber so that the workgroups of
    // one XCD take consecutive (row block, chunk) slots, chunk-major.
    const int groups = p.row_blocks * p.col_chunks;
    const int xcd = blockIdx.x % kXcds;
    const int slot = xcd * (groups / kXcds) + min(xcd, groups % kXcds) + (int)blockIdx.x / kXcds;
    const int rb = slot % p.row_blocks;
    const int cc = slot / p.row_blocks;
    const int row0 = rb * kBM;
    const int c_begin = cc * p.col_chunk;
    const int c_end = min(c_begin + p.col_chunk, p.out_cols);
    const int n_tiles = (c_end - c_begin + kBN - 1) / kBN;

    // Line-aligned stores (kModeScoresExact).  A row that starts partway
    // into a 128-byte line would have every 256-byte tile segment straddle
    // three lines, two of them partly written, which costs HBM write
    // throughput.  So the 16 rows of a wave are spaced `dl` rows apart,
    // which puts all of them at the same offset within a line (dl * row
    // pitch is a multiple of 128 bytes), and each lane's columns are rotated
    // by that offset: lane n computes tile columns 4*((n - rot) mod 16) ..
    // +3 (B fragments read rotated), and the store of a slice covers the
    // line-aligned columns tile_c - 4*rot .. tile_c + 63 - 4*rot.  Lanes
    // n < rot store the previous tile's cells, which they still hold.
    // Without kRotate (the other modes, or every row on a line boundary),
    // dl = 1 and rot = 0.
    int dl = 1;
    if (kRotate) {
        const int u = (int)((p.out_stride >> 2) & 7);  // 16-byte units per row, mod 8
        dl = u == 0 ? 1 : ((u & 1) ? 8 : ((u & 2) ? 4 : 2));
    }
    const int a_w = (wave % dl) + kRowsPerWave * dl * (wave / dl);  // wave row j is a_w + dl * j
    const int rot = kRotate ? __builtin_amdgcn_readfirstlane(
                                  (int)((((uintptr_t)p.out + (uint64_t)(row0 + a_w) * (uint64_t)p.out_stride * 4) >> 4) & 7))
                            : 0;
    if (kKeys && blockIdx.x == 0 && tid == 0) *p.hard_count = 0;  // read by the selects that follow
    const int lc = 4 * ((n - rot) & 15);  // first tile column of this lane's cells
    const int sc = 4 * (n - rot);         // first column of this lane's store, relative to the tile
    const bool lo = kRotate && n < rot;   // stores the previous tile's cells

    for (int i = tid; i < kBM; i += kThreads) {
        const int t = row0 + i;
        if (t < p.num_rows) {
            const int ks = p.row_k_start[t];
            const int ke = p.row_k_end[t];
            s_start[i] = ks;
            s_end[i] = (int64_t)ke < p.num_keys ? ke : (int)p.num_keys;
            s_done[i] = 0;
        } else {
            s_start[i] = 0;
            s_end[i] = 0;
            s_done[i] = 1;
        }
    }

    // Q fragments of this wave's 16 rows: tile mt covers rows 4mt..4mt+3,
    // lane (n, q4) holds row 4mt + n/4, head n%4, features 32ks + 8q4 .. +7.
    u32x4 qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int t = row0 + a_w + dl * (4 * mt + (n >> 2));
        const uint16_t *src = p.q + (int64_t)t * p.q_stride_row + (int64_t)(n & 3) * p.q_stride_head + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qa[mt][ks] = t < p.num_rows ? load_u32x4(src + 32 * ks) : zero_u32x4();
    }
    // Complete the Q loads here, so that no wait inside the tile loop has to
    // cover them (the loop's only vector-memory loads are the key prefetch).
    __builtin_amdgcn_s_waitcnt(0);

    // Key staging goes straight from global memory to LDS (buffer loads
    // that write LDS): one instruction moves 1 KB, lane l writing bytes
    // 16l .. 16l+15 of the block.  Block b of a tile holds keys
    // 4b .. 4b+3; lane l of block b therefore fetches key 4b + l/16, chunk
    // (l%16) ^ (b%16), which puts the XOR swizzle of lds_offset() in place.
    // Wave w stages blocks w*kBlocksPerWave .. +kBlocksPerWave-1.
    uint32_t st_goff[kBlocksPerWave];  // byte offset from the tile's first key
#pragma unroll
    for (int i = 0; i < kBlocksPerWave; ++i) {
        const int b = wave * kBlocksPerWave + i;
        const int key = 4 * b + (lane >> 4);
        st_goff[i] = (uint32_t)(key * p.k_stride * 2 + (((lane & 15) ^ (b & 15)) << 4));
    }
    // B-fragment read offsets: key lc + g, chunk 4ks + q4; g adds 128 elements.
    int rd_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rd_off[ks] = lds_offset(lc, 4 * ks + q4);

    for (;;) {
        if (tid == 0) {
            s_cur = INT_MAX;
            s_lim = INT_MIN;
        }
        __syncthreads();
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i]) atomicMin(&s_cur, s_start[i]);
        __syncthreads();
        const int cur = __builtin_amdgcn_readfirstlane(s_cur);
        if (cur == INT_MAX) break;
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i] && s_start[i] == cur)
                atomicMax(&s_lim, clamp_cols((int64_t)s_end[i] - cur, -1, INT_MAX - kBN));
        __syncthreads();
        const int lim = __builtin_amdgcn_readfirstlane(s_lim);  // columns >= lim hold no key for any row of this pass

        // This lane's output rows (MFMA result layout: row 4mt + q4).
        bool in_pass[4];
        int row_lim[4];
        int lane_min_lim = INT_MAX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int idx = a_w + dl * (4 * mt + q4);
            in_pass[mt] = !s_done[idx] && s_start[idx] == cur;
            row_lim[mt] = clamp_cols((int64_t)s_end[idx] - cur, -1, INT_MAX - kBN);
            if (in_pass[mt]) lane_min_lim = min(lane_min_lim, row_lim[mt]);
        }
        // Tiles inside [col_min, wave_lim) need no mask for any row of this wave.
        const int wave_lim = wave_min(lane_min_lim);

        // Fused top-k state, per slice row of this lane.
        float gm[4];        // kModeGroupMax: maximum of the open group
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) gm[mt] = neg_inf();
        // kModeCandidates, per slice row of this lane: keys equal to the
        // floor seen so far in this chunk, and candidates written.  Every
        // lane of the row's 16 keeps the same copy in registers, so a slice
        // updates them with no memory round trip.
        int c_teq[4] = {}, c_ncand[4] = {};
        if (kMode == kModeCandidates) {
            for (int i = tid; i < kBM; i += kThreads) {
                const int row = row0 + i;
                const bool cand = !s_done[i] && s_start[i] == cur;
                const int32_t *so = p.seg_off + (int64_t)row * (p.col_chunks + 1) + cc;
                const int s0 = cand ? min(so[0], p.pool_cap) : 0;
                // The float f whose key is the floor key F.  Keys order like
                // the floats (-0 with +0; -inf and NaN have key 0), so for a
                // score x: key(x) > F iff x > f, and key(x) == F iff x == f.
                // F = 0 (no floor): f = -inf, which every visible score is
                // above and none equals.  Rows outside this pass: f = NaN,
                // which nothing is above or equal to; cells outside a row's
                // keys are NaN in the epilogue for the same reason.
                const uint32_t fk = cand ? p.floor_key[row] : 0u;
                const float f = __uint_as_float((fk & 0x80000000u) ? (fk & 0x7fffffffu) : ~fk);
                c_floor[i] = !cand ? __uint_as_float(0x7fc00000u) : (fk == 0u ? neg_inf() : f);
                c_sbase[i] = i * p.pool_cap + s0;
                c_segn[i] = cand ? min(so[1], p.pool_cap) - s0 : 0;  // within the pool in any case
            }
            __syncthreads();
        }
        const int col_min = clamp_cols(-(int64_t)cur, 0, INT_MAX - kBN);  // key index >= 0

        int n_compute = 0;
        if (lim > c_begin) n_compute = min(n_tiles, (lim - c_begin + kBN - 1) / kBN);

        // Stage one key tile (64 keys x 256 bytes) into LDS buffer `buf`: a
        // uniform base plus per-lane constant offsets; a tile that reaches
        // past either end of the keys is zero-filled and loaded per key.
        // Keys of this pass as one raw buffer that starts at the first key
        // the chunk can touch (or key 0) and ends at the last key: a lane
        // whose key lies outside [0, num_keys) gets an offset outside the
        // buffer (negative offsets wrap past its end), and the hardware
        // writes zeros to LDS for it.  Staging is therefore the same four
        // direct-to-LDS loads for every tile, edges included.
        int64_t k_first = (int64_t)cur + c_begin;
        if (k_first < 0) k_first = 0;
        int64_t k_bytes = p.num_keys - k_first;
        k_bytes = k_bytes < 0 ? 0 : k_bytes * p.k_stride * 2;
        const int k_records = __builtin_amdgcn_readfirstlane((int)(k_bytes > INT_MAX ? INT_MAX : k_bytes));
        const uint64_t k_base = (uint64_t)(p.k + k_first * p.k_stride);
        const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(k_base >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)k_base)),
            0, k_records, kBufferWord3);
        // Stage one key tile (64 keys x 256 bytes) into LDS buffer `buf`.
        auto stage = [&](int tile_c, uint16_t *buf) {
            const uint32_t tile_off = (uint32_t)(((int64_t)cur + tile_c - k_first) * p.k_stride * 2);
#pragma unroll
            for (int i = 0; i < kBlocksPerWave; ++i) {
                const int b = wave * kBlocksPerWave + i;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (__attribute__((address_space(3))) void *)&buf[b * 512],
                                                         16, tile_off + st_goff[i], 0, 0, 0);
            }
        };

        // The workgroup's output rows as one raw buffer.  A slice of scores
        // (4 rows x 64 keys of one wave) goes out as exactly one buffer store
        // per lane: lanes whose row is not in this pass, and the placeholder
        // slice before a pass's first tile, store to an offset past the
        // buffer's end, which the hardware drops.  With that fixed count the
        // wait for a buffer of keys can leave the latest stores in flight.
        const __amdgpu_buffer_rsrc_t out_rsrc =
            kKeys ? __builtin_amdgcn_make_buffer_rsrc(p.keys16 + (int64_t)row0 * p.keys_stride, 0,
                                                      (int)((int64_t)min(kBM, p.num_rows - row0) * p.keys_stride * 2),
                                                      kBufferWord3)
                  : __builtin_amdgcn_make_buffer_rsrc(
                        p.out + (int64_t)row0 * p.out_stride, 0,
                        kExact ? (int)((int64_t)min(kBM, p.num_rows - row0) * p.out_stride * 4) : 0, kBufferWord3);
        constexpr uint32_t kDropped = 0x80000000u;
        // The fused passes' outputs of this workgroup's rows as one raw
        // buffer (group maxima, or candidate pools), for the same reason:
        // every slice issues a fixed number of stores.
        const int wg_rows = min(kBM, p.num_rows - row0);
        const __amdgpu_buffer_rsrc_t fused_rsrc =
            kMode == kModeGroupMax
                ? __builtin_amdgcn_make_buffer_rsrc(p.gmax + (int64_t)row0 * p.gmax_stride, 0,
                                                    wg_rows * p.gmax_stride * 4, kBufferWord3)
            : kMode == kModeCandidates
                ? __builtin_amdgcn_make_buffer_rsrc(p.cand + (int64_t)row0 * p.pool_cap * 2, 0,
                                                    wg_rows * p.pool_cap * 8, kBufferWord3)
                : __builtin_amdgcn_make_buffer_rsrc(p.out, 0, 0, kBufferWord3);
        // Byte offset of (row, column sc) in out_rsrc, modulo 2^32: it is
        // negative for row 0 and lanes n < rot, whose stores then lie at
        // least one tile in (the first tile's are dropped).
        uint32_t row_boff[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int idx = a_w + dl * (4 * mt + q4);
            row_boff[mt] = !in_pass[mt] ? kDropped
                           : kKeys      ? (uint32_t)(((int64_t)idx * p.keys_stride + sc) * 2)
                                        : (uint32_t)(((int64_t)idx * p.out_stride + sc) * 4);
        }
        // Element offset of (row of slice mt, column col) from out_wg, for the
        // plain stores of partial and -inf-only tiles.
        float *const out_wg = p.out + (int64_t)row0 * p.out_stride;
        auto row_elem = [&](int mt, int col) {
            return (int64_t)(a_w + dl * (4 * mt + q4)) * p.out_stride + col;
        };
        // kModeScoresExact: the cells of the previous tile, per slice.
        f32x4 keep[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) keep[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Scores of one slice: rows 4mt .. 4mt+3 of the wave (x 4 heads, the
        // MFMA's m = 4 * row + head) against the tile's 64 keys.
        auto multiply = [&](int mt, const u32x4 (&b)[4][4], f32x4 (&acc)[4]) {
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[g] = mfma_qk<kF16>(qa[mt][ks], b[ks][g], acc[g]);
        };
        // Epilogue and store of a slice whose tile needs no mask and lies
        // wholly inside the chunk (tile_c < 0: placeholder, store dropped).
        auto finish_fast = [&](int mt, int tile_c, const f32x4 (&acc)[4]) {
            const f32x4 v{head_sum_score(acc[0], p.scale), head_sum_score(acc[1], p.scale),
                          head_sum_score(acc[2], p.scale), head_sum_score(acc[3], p.scale)};
            if constexpr (kKeys) {
                const u32x2 kw{score_keys16(v[0], v[1]), score_keys16(v[2], v[3])};
                __builtin_amdgcn_raw_buffer_store_b64(kw, out_rsrc, tile_c >= 0 ? row_boff[mt] : kDropped,
                                                      2 * max(tile_c, 0), kStoreNT);
            } else if constexpr (kRotate) {
                const f32x4 w = lo ? keep[mt] : v;
                keep[mt] = v;
                const bool drop = tile_c < 0 || (lo && tile_c == c_begin);
                __builtin_amdgcn_raw_buffer_store_b128(w, out_rsrc, drop ? kDropped : row_boff[mt] + 4 * tile_c, 0,
                                                       kStoreNT);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(v, out_rsrc, tile_c >= 0 ? row_boff[mt] : kDropped,
                                                       4 * max(tile_c, 0), kStoreNT);
            }
        };
        // Any slice: mask per cell, partial tiles and unbounded rows.
        auto finish_general = [&](int mt, int tile_c, bool masked, const f32x4 (&acc)[4]) {
            if constexpr (kKeys) {
                // Cells outside the row's keys, or past the chunk's end (the
                // row's padding), get key 0; the store covers the whole tile.
                const int col = tile_c + lc;
                bool ok[4];
                f32x4 v;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = col + g;
                    ok[g] = !masked || (c < row_lim[mt] && c >= col_min && c < c_end);
                    v[g] = head_sum_score(acc[g], p.scale);
                }
                const u32x2 kw{score_keys16(v[0], v[1], ok[0], ok[1]), score_keys16(v[2], v[3], ok[2], ok[3])};
                __builtin_amdgcn_raw_buffer_store_b64(kw, out_rsrc, tile_c >= 0 ? row_boff[mt] : kDropped,
                                                      2 * max(tile_c, 0), kStoreNT);
                return;
            }
            f32x4 v;
            if (!masked) {
                v = f32x4{head_sum_score(acc[0], p.scale), head_sum_score(acc[1], p.scale),
                          head_sum_score(acc[2], p.scale), head_sum_score(acc[3], p.scale)};
            } else {
                const int col = tile_c + lc;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = col + g;
                    v[g] = (c < row_lim[mt] && c >= col_min) ? head_sum_score(acc[g], p.scale) : neg_inf();
                }
            }
            if (kExact) {
                // Lanes wholly inside the chunk take the buffer store; the one
                // lane that straddles the chunk's end stores its cells singly.
                f32x4 w = v;
                if constexpr (kRotate) {
                    w = lo ? keep[mt] : v;
                    keep[mt] = v;
                }
                const int cs = tile_c + sc;
                const bool drop = tile_c < 0 || (lo && tile_c == c_begin);
                if constexpr (kRotate)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        w, out_rsrc, (!drop && cs + 3 < c_end) ? row_boff[mt] + 4 * tile_c : kDropped, 0, kStoreNT);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(w, out_rsrc, (!drop && cs + 3 < c_end) ? row_boff[mt] : kDropped,
                                                           4 * max(tile_c, 0), kStoreNT);
                if (!drop && in_pass[mt] && cs < c_end && cs + 3 >= c_end)
                    store4(out_wg + row_elem(mt, cs), false, cs, c_end, w[0], w[1], w[2], w[3]);
            } else if (tile_c >= 0 && in_pass[mt]) {
                const int col = tile_c + 4 * n;
                store4(out_wg + row_elem(mt, col), p.out_vec, col, c_end, v[0], v[1], v[2], v[3]);
            }
        };
        // Fused top-k epilogue of one slice (kModeGroupMax, kModeCandidates).
        // `masked` is a literal at each call, so the unmasked form folds.
        auto finish_topk = [&](int mt, int tile_c, bool masked, const f32x4 (&acc)[4]) {
            if (tile_c < 0) {  // placeholder before a pass's first tile: dropped stores only
                if (kMode == kModeGroupMax)
                    __builtin_amdgcn_raw_buffer_store_b32(0u, fused_rsrc, kDropped, 0, 0);
                else
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, fused_rsrc, kDropped, 0, 0);
                return;
            }
            const int ri = a_w + dl * (4 * mt + q4);  // row in the workgroup
            const int col = tile_c + lc;
            // Rows outside this pass are never stored (group maxima) or have
            // a NaN floor (candidates), so only the key range is checked.
            f32x4 v;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = col + g;
                const bool ok = !masked || (c < row_lim[mt] && c >= col_min && c < c_end);
                v[g] = ok ? head_sum_score(acc[g], p.scale)
                          : (kMode == kModeCandidates ? __uint_as_float(0x7fc00000u) : neg_inf());
            }
            if (kMode == kModeGroupMax) {
                gm[mt] = max(gm[mt], max(max(v[0], v[1]), max(v[2], v[3])));
                const int tix = tile_c / kBN;  // chunks start on group boundaries
                // Exactly one store per slice (dropped unless the group closes).
                const bool closes = tix % kGroupTiles == kGroupTiles - 1 || tile_c + kBN >= c_end;
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(gm[mt]), fused_rsrc,
                    closes && in_pass[mt] ? (uint32_t)((ri * p.gmax_stride + (tix / kGroupTiles) * 16 + n) * 4)
                                          : kDropped,
                    0, 0);
                if (closes) gm[mt] = neg_inf();
            } else {
                // Cells above the floor, and the first `topk` cells equal to
                // it in this chunk, appended in column order to the row's
                // segment for this chunk (lanes 16q4 .. 16q4+15 hold this
                // row's keys 4n .. 4n+3).  The floor is compared as a float,
                // which orders scores as their keys do.  Entries hold the
                // score's bits: a taken score is >= +0, so its key is those
                // bits with the sign bit set.
                const float f = c_floor[ri];
                bool gt[4], eq[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    gt[g] = v[g] > f;
                    eq[g] = v[g] == f;
                }
                const int nc = c_ncand[mt], segn = c_segn[ri], sbase = c_sbase[ri];
                // The row's totals below: lane 15 of each 16-lane row,
                // broadcast within the row by DPP (row_newbcast:15).
                if (__builtin_expect(__ballot((eq[0] || eq[1]) || (eq[2] || eq[3])) == 0, 1)) {
                    // No cell of the wave equals its row's floor (the usual
                    // case): the cells above it, in column order.
                    const uint32_t cnt = (uint32_t)(((int)gt[0] + (int)gt[1]) + ((int)gt[2] + (int)gt[3]));
                    const uint32_t incl = row16_inclusive_scan(cnt);
                    const uint32_t tot = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x15F, 0xf, 0xf, false);
                    int pos = nc + (int)incl - (int)cnt;
                    c_ncand[mt] = nc + (int)tot;
                    // The segment holds every candidate by construction; a
                    // lane whose cells would not all fit drops them all.
                    const bool fits = pos + (int)cnt <= segn;
                    // Exactly four 8-byte stores per slice, one per cell
                    // (dropped unless the cell is taken).
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        __builtin_amdgcn_raw_buffer_store_b64(
                            u32x2{__float_as_uint(v[g]), (uint32_t)(col + g)}, fused_rsrc,
                            gt[g] && fits ? (uint32_t)(sbase + pos) * 8u : kDropped, 0, 0);
                        pos += gt[g];
                    }
                } else {
                    int ngt = 0, neq = 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        ngt += gt[g];
                        neq += eq[g];
                    }
                    const uint32_t packed = ((uint32_t)ngt << 16) | (uint32_t)neq;
                    const uint32_t incl = row16_inclusive_scan(packed);
                    const uint32_t excl = incl - packed;
                    const uint32_t tot = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x15F, 0xf, 0xf, false);
                    const int teq = c_teq[mt];
                    const int avail = max(p.topk - teq, 0);
                    const int nw = (int)(tot >> 16) + min((int)(tot & 0xffffu), avail);
                    int eqi = (int)(excl & 0xffffu);
                    int pos = nc + (int)(excl >> 16) + min(eqi, avail);
                    c_teq[mt] = teq + (int)(tot & 0xffffu);
                    c_ncand[mt] = nc + nw;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const bool take = gt[g] || (eq[g] && eqi < avail);
                        __builtin_amdgcn_raw_buffer_store_b64(
                            u32x2{__float_as_uint(v[g]), (uint32_t)(col + g)}, fused_rsrc,
                            take && pos < segn ? (uint32_t)(sbase + pos) * 8u : kDropped, 0, 0);
                        pos += take;
                        eqi += eq[g];
                    }
                }
            }
        };

        // Software pipeline over slices: the epilogue and store of slice s
        // run while the matrix cores multiply slice s + 1, so vector ALU work
        // and stores hide under MFMA time.  Slice 3 of a tile is finished
        // during slice 0 of the next.  accA/accB alternate; accB carries the
        // deferred slice from tile to tile.
        f32x4 accA[4], accB[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) accB[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        int prev_c = -1;
        bool prev_masked = false;
        auto interleave = [&]() {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
            }
            __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);      // the store
        };
        auto interleave_valu = [&]() {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
            }
        };
        auto load_b = [&](const uint16_t *tile, u32x4 (&b)[4][4]) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int g = 0; g < 4; ++g) b[ks][g] = *reinterpret_cast<const u32x4 *>(&tile[rd_off[ks] + g * kDim]);
        };
        auto do_tile = [&](int tile_c, const u32x4 (&b)[4][4]) {
            const bool masked =
                !(tile_c + kBN <= wave_lim && tile_c >= col_min) || ((kFused || kKeys) && tile_c + kBN > c_end);
            const bool full = p.out_vec && tile_c + kBN <= c_end;
            if (kFused) {
                if (!masked && !prev_masked) {
                    // The group-maximum epilogue is plain VALU work: interleaved
                    // with the MFMAs like the score path's.
                    multiply(0, b, accA);
                    finish_topk(3, prev_c, false, accB);
                    if (kMode == kModeGroupMax) interleave_valu();
                    multiply(1, b, accB);
                    finish_topk(0, tile_c, false, accA);
                    if (kMode == kModeGroupMax) interleave_valu();
                    multiply(2, b, accA);
                    finish_topk(1, tile_c, false, accB);
                    if (kMode == kModeGroupMax) interleave_valu();
                    multiply(3, b, accB);
                    finish_topk(2, tile_c, false, accA);
                    if (kMode == kModeGroupMax) interleave_valu();
                } else {
                    multiply(0, b, accA);
                    finish_topk(3, prev_c, prev_masked, accB);
                    multiply(1, b, accB);
                    finish_topk(0, tile_c, masked, accA);
                    multiply(2, b, accA);
                    finish_topk(1, tile_c, masked, accB);
                    multiply(3, b, accB);
                    finish_topk(2, tile_c, masked, accA);
                }
            } else if ((kKeys || (kExact && full)) && !masked && !prev_masked) {
                multiply(0, b, accA);
                finish_fast(3, prev_c, accB);
                interleave();
                multiply(1, b, accB);
                finish_fast(0, tile_c, accA);
                interleave();
                multiply(2, b, accA);
                finish_fast(1, tile_c, accB);
                interleave();
                multiply(3, b, accB);
                finish_fast(2, tile_c, accA);
                interleave();
            } else {
                multiply(0, b, accA);
                finish_general(3, prev_c, prev_masked, accB);
                multiply(1, b, accB);
                finish_general(0, tile_c, masked, accA);
                multiply(2, b, accA);
                finish_general(1, tile_c, masked, accB);
                multiply(3, b, accB);
                finish_general(2, tile_c, masked, accA);
            }
            prev_c = tile_c;
            prev_masked = masked;
        };

        // One LDS buffer holds kTilesPerStage consecutive tiles; the next
        // buffer's loads are in flight while this one is multiplied.
        auto stage_tiles = [&](int it, uint16_t *buf) {
#pragma unroll
            for (int h = 0; h < kTilesPerStage; ++h)
                if (it + h < n_compute) stage(c_begin + (it + h) * kBN, buf + h * kTileElems);
        };
        // Stores issued after a buffer's loads: per slice one (scores, group
        // maxima) or four (candidates); 4 slices per tile.
        constexpr int kStoresPerSlice = kMode == kModeCandidates ? 4 : 1;
        constexpr int kStoresPerStage = 4 * kStoresPerSlice * kTilesPerStage;
        constexpr bool kFixedStores = kExact || kFused || kKeys;
        constexpr int kInFlight = kMode == kModeCandidates ? 16 : kStoresInFlight;
        static_assert(kInFlight <= kStoresPerStage && kInFlight <= 63, "vmcnt field");
        // s_waitcnt vmcnt(kInFlight) lgkmcnt(0) (vmcnt split over bits 3:0 and 15:14).
        constexpr int kStageWait = ((kInFlight >> 4) << 14) | 0x0070 | (kInFlight & 15);
        auto run_stage = [&](int it, const uint16_t *cur_buf, uint16_t *next_buf) {
            // The buffer is in LDS once every wave's loads for it have
            // landed.  Vector-memory ops complete in issue order, and the
            // previous stage issued exactly kStoresPerStage stores after
            // them, so up to that many may stay in flight.
            if (kFixedStores) __builtin_amdgcn_s_waitcnt(kStageWait);
            else __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // The first tile's key fragments are read before the next
            // buffer's loads are issued.
            u32x4 b0[4][4];
            load_b(cur_buf, b0);
            if (it + kTilesPerStage < n_compute) stage_tiles(it + kTilesPerStage, next_buf);
#pragma unroll
            for (int h = 0; h < kTilesPerStage; ++h) {
                if (h == 0) {
                    do_tile(c_begin + it * kBN, b0);
                } else if (it + h < n_compute) {
                    u32x4 b[4][4];
                    load_b(cur_buf + h * kTileElems, b);
                    do_tile(c_begin + (it + h) * kBN, b);
                } else if (kExact) {
                    // Keep the store count of a stage fixed (dropped stores).
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        __builtin_amdgcn_raw_buffer_store_b128(f32x4{0.f, 0.f, 0.f, 0.f}, out_rsrc, kDropped, 0, 0);
                } else if (kKeys) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, out_rsrc, kDropped, 0, 0);
                } else if (kFused) {
#pragma unroll
                    for (int i = 0; i < 4 * kStoresPerSlice; ++i) {
                        if (kMode == kModeGroupMax) __builtin_amdgcn_raw_buffer_store_b32(0u, fused_rsrc, kDropped, 0, 0);
                        else __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, fused_rsrc, kDropped, 0, 0);
                    }
                }
            }
        };

        if (n_compute > 0) {
            stage_tiles(0, ktile0);
            __builtin_amdgcn_s_waitcnt(0);
        }
        for (int it = 0; it < n_compute; it += 2 * kTilesPerStage) {
            run_stage(it, ktile0, ktile1);
            if (it + kTilesPerStage < n_compute) run_stage(it + kTilesPerStage, ktile1, ktile0);
        }
        if (prev_c >= 0) {
            if (kFused) finish_topk(3, prev_c, prev_masked, accB);
            else finish_general(3, prev_c, prev_masked, accB);
        }
        if (kRotate && n_compute > 0 && lo) {
            // The last segment's end: columns end - 4*rot .. end - 1 of the
            // last computed tile, held by lanes n < rot.
            const int cs = c_begin + n_compute * kBN + sc;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (in_pass[mt] && cs < c_end)
                    store4(out_wg + row_elem(mt, cs), true, cs, c_end, keep[mt][0], keep[mt][1], keep[mt][2], keep[mt][3]);
        }
        if (kMode == kModeCandidates) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (n == 0 && in_pass[mt])
                    p.cand_cnt[(int64_t)(row0 + a_w + dl * (4 * mt + q4)) * p.col_chunks + cc] = c_ncand[mt];
        }
        if (kMode == kModeGroupMax) {
            // Close the group the last computed tile left open, and give the
            // chunk's groups past the last visible key -inf.
            constexpr int kGroupCols = kGroupTiles * kBN;
            int g_next = c_begin / kGroupCols;
            if (n_compute > 0) {
                const int last = c_begin / kBN + n_compute - 1;  // global tile index
                const bool closed = last % kGroupTiles == kGroupTiles - 1 || (last + 1) * kBN >= c_end;
                g_next = last / kGroupTiles + 1;
                if (!closed) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const int row = row0 + a_w + dl * (4 * mt + q4);
                        if (in_pass[mt]) p.gmax[(int64_t)row * p.gmax_stride + (last / kGroupTiles) * 16 + n] = gm[mt];
                    }
                }
            }
            const int g_end = (c_end + kGroupCols - 1) / kGroupCols;
            for (int gi = g_next; gi < g_end; ++gi) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int row = row0 + a_w + dl * (4 * mt + q4);
                    if (in_pass[mt]) p.gmax[(int64_t)row * p.gmax_stride + gi * 16 + n] = neg_inf();
                }
            }
        }

        // Tiles that no row of this pass can see: -inf only (score modes),
        // key 0 (key mode, whole tiles).
        for (int it = n_compute; kKeys && it < n_tiles; ++it) {
            const int col = c_begin + it * kBN + 4 * n;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (in_pass[mt])
                    *reinterpret_cast<u32x2 *>(p.keys16 + (int64_t)(row0 + a_w + dl * (4 * mt + q4)) * p.keys_stride + col) =
                        u32x2{0u, 0u};
        }
        const float ni = neg_inf();
        for (int it = n_compute; !kFused && !kKeys && it < n_tiles; ++it) {
            const int tile_c = c_begin + it * kBN;
            const int col = tile_c + 4 * n;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (in_pass[mt]) store4(out_wg + row_elem(mt, col), p.out_vec, col, c_end, ni, ni, ni, ni);
        }

        __syncthreads();
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i] && s_start[i] == cur) s_done[i] = 1;
    }
}

}  // namespace

int prefill_col_chunk(int64_t num_rows, int32_t out_cols, int64_t k_stride, int num_cus) {
    // One round of workgroups (one per CU), each walking a long run of
    // columns: the per-workgroup setup is paid once, and each workgroup's
    // stores cover long stretches of its rows.
    const int64_t row_blocks = (num_rows + kBM - 1) / kBM;
    const int64_t tiles = ((int64_t)out_cols + kBN - 1) / kBN;
    const int64_t target_groups = (int64_t)(num_cus > 0 ? num_cus : 256);
    int64_t per_chunk = (tiles * row_blocks + target_groups - 1) / target_groups;
    if (per_chunk < 8) per_chunk = 8;
    // Key offsets inside a chunk's buffer resource are 32-bit: keep a
    // chunk's keys (plus one tile) within 2^30 bytes.
    const int64_t max_chunk = ((int64_t)1 << 30) / (kBN * k_stride * 2) - 1;
    if (per_chunk > max_chunk) per_chunk = max_chunk;
    if (per_chunk > tiles) per_chunk = tiles;
    if (per_chunk < 1) per_chunk = 1;
    return (int)(per_chunk * kBN);
}

int64_t prefill_max_k_stride() { return ((int64_t)1 << 30) / (2 * kBN * 2); }

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    if (p.f16) {
        if (p.exact_stores && p.rotate)
            return launch_kernel(prefill_kernel<kModeScoresExact, true, true>, grid, dim3(kThreads), stream, p);
        if (p.exact_stores)
            return launch_kernel(prefill_kernel<kModeScoresExact, true, false>, grid, dim3(kThreads), stream, p);
        return launch_kernel(prefill_kernel<kModeScores, true, false>, grid, dim3(kThreads), stream, p);
    }
    if (p.exact_stores && p.rotate)
        return launch_kernel(prefill_kernel<kModeScoresExact, false, true>, grid, dim3(kThreads), stream, p);
    if (p.exact_stores)
        return launch_kernel(prefill_kernel<kModeScoresExact, false, false>, grid, dim3(kThreads), stream, p);
    return launch_kernel(prefill_kernel<kModeScores, false, false>, grid, dim3(kThreads), stream, p);
}

hipError_t launch_prefill_group_max(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    return launch_kernel(prefill_kernel<kModeGroupMax, false, false>, grid, dim3(kThreads), stream, p);
}

hipError_t launch_prefill_candidates(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    return launch_kernel(prefill_kernel<kModeCandidates, false, false>, grid, dim3(kThreads), stream, p);
}

hipError_t launch_prefill_keys16(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    if (p.f16) return launch_kernel(prefill_kernel<kModeKeys16, true, false>, grid, dim3(kThreads), stream, p);
    return launch_kernel(prefill_kernel<kModeKeys16, false, false>, grid, dim3(kThreads), stream, p);
}

int prefill_rows_per_block() { return kBM; }

}  // namespace qsa
