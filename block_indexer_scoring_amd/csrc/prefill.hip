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
//   - A workgroup owns kBM query rows (16 per wavefront) and a chunk of
//     output columns.  Each wavefront keeps its 16 rows x 4 heads of Q in
//     registers as MFMA A fragments for the whole chunk (m = 4*row + head).
//   - Key tiles of 64 keys (16 KB) are staged in LDS with direct
//     global-to-LDS loads, two tiles per buffer and two buffers: the loads
//     of the next pair are in flight while the current pair is multiplied
//     (one workgroup barrier per 128 keys), and every wave of the workgroup
//     reuses each staged tile.  LDS rows are XOR-swizzled in 16-byte units
//     so the B-fragment reads are free of bank conflicts.
//   - Registers are held to two wavefronts per SIMD, so one wave's epilogue
//     and stores overlap the other's MFMAs.
//   - In the MFMA result a lane holds the 4 heads of one (row, key), so
//     ReLU, head sum and scale run in-lane; tile key c + 4n + g sits in
//     column n of group g, giving each lane 4 consecutive keys for one
//     16-byte store.  Only tiles that cross a row's interval end (or start)
//     evaluate the mask.  The output (4 bytes per cell, the bulk of the
//     traffic) goes out with ordinary cached stores: on this GPU they write
//     the tiled pattern markedly faster than non-temporal stores.
//   - Tiles past the last key any row of the workgroup may see are not
//     multiplied: they are written as -inf only (causal tile skip).
// Rows of one workgroup normally share row_k_start (packed requests); rows
// with different starts are handled in one pass per distinct start.
#include <climits>

#include "qsa_device.h"
#include "qsa_internal.h"

#ifndef QSA_PREFILL_WAVES
#define QSA_PREFILL_WAVES 4
#endif
#ifndef QSA_PREFILL_TILES_PER_STAGE
#define QSA_PREFILL_TILES_PER_STAGE 2
#endif

namespace qsa {
namespace {

constexpr int kWaves = QSA_PREFILL_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 64;                     // keys per LDS tile
constexpr int kTileElems = kBN * kDim;      // bf16 elements per tile
constexpr int kBlocksPerWave = kBN / 4 / kWaves;  // 1 KB LDS blocks staged per wave per tile
constexpr int kTilesPerStage = QSA_PREFILL_TILES_PER_STAGE;  // key tiles per LDS buffer

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

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillParams p) {
    // Two separate LDS objects (not one [2][...] array), so the compiler can
    // tell the buffer being read from the one being filled and does not wait
    // for the prefetch before reading the current tile.
    __shared__ __attribute__((aligned(16))) uint16_t ktile0[kTilesPerStage * kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t ktile1[kTilesPerStage * kTileElems];
    __shared__ int s_start[kBM];
    __shared__ int s_end[kBM];  // min(row_k_end, num_keys)
    __shared__ int s_done[kBM];
    __shared__ int s_cur, s_lim;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const int rb = blockIdx.x % p.row_blocks;
    const int cc = blockIdx.x / p.row_blocks;
    const int row0 = rb * kBM;
    const int c_begin = cc * p.col_chunk;
    const int c_end = min(c_begin + p.col_chunk, p.out_cols);
    const int n_tiles = (c_end - c_begin + kBN - 1) / kBN;

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
        const int t = row0 + wave * kRowsPerWave + 4 * mt + (n >> 2);
        const uint16_t *src = p.q + (int64_t)t * p.q_stride_row + (int64_t)(n & 3) * p.q_stride_head + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qa[mt][ks] = t < p.num_rows ? load_u32x4(src + 32 * ks) : zero_u32x4();
    }
    // Complete the Q loads here, so that no wait inside the tile loop has to
    // cover them (the loop's only vector-memory loads are the key prefetch).
    __builtin_amdgcn_s_waitcnt(0);

    // Key staging goes straight from global memory to LDS
    // (global_load_lds_dwordx4): one instruction moves 1 KB, lane l writing
    // bytes 16l .. 16l+15 of the block.  Block b of a tile holds keys
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
    // B-fragment read offsets: key 4n + g, chunk 4ks + q4; g adds 128 elements.
    int rd_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rd_off[ks] = lds_offset(4 * n, 4 * ks + q4);

    for (;;) {
        if (tid == 0) {
            s_cur = INT_MAX;
            s_lim = INT_MIN;
        }
        __syncthreads();
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i]) atomicMin(&s_cur, s_start[i]);
        __syncthreads();
        const int cur = s_cur;
        if (cur == INT_MAX) break;
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i] && s_start[i] == cur)
                atomicMax(&s_lim, clamp_cols((int64_t)s_end[i] - cur, -1, INT_MAX - kBN));
        __syncthreads();
        const int lim = s_lim;  // columns >= lim hold no key for any row of this pass

        // This lane's output rows (MFMA result layout: row 4mt + q4).
        bool in_pass[4];
        int row_lim[4];
        float *row_ptr[4];
        int lane_min_lim = INT_MAX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int idx = wave * kRowsPerWave + 4 * mt + q4;
            in_pass[mt] = !s_done[idx] && s_start[idx] == cur;
            row_lim[mt] = clamp_cols((int64_t)s_end[idx] - cur, -1, INT_MAX - kBN);
            row_ptr[mt] = p.out + (int64_t)(row0 + idx) * p.out_stride + 4 * n;
            if (in_pass[mt]) lane_min_lim = min(lane_min_lim, row_lim[mt]);
        }
        // Tiles inside [col_min, wave_lim) need no mask for any row of this wave.
        const int wave_lim = wave_min(lane_min_lim);
        const int col_min = clamp_cols(-(int64_t)cur, 0, INT_MAX - kBN);  // key index >= 0

        int n_compute = 0;
        if (lim > c_begin) n_compute = min(n_tiles, (lim - c_begin + kBN - 1) / kBN);

        // Stage one key tile (64 keys x 256 bytes) into LDS buffer `buf`: a
        // uniform base plus per-lane constant offsets; a tile that reaches
        // past either end of the keys is zero-filled and loaded per key.
        auto stage = [&](int tile_c, uint16_t *buf) {
            const int64_t first = (int64_t)cur + tile_c;
            if (first >= 0 && first + kBN <= p.num_keys) {
                const char *base = reinterpret_cast<const char *>(p.k + first * p.k_stride);
#pragma unroll
                for (int i = 0; i < kBlocksPerWave; ++i) {
                    const int b = wave * kBlocksPerWave + i;
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)(base + st_goff[i]),
                        (__attribute__((address_space(3))) void *)&buf[b * 512], 16, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kBlocksPerWave; ++i) {
                    const int b = wave * kBlocksPerWave + i;
                    const int key = 4 * b + (lane >> 4);
                    const int chunk = (lane & 15) ^ (b & 15);
                    const int64_t kn = first + key;
                    const u32x4 v = (kn >= 0 && kn < p.num_keys) ? load_u32x4(p.k + kn * p.k_stride + chunk * 8)
                                                                 : zero_u32x4();
                    *reinterpret_cast<u32x4 *>(&buf[b * 512 + lane * 8]) = v;
                }
            }
        };

        // Scores of the previous tile wait in registers and are stored at the
        // start of the next iteration, before its key prefetch is issued:
        // stores count in the same in-order vector-memory counter as loads,
        // so the wait for the prefetch then only covers stores that have
        // had a whole tile of MFMA time to drain.
        f32x4 pend[4];
        int pend_c = -1;  // tile column of the pending scores, -1 if none
        // The workgroup's output rows as one raw buffer.  A full tile's
        // scores go out as exactly four buffer stores per wave: lanes whose
        // row is not in this pass store to an offset past the buffer's end,
        // which the hardware drops.  With that fixed count, the wait before
        // a buffer of keys can leave the most recent tile's stores in flight.
        const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            p.out + (int64_t)row0 * p.out_stride, 0,
            p.exact_stores ? (int)((int64_t)min(kBM, p.num_rows - row0) * p.out_stride * 4) : 0, kBufferWord3);
        uint32_t row_boff[4];  // byte offset of (row, column 4n) in out_rsrc
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int idx = wave * kRowsPerWave + 4 * mt + q4;
            row_boff[mt] = in_pass[mt] ? (uint32_t)(((int64_t)idx * p.out_stride + 4 * n) * 4) : 0x80000000u;
        }
        auto flush = [&]() {
            if (pend_c < 0) return;
            const int col = pend_c + 4 * n;
            const bool full = p.out_vec && pend_c + kBN <= c_end;
            if (full && p.exact_stores) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    __builtin_amdgcn_raw_buffer_store_b128(pend[mt], out_rsrc, row_boff[mt] + 4u * (uint32_t)pend_c,
                                                           0, 0);
                pend_c = -1;
                return;
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (!in_pass[mt]) continue;
                if (full)
                    *reinterpret_cast<f32x4 *>(row_ptr[mt] + pend_c) = pend[mt];
                else
                    store4(row_ptr[mt] + pend_c, p.out_vec, col, c_end, pend[mt][0], pend[mt][1], pend[mt][2],
                           pend[mt][3]);
            }
            pend_c = -1;
        };

        auto compute_tile = [&](int tile_c, const uint16_t *tile) {
            f32x4 acc[4][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(&tile[rd_off[ks] + g * kDim]);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[mt][g] = mfma16x16x32(qa[mt][ks], b, acc[mt][g]);
                }
            }

            const bool masked = !(tile_c + kBN <= wave_lim && tile_c >= col_min);
            if (!masked) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    pend[mt] = f32x4{head_sum_score(acc[mt][0], p.scale), head_sum_score(acc[mt][1], p.scale),
                                     head_sum_score(acc[mt][2], p.scale), head_sum_score(acc[mt][3], p.scale)};
            } else {
                const int col = tile_c + 4 * n;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c = col + g;
                        pend[mt][g] = (c < row_lim[mt] && c >= col_min) ? head_sum_score(acc[mt][g], p.scale)
                                                                        : neg_inf();
                    }
            }
            pend_c = tile_c;
        };

        // One LDS buffer holds kTilesPerStage consecutive tiles; the next
        // buffer's loads are in flight while this one is multiplied.
        auto stage_tiles = [&](int it, uint16_t *buf) {
#pragma unroll
            for (int h = 0; h < kTilesPerStage; ++h)
                if (it + h < n_compute) stage(c_begin + (it + h) * kBN, buf + h * kTileElems);
        };
        auto run_stage = [&](int it, const uint16_t *cur_buf, uint16_t *next_buf) {
            // The buffer is in LDS once every wave's loads for it have landed.
            // Vector-memory ops complete in issue order; from the third
            // stage on, the only ops issued after this buffer's loads are
            // the four stores of the previous stage's first tile, which may
            // stay in flight (s_waitcnt vmcnt(4) lgkmcnt(0)).
            if (p.exact_stores && it >= 2 * kTilesPerStage) __builtin_amdgcn_s_waitcnt(0x0074);
            else __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            flush();
            if (it + kTilesPerStage < n_compute) stage_tiles(it + kTilesPerStage, next_buf);
#pragma unroll
            for (int h = 0; h < kTilesPerStage; ++h) {
                if (it + h < n_compute) {
                    if (h > 0) flush();
                    compute_tile(c_begin + (it + h) * kBN, cur_buf + h * kTileElems);
                }
            }
        };

        if (n_compute > 0) stage_tiles(0, ktile0);
        for (int it = 0; it < n_compute; it += 2 * kTilesPerStage) {
            run_stage(it, ktile0, ktile1);
            if (it + kTilesPerStage < n_compute) run_stage(it + kTilesPerStage, ktile1, ktile0);
        }
        flush();

        // Tiles that no row of this pass can see: -inf only.
        const float ni = neg_inf();
        for (int it = n_compute; it < n_tiles; ++it) {
            const int tile_c = c_begin + it * kBN;
            const int col = tile_c + 4 * n;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (in_pass[mt]) store4(row_ptr[mt] + tile_c, p.out_vec, col, c_end, ni, ni, ni, ni);
        }

        __syncthreads();
        for (int i = tid; i < kBM; i += kThreads)
            if (!s_done[i] && s_start[i] == cur) s_done[i] = 1;
    }
}

}  // namespace

int prefill_col_chunk(int64_t num_rows, int32_t out_cols, int num_cus) {
    // One round of workgroups (two per CU), each walking a long run of
    // columns: the per-workgroup setup is paid once, and each workgroup's
    // stores cover long stretches of its rows.
    const int64_t row_blocks = (num_rows + kBM - 1) / kBM;
    const int64_t tiles = ((int64_t)out_cols + kBN - 1) / kBN;
    const int64_t target_groups = 2 * (int64_t)(num_cus > 0 ? num_cus : 256);
    int64_t per_chunk = (tiles * row_blocks + target_groups - 1) / target_groups;
    if (per_chunk < 8) per_chunk = 8;
    if (per_chunk > tiles) per_chunk = tiles;
    if (per_chunk < 1) per_chunk = 1;
    return (int)(per_chunk * kBN);
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    return launch_kernel(prefill_kernel, grid, dim3(kThreads), stream, p);
}

int prefill_rows_per_block() { return kBM; }

}  // namespace qsa
