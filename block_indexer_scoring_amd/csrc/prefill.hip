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
//   - A workgroup owns 64 query rows (16 per wavefront) and a chunk of
//     output columns.  Each wavefront keeps its 16 rows x 4 heads of Q in
//     registers as MFMA A fragments for the whole chunk (m = 4*row + head).
//   - Key tiles of 64 keys (16 KB) are staged in LDS, double-buffered: the
//     global loads of tile i+1 are in flight while tile i is multiplied.
//     LDS rows are XOR-swizzled in 16-byte units so the B-fragment reads are
//     free of bank conflicts.
//   - In the MFMA result a lane holds the 4 heads of one (row, key), so
//     ReLU, head sum, scale and the interval mask run in-lane; tile key
//     c + 4n + g sits in column n of group g, giving each lane 4
//     consecutive keys for one 16-byte non-temporal store.
//   - Tiles past the last key any row of the workgroup may see are not
//     multiplied: they are written as -inf only (causal tile skip).
// Rows of one workgroup normally share row_k_start (packed requests); rows
// with different starts are handled in one pass per distinct start.
#include <climits>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 64;                     // keys per LDS tile
constexpr int kTileElems = kBN * kDim;      // bf16 elements per tile

// LDS element offset of 16-byte chunk `chunk` (0..15) of tile key `key`.
__device__ __forceinline__ int lds_offset(int key, int chunk) {
    return key * kDim + ((chunk ^ ((key >> 2) & 15)) << 3);
}

__device__ __forceinline__ int clamp_cols(int64_t v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : (int)v);
}

__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ktile[2][kTileElems];
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

    if (tid < kBM) {
        const int t = row0 + tid;
        if (t < p.num_rows) {
            const int ks = p.row_k_start[t];
            const int ke = p.row_k_end[t];
            s_start[tid] = ks;
            s_end[tid] = (int64_t)ke < p.num_keys ? ke : (int)p.num_keys;
            s_done[tid] = 0;
        } else {
            s_start[tid] = 0;
            s_end[tid] = 0;
            s_done[tid] = 1;
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

    for (;;) {
        if (tid == 0) {
            s_cur = INT_MAX;
            s_lim = INT_MIN;
        }
        __syncthreads();
        if (tid < kBM && !s_done[tid]) atomicMin(&s_cur, s_start[tid]);
        __syncthreads();
        const int cur = s_cur;
        if (cur == INT_MAX) break;
        if (tid < kBM && !s_done[tid] && s_start[tid] == cur)
            atomicMax(&s_lim, clamp_cols((int64_t)s_end[tid] - cur, -1, INT_MAX - kBN));
        __syncthreads();
        const int lim = s_lim;  // columns >= lim hold no key for any row of this pass

        // This lane's output rows (MFMA result layout: row 4mt + q4).
        bool in_pass[4];
        int row_lim[4];
        int64_t out_row[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int idx = wave * kRowsPerWave + 4 * mt + q4;
            in_pass[mt] = !s_done[idx] && s_start[idx] == cur;
            row_lim[mt] = clamp_cols((int64_t)s_end[idx] - cur, -1, INT_MAX - kBN);
            out_row[mt] = (int64_t)(row0 + idx) * p.out_stride;
        }
        const int col_min = clamp_cols(-(int64_t)cur, 0, INT_MAX - kBN);  // key index >= 0

        int n_compute = 0;
        if (lim > c_begin) n_compute = min(n_tiles, (lim - c_begin + kBN - 1) / kBN);

        // Global -> register staging of one key tile: 64 keys x 16 chunks of
        // 16 bytes, 4 chunks per thread, consecutive threads on consecutive
        // 16-byte chunks.
        u32x4 stage[4];
        auto gload = [&](int tile_c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int piece = tid + kThreads * i;
                const int key = piece >> 4;
                const int chunk = piece & 15;
                const int64_t kn = (int64_t)cur + tile_c + key;
                stage[i] = (kn >= 0 && kn < p.num_keys)
                               ? load_u32x4(p.k + kn * p.k_stride + chunk * 8)
                               : zero_u32x4();
            }
        };
        auto swrite = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int piece = tid + kThreads * i;
                *reinterpret_cast<u32x4 *>(&ktile[buf][lds_offset(piece >> 4, piece & 15)]) = stage[i];
            }
        };

        if (n_compute > 0) {
            gload(c_begin);
            swrite(0);
        }
        __syncthreads();
        for (int it = 0; it < n_compute; ++it) {
            const int tile_c = c_begin + it * kBN;
            if (it + 1 < n_compute) gload(tile_c + kBN);

            const uint16_t *tile = ktile[it & 1];
            f32x4 acc[4][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(&tile[lds_offset(4 * n + g, 4 * ks + q4)]);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[mt][g] = mfma16x16x32(qa[mt][ks], b, acc[mt][g]);
                }
            }

            const int col = tile_c + 4 * n;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (!in_pass[mt]) continue;
                float v[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = col + g;
                    v[g] = (c < row_lim[mt] && c >= col_min) ? head_sum_score(acc[mt][g], p.scale) : neg_inf();
                }
                float *dst = p.out + out_row[mt] + col;
                if (p.out_vec && col + 3 < c_end) {
                    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(dst));
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if (col + g < c_end) dst[g] = v[g];
                }
            }

            if (it + 1 < n_compute) swrite((it + 1) & 1);
            __syncthreads();
        }

        // Tiles that no row of this pass can see: -inf only.
        for (int it = n_compute; it < n_tiles; ++it) {
            const int col = c_begin + it * kBN + 4 * n;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (!in_pass[mt]) continue;
                float *dst = p.out + out_row[mt] + col;
                if (p.out_vec && col + 3 < c_end) {
                    const float ni = neg_inf();
                    __builtin_nontemporal_store(f32x4{ni, ni, ni, ni}, reinterpret_cast<f32x4 *>(dst));
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if (col + g < c_end) dst[g] = neg_inf();
                }
            }
        }

        __syncthreads();
        if (tid < kBM && !s_done[tid] && s_start[tid] == cur) s_done[tid] = 1;
    }
}

}  // namespace

int prefill_col_chunk(int64_t num_rows, int32_t out_cols) {
    // Enough workgroups to fill 256 CUs several times over, in whole tiles.
    const int64_t row_blocks = (num_rows + kBM - 1) / kBM;
    const int64_t tiles = ((int64_t)out_cols + kBN - 1) / kBN;
    const int64_t target_groups = 2048;
    int64_t per_chunk = (tiles * row_blocks + target_groups - 1) / target_groups;
    if (per_chunk < 8) per_chunk = 8;
    if (per_chunk > tiles) per_chunk = tiles;
    if (per_chunk < 1) per_chunk = 1;
    return (int)(per_chunk * kBN);
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.row_blocks * p.col_chunks));
    hipLaunchKernelGGL(prefill_kernel, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

int prefill_rows_per_block() { return kBM; }

}  // namespace qsa
