// Step 2: block scores of the MQA indexer (Qwen3.8-Flash-Next model card,
// "Model Overview": indexer = MQA with 4 query heads and 1 shared key head
// of dim 128; blog "Attention: GDN + QSA": importance is estimated per block).
//
//   s[t][j] = sum_{h<4} sum_{d<128} q_idx[t][h][d] * kbar[j][d],   j < (q_pos0 + t) / 4
//
// A dense bf16 contraction on the matrix cores (v_mfma_f32_16x16x32_bf16):
//   A (16 x 32): rows are (token, head) pairs -- 4 tokens x 4 heads per tile,
//                which are 16 consecutive 256-byte rows of q_idx;
//   B (32 x 16): columns are blocks; column c of column tile n is block
//                j0 + 4c + n, so each lane ends with 4 consecutive blocks;
//   D (16 x 16): lane l holds rows 4*(l/16) + r, r < 4 -- the 4 heads of one
//                token -- for one block, so the head sum is an in-lane add.
// Products are exact in float32 and accumulate in float32; the head sum is
// ((h0 + h1) + h2) + h3.  Every launch shape computes a given score with
// the same instruction sequence, so scores do not depend on tiling.
//
// One wave owns 16 query rows (4 row tiles, A kept in registers) and a chunk
// of block columns, streaming 64 blocks (16 KiB of kbar) per step; each lane
// stores one float4 per row tile, and 16 lanes cover 256 contiguous bytes of
// a score row.  Causality: a wave stops at the last block its last row sees.
#include "index_common.h"

namespace qsa {

constexpr int kTokTile = 16;    // query rows per wave
constexpr int kColStep = 64;    // blocks per inner step

__global__ __launch_bounds__(256) void index_scores_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos0, int tq, int n_tt, int n_cc, int cols_per_chunk, int64_t n_items,
    float* __restrict__ scores, int64_t ld, int64_t ss) {
    const int lane = threadIdx.x & 63;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (item >= n_items) return;                         // wave-uniform
    const int tt = static_cast<int>(item % n_tt);
    const int64_t rest = item / n_tt;
    const int cc = static_cast<int>(rest % n_cc);
    const int b = static_cast<int>(rest / n_cc);

    const int t0 = tt * kTokTile;
    const int n_tok = min(kTokTile, tq - t0);
    const int jmax = (pos0.p[b] + t0 + n_tok - 1) / kBlock;   // blocks the tile's last row sees
    const int j_begin = cc * cols_per_chunk;
    const int j_end = min(j_begin + cols_per_chunk, jmax);
    if (j_begin >= j_end) return;

    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int m_tiles = (n_tok + 3) / 4;

    bf16x8_t a[4][4];
    const uint16_t* qb = q_idx + b * qs;
#pragma unroll
    for (int m = 0; m < 4; ++m) load_index_a(qb, t0 + 4 * m, tq, a[m]);

    const uint16_t* kb = kbar + b * kbs;
    float* sb = scores + b * ss;
    for (int j0 = j_begin; j0 < j_end; j0 += kColStep) {
        bf16x8_t bf[4][4];
#pragma unroll
        for (int n = 0; n < 4; ++n) load_index_b(kb, j0, n, j_end, bf[n]);
        const int jj = j0 + 4 * c16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m < m_tiles) {                               // wave-uniform
                float4 out;
                out.x = block_score(a[m], bf[0]);
                out.y = block_score(a[m], bf[1]);
                out.z = block_score(a[m], bf[2]);
                out.w = block_score(a[m], bf[3]);
                const int tok = t0 + 4 * m + G;
                if (tok < tq && jj < j_end)
                    *reinterpret_cast<float4*>(sb + static_cast<int64_t>(tok) * ld + jj) = out;
            }
        }
    }
}

hipError_t launch_index_scores(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                               int64_t kbs, const Positions& pos0, int batch, int tq,
                               float* scores, int64_t ld, int64_t ss, hipStream_t stream) {
    if (tq <= 0) return hipSuccess;
    int jmax = 0;
    for (int b = 0; b < batch; ++b) jmax = max(jmax, (pos0.p[b] + tq - 1) / kBlock);
    if (jmax <= 0) return hipSuccess;
    const int n_tt = (tq + kTokTile - 1) / kTokTile;
    const int64_t steps = (jmax + kColStep - 1) / kColStep;
    // enough waves to fill 256 CUs several times over, at most 64 steps per wave
    const int64_t target_waves = 16384;
    int64_t per = (static_cast<int64_t>(batch) * n_tt * steps) / target_waves;
    per = per < 1 ? 1 : (per > 64 ? 64 : per);
    const int cols_per_chunk = static_cast<int>(per * kColStep);
    const int n_cc = static_cast<int>((jmax + cols_per_chunk - 1) / cols_per_chunk);
    const int64_t n_items = static_cast<int64_t>(batch) * n_cc * n_tt;
    const unsigned grid = static_cast<unsigned>((n_items + 3) / 4);
    hipLaunchKernelGGL(index_scores_kernel, dim3(grid), dim3(256), 0, stream, q_idx, qs, kbar, kbs,
                       pos0, tq, n_tt, n_cc, cols_per_chunk, n_items, scores, ld, ss);
    return hipGetLastError();
}

}  // namespace qsa
