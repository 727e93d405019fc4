// Step 2: block scores of the MQA indexer (Qwen3.8-Flash-Next model card,
// "Model Overview": indexer = MQA with 4 query heads and 1 shared key head
// of dim 128; blog "Attention: GDN + QSA": importance is estimated per block).
//
//   s[t][j] = sum_{h<4} sum_{d<128} q_idx[t][h][d] * kbar[j][d],   j < (q_pos0 + t) / 4
//
// A dense bf16 contraction on the matrix cores with the head sum folded into
// K (index_common.h): per 16 blocks x 16 tokens, one chain of 16
// v_mfma_f32_16x16x32_bf16 gives finished scores, 4 consecutive blocks of one
// token per lane.  Every launch shape computes a given score with the same
// instruction sequence, so scores do not depend on tiling.
//
// A workgroup of 4 waves owns 64 query rows (16 per wave, whose B operands
// stay in registers) and a chunk of block columns.  Each step the workgroup
// stages 64 blocks (16 KiB) of kbar in LDS -- LDS-direct loads issued two
// steps ahead into three buffers -- and every wave reads its A operands from
// there, so each kbar byte crosses the vector memory path once per 64 rows.
// A wave stores 4 float4 per lane per step (16 rows x 256 bytes).
// Causality: the workgroup stops at the last block its last row sees.
#include "index_common.h"

namespace qsa {

constexpr int kTokTile = 16;    // query rows per wave
constexpr int kWgTok = 64;      // query rows per workgroup
constexpr int kColStep = 64;    // blocks per step

// One step of kbar in LDS: block jb of the step is row jb (256 bytes); the
// 16-byte chunk c of row r is stored at position c ^ (r % 16), so the 16
// lanes reading one k-slice of a 16-block tile touch 16 distinct positions,
// i.e. every bank once.
struct KTile {
    uint4 chunk[kColStep][16];
};

// The three step buffers are separate LDS objects.
__shared__ KTile tA, tB, tC;

// Stages one step of kbar into t with LDS-direct loads (no registers): wave
// w fills rows 16w .. 16w + 15 with 4 loads of 1 KiB; lane L of load i
// writes row 16w + 4i + L / 16 at position L % 16.  Blocks at or past j_end
// read block j_end - 1 (never stored as a score).
//
// The load is issued from inline assembly: with the compiler's LDS-DMA
// intrinsic, its wait-count pass assumes every LDS read may depend on every
// staged load in flight and waits for all vector memory, stores included,
// before each step, which serialises the score stores with the next step.
// The instruction has no register results (it writes LDS only, and its
// address registers are read at issue); completion is tracked explicitly by
// step_sync's vmcnt waits.
__device__ __forceinline__ void stage_dma(const uint16_t* kb, int j0, int j_end, KTile& t) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int j = min(j0 + r, j_end - 1);
        const uint16_t* src = kb + static_cast<int64_t>(j) * kDi + 8 * c;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&t.chunk[16 * wave + 4 * i][0])));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
#pragma clang diagnostic pop
    }
}

// Wait until this wave's loads of step s have landed, then meet the other
// waves.  Vector memory ops complete in issue order; after the 4 loads of
// step s a wave with rows issues 4 score stores per scored step and the 4
// loads of step s + 1, so at most that many may stay in flight.  A wave
// without rows (at most three per launch, in the last row tile) waits for all.
__device__ __forceinline__ void step_sync(int s, bool has_rows) {
    if (!has_rows) __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0)
    else if (s == 0) __builtin_amdgcn_s_waitcnt(0x0f74);   // vmcnt(4)
    else if (s == 1) __builtin_amdgcn_s_waitcnt(0x0f78);   // vmcnt(8)
    else __builtin_amdgcn_s_waitcnt(0x0f7c);               // vmcnt(12)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scores of one staged step (4 tiles of 16 blocks) for the wave's 16 rows.
__device__ __forceinline__ void score_step(const KTile& t, const bf16x8_t (&qf)[16], int j0, int j_end,
                                           int t0, int tq, float* sb, int64_t ld) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    f32x4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        bf16x8_t kf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = t.chunk[16 * nt + c16][(4 * q + G) ^ c16];
            kf[q] = *reinterpret_cast<const bf16x8_t*>(&v);
        }
        acc[nt] = block_scores(kf, qf);
    }
    const int tok = t0 + c16;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int jj = j0 + 16 * nt + 4 * G;
        if (tok < tq && jj < j_end)        // streaming store: the scores are read back once, much later
            __builtin_nontemporal_store(acc[nt], reinterpret_cast<f32x4_t*>(sb + static_cast<int64_t>(tok) * ld + jj));
    }
}

__global__ __launch_bounds__(256) void index_scores_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos0, int tq, int n_wt, int n_cc, int cols_per_chunk, int64_t n_wg,
    float* __restrict__ scores, int64_t ld, int64_t ss) {
    // workgroups are dealt to the 8 XCDs round-robin; renumber them so each
    // XCD works through one contiguous range, and the row tiles that share a
    // column chunk of kbar share that XCD's L2
    const int64_t per_xcd = gridDim.x / 8;                // the grid is a multiple of 8
    const int64_t wg = static_cast<int64_t>(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (wg >= n_wg) return;                               // whole workgroup
    const int wt = static_cast<int>(wg % n_wt);
    const int64_t rest = wg / n_wt;
    const int cc = static_cast<int>(rest % n_cc);
    const int b = static_cast<int>(rest / n_cc);

    const int t_wg = wt * kWgTok;
    const int n_tok_wg = min(kWgTok, tq - t_wg);
    const int jmax = (pos0.p[b] + t_wg + n_tok_wg - 1) / kBlock;   // blocks the last row sees
    const int j_begin = cc * cols_per_chunk;
    const int j_end = min(j_begin + cols_per_chunk, jmax);
    if (j_begin >= j_end) return;                         // whole workgroup

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = t_wg + kTokTile * wave;
    const bool has_rows = t0 < tq;

    bf16x8_t qf[16];
    load_index_q(q_idx + b * qs, t0, tq, qf);
    __builtin_amdgcn_s_waitcnt(0x0f70);                   // B in registers before the load pipeline starts

    const uint16_t* kb = kbar + b * kbs;
    float* sb = scores + b * ss;
    const int n_steps = (j_end - j_begin + kColStep - 1) / kColStep;
    // three LDS buffers: step s is scored while steps s + 1 and s + 2 load
    stage_dma(kb, j_begin, j_end, tA);
    stage_dma(kb, j_begin + kColStep, j_end, tB);
    for (int s = 0; s < n_steps; s += 3) {
        step_sync(s, has_rows);
        stage_dma(kb, j_begin + kColStep * (s + 2), j_end, tC);
        if (has_rows) score_step(tA, qf, j_begin + kColStep * s, j_end, t0, tq, sb, ld);
        if (s + 1 >= n_steps) break;
        step_sync(s + 1, has_rows);
        stage_dma(kb, j_begin + kColStep * (s + 3), j_end, tA);
        if (has_rows) score_step(tB, qf, j_begin + kColStep * (s + 1), j_end, t0, tq, sb, ld);
        if (s + 2 >= n_steps) break;
        step_sync(s + 2, has_rows);
        stage_dma(kb, j_begin + kColStep * (s + 4), j_end, tB);
        if (has_rows) score_step(tC, qf, j_begin + kColStep * (s + 2), j_end, t0, tq, sb, ld);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);                   // no load into LDS outlives the workgroup
}

static void index_grid(const Positions& pos0, int batch, int tq, int* n_wt, int* n_cc, int* cols_per_chunk,
                       int64_t* n_wg) {
    int jmax = 0;
    for (int b = 0; b < batch; ++b) jmax = max(jmax, (pos0.p[b] + tq - 1) / kBlock);
    *n_wt = (tq + kWgTok - 1) / kWgTok;
    const int64_t steps = (jmax + kColStep - 1) / kColStep;
    // enough workgroups to fill 256 CUs several times over, at most 64 steps each
    const int64_t target_wgs = 4096;
    int64_t per = (static_cast<int64_t>(batch) * *n_wt * steps) / target_wgs;
    per = per < 1 ? 1 : (per > 64 ? 64 : per);
    *cols_per_chunk = static_cast<int>(per * kColStep);
    *n_cc = max(1, static_cast<int>((jmax + *cols_per_chunk - 1) / *cols_per_chunk));
    *n_wg = static_cast<int64_t>(batch) * *n_cc * *n_wt;
}

hipError_t launch_index_scores(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                               int64_t kbs, const Positions& pos0, int batch, int tq,
                               float* scores, int64_t ld, int64_t ss, hipStream_t stream) {
    if (tq <= 0) return hipSuccess;
    int n_wt, n_cc, cpc;
    int64_t n_wg;
    index_grid(pos0, batch, tq, &n_wt, &n_cc, &cpc, &n_wg);
    const unsigned grid = static_cast<unsigned>((n_wg + 7) / 8 * 8);
    hipLaunchKernelGGL(index_scores_kernel, dim3(grid), dim3(256), 0, stream, q_idx, qs, kbar, kbs,
                       pos0, tq, n_wt, n_cc, cpc, n_wg, scores, ld, ss);
    return hipGetLastError();
}

}  // namespace qsa
