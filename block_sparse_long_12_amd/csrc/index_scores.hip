// Step 2: block scores of the MQA indexer (Qwen3.8-Flash-Next model card,
// "Model Overview": indexer = MQA with 4 query heads and 1 shared key head
// of dim 128; blog "Attention: GDN + QSA": importance is estimated per block).
//
//   s[t][j] = sum_{h<4} sum_{d<128} q_idx[t][h][d] * kbar[j][d],   j < (q_pos0 + t) / 4
//
// A dense bf16 contraction on the matrix cores with the head sum taken on
// the query side and split into three exact bf16 terms (index_common.h): per
// 16 blocks x 16 tokens, one chain of 12 v_mfma_f32_16x16x32_bf16 gives
// finished scores, 4 consecutive blocks of one token per lane.  Every launch shape and mode computes a given score with
// the same instruction sequence, so scores do not depend on tiling.
//
// A workgroup of 4 waves owns 64 query rows (16 per wave, whose B operands
// stay in registers) and a chunk of block columns.  Each step the workgroup
// stages 64 blocks (16 KiB) of kbar in LDS with LDS-direct loads and every
// wave reads its A operands from there, so each kbar byte crosses the vector
// memory path once per 64 rows.  Three modes share the machinery:
//   scores  -- store every score (4 float4 per lane per step), three LDS
//              buffers so loads run two steps ahead of the stores;
//   sample  -- the same over a fixed sample of blocks (256 evenly spread
//              runs of 16), stored compactly; feeds the per-row thresholds;
//   collect -- no score matrix: scores at or above the row's threshold are
//              appended to per-wave LDS lists and, at the end, to the row's
//              global candidate list (one atomic per row and workgroup) as
//              (ordered key, ~block) pairs.  A workgroup whose LDS lists
//              overflow (candidates dense in a stretch of blocks: high scores
//              that cluster) hands nothing off and marks itself;
//   collect retry -- run after collect with the same grid: only the marked
//              workgroups score their blocks again, and a candidate that finds
//              its wave's list full goes straight to its row's global list.
// Causality: a workgroup stops at the last block its last row sees; collect
// also drops each row's blocks at or past its own block.
#include "index_common.h"
#include "select_common.h"

namespace qsa {

constexpr int kTokTile = 16;    // query rows per wave
constexpr int kWgTok = 64;      // query rows per workgroup
constexpr int kColStep = 64;    // blocks per step

enum { kModeScores = 0, kModeSample = 1, kModeCollect = 2, kModeCollectRetry = 3 };

// One step of kbar in LDS: block jb of the step is row jb (256 bytes); the
// 16-byte chunk c of row r is stored at position c ^ (r % 16), so the 16
// lanes reading one k-slice of a 16-block tile touch 16 distinct positions,
// i.e. every bank once.
struct KTile {
    uint4 chunk[kColStep][16];
};

// The step buffers are separate LDS objects; collect uses two of them plus
// the candidate list.
__shared__ KTile tA, tB, tC;
__shared__ uint64_t lcand[kCollectCap];
__shared__ int lrow[kWgTok];
__shared__ int lrow_base[kWgTok];
__shared__ int lwcnt[4];

// Block of column jv: itself, or in sample mode run jv / 16 of kSampleRuns
// runs of 16 blocks spread evenly over [0, omin) (with paged block keys each
// run starts on a multiple of 16 blocks, so the run's tile stays inside one
// page).  Short runs spread wide keep the sample representative when high
// scores cluster in a stretch of blocks (a run of 256 inside such a stretch
// over-weighted it 16-fold).
template <int kMode, bool kPaged = false>
__device__ __forceinline__ int column_block(int jv, int omin) {
    if (kMode == kModeSample) {
        const int run = jv / kSampleRunLen;
        int base = static_cast<int>(static_cast<int64_t>(run) * (omin - kSampleRunLen) / (kSampleRuns - 1));
        if (kPaged) base &= ~15;
        return base + jv % kSampleRunLen;
    }
    return jv;
}

// Paged block keys: the sequence's block-table row and the page geometry.
struct KbPages {
    const int32_t* tbl;
    int shift;          // log2 of tokens per page
    int n_pages;
};

// Stages one step of kbar into t with LDS-direct loads (no registers): wave
// w fills rows 16w .. 16w + 15 with 4 loads of 1 KiB; lane L of load i
// writes row 16w + 4i + L / 16 at position L % 16.  Columns at or past j_end
// read column j_end - 1 (never stored or collected).
//
// The load is issued from inline assembly: with the compiler's LDS-DMA
// intrinsic, its wait-count pass assumes every LDS read may depend on every
// staged load in flight and waits for all vector memory, stores included,
// before each step, which serialises the score stores with the next step.
// The instruction has no register results (it writes LDS only, and its
// address registers are read at issue); completion is tracked explicitly by
// the vmcnt waits of the step loop.
// Byte offset of lane L's 16-byte chunk for load i of a step, from the
// step's first row (see stage_dma).
struct DmaOffsets {
    uint32_t off[4];
};

__device__ __forceinline__ DmaOffsets dma_offsets() {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    DmaOffsets d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        d.off[i] = static_cast<uint32_t>((r * kDi + 8 * c) * 2);
    }
    return d;
}

template <int kMode, bool kPaged = false>
__device__ __forceinline__ void stage_dma(const uint16_t* kb, int j0, int j_end, int omin, const KbPages& kp,
                                          const DmaOffsets& d, KTile& t) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (kMode != kModeSample) {
        // a step wholly below j_end needs no clamp: the step's rows start at
        // a scalar base and each lane's byte offset from it is fixed, so the
        // loads take the scalar-base form and cost no vector address
        // arithmetic.  Paged, the base is the wave's first row: its 16 rows
        // are one 16-aligned run inside one page (pages hold >= 16 blocks).
        if (j0 + kColStep <= j_end) {
            const uint16_t* base;
            uint32_t sub = 0;
            if constexpr (kPaged) {
                const int jw = j0 + 16 * wave;
                const int pg = __builtin_amdgcn_readfirstlane(min(max(kp.tbl[(jw * kBlock) >> kp.shift], 0), kp.n_pages - 1));
                const int64_t row0 = (static_cast<int64_t>(pg) << (kp.shift - 2)) | (jw & ((1 << (kp.shift - 2)) - 1));
                base = kb + row0 * kDi;
                sub = static_cast<uint32_t>(16 * wave * kDi * 2);
            } else {
                base = kb + static_cast<int64_t>(j0) * kDi;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = d.off[i] - sub;
                const uint32_t lds = __builtin_amdgcn_readfirstlane(
                    static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&t.chunk[16 * wave + 4 * i][0])));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                             : "memory", "m0");
#pragma clang diagnostic pop
            }
            return;
        }
    }
    // paged: the wave's 16 rows form one 16-block tile (the step start is a
    // multiple of 64, sample runs start on multiples of 16, and clamped rows
    // fall in the tile of j_end - 1), so one wave-uniform table read serves
    // them all
    int64_t page_base = 0;
    if constexpr (kPaged) {
        const int jr = column_block<kMode, true>(min(j0 + 16 * wave, j_end - 1), omin);
        const int pg = min(max(kp.tbl[(jr * kBlock) >> kp.shift], 0), kp.n_pages - 1);
        page_base = static_cast<int64_t>(pg) << (kp.shift - 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int j = column_block<kMode, kPaged>(min(j0 + r, j_end - 1), omin);
        const int64_t row = kPaged ? (page_base | (j & ((1 << (kp.shift - 2)) - 1))) : static_cast<int64_t>(j);
        const uint16_t* src = kb + row * kDi + 8 * c;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&t.chunk[16 * wave + 4 * i][0])));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
#pragma clang diagnostic pop
    }
}

// Waits for this wave's vector memory ops until at most N are in flight,
// then meets the other waves.
template <int N>
__device__ __forceinline__ void wait_and_meet() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | N);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// scores / sample: wait until this wave's loads of step s have landed.
// Vector memory ops complete in issue order; after the 4 loads of step s a
// wave with rows issues 4 score stores per scored step and the 4 loads of
// step s + 1, so at most that many may stay in flight.  A wave without rows
// (only in the last row tile) waits for all.
__device__ __forceinline__ void step_sync(int s, bool has_rows) {
    if (!has_rows) wait_and_meet<0>();
    else if (s == 0) wait_and_meet<4>();
    else if (s == 1) wait_and_meet<8>();
    else wait_and_meet<12>();
}

// Scores of one staged step (4 tiles of 16 blocks) for the wave's 16 rows:
// lane l ends with blocks j0 + 16 nt + 4 (l / 16) .. + 3 of token l % 16.
template <int kTilesLive = 4>
__device__ __forceinline__ void step_scores(const KTile& t, const bf16x8_t (&qf)[kIdxSlices], f32x4_t (&acc)[4]) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    if constexpr (kTilesLive == 4) {
        bf16x8_t kf[4][4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = t.chunk[16 * nt + c16][(4 * q + G) ^ c16];
                kf[nt][q] = *reinterpret_cast<const bf16x8_t*>(&v);
            }
        block_scores4(kf, qf, acc);
    } else {
        // one 16-block tile at a time: 16 operand registers live instead of
        // 64, so more waves fit on a SIMD
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
    }
}

__device__ __forceinline__ void store_step(const KTile& t, const bf16x8_t (&qf)[kIdxSlices], int j0, int j_end, int t0,
                                           int tq, float* sb, int64_t ld) {
    f32x4_t acc[4];
    step_scores(t, qf, acc);
    const int lane = threadIdx.x & 63;
    const int tok = t0 + (lane & 15);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int jj = j0 + 16 * nt + 4 * (lane >> 4);
        if (tok < tq && jj < j_end)        // streaming store: the scores are read back once, much later
            __builtin_nontemporal_store(acc[nt], reinterpret_cast<f32x4_t*>(sb + static_cast<int64_t>(tok) * ld + jj));
    }
}

// Ordered key of a score that passed >= tau (so not NaN): -0.0 and +0.0
// share 0x80000000, as in score_key.
__device__ __forceinline__ uint32_t passed_key(uint32_t u) {
    return u == 0x80000000u ? 0x80000000u : (u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u));
}

// collect: append (score bits << 32 | row_local << 16 | (j - j_begin)) for
// every score of the lane's row at or above its threshold tau, for blocks
// below lim (the row's own block and the chunk end), to the wave's own LDS
// list: one ballot per score slot, positions by mbcnt, the count kept
// wave-uniform in a scalar register (no atomics).  The ordered key is formed
// later, once per listed candidate.  A NaN tau passes nothing.
//
// Most slots pass in no lane, so a slot costs one compare into a scalar
// mask; a passing slot costs its position (two mbcnt), the packed index (one
// add from the step's per-lane base) and the LDS write.  While the list has
// room for every lane of the slot (a scalar test) no lane checks its
// position.  With kSpill (the retry pass) a candidate that finds the list
// full goes to its row's global list (one atomic on its count each).
template <bool kLimit, bool kSpill>
__device__ __forceinline__ void collect_scan(const f32x4_t (&acc)[4], int jl, int lim, float tau, uint32_t base,
                                             uint64_t* seg, int& cnt, uint64_t* row_list, int* row_cnt) {
    constexpr int kWaveCap = kCollectCap / 4;
    int c = __builtin_amdgcn_readfirstlane(cnt);
    bool q[16];
    uint64_t m[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int off = 16 * (e >> 2) + (e & 3);
        q[e] = (!kLimit || jl + off < lim) && acc[e >> 2][e & 3] >= tau;
        m[e] = __builtin_amdgcn_ballot_w64(q[e]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (m[e] != 0ull) {                               // wave-uniform
            const int off = 16 * (e >> 2) + (e & 3);
            const float v = acc[e >> 2][e & 3];
            const int c0 = c;
            const int n = __popcll(m[e]);
            c = c0 + n;
            if (q[e]) {
                const int pos = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                    static_cast<uint32_t>(m[e] >> 32),
                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m[e]), static_cast<uint32_t>(c0))));
                if (c0 + n <= kWaveCap || pos < kWaveCap) {
                    seg[pos] = (static_cast<uint64_t>(__float_as_uint(v)) << 32) | (base + static_cast<uint32_t>(off));
                } else if constexpr (kSpill) {
                    const int gp = atomicAdd(row_cnt, 1);
                    if (gp < kRowCap)
                        row_list[gp] = (static_cast<uint64_t>(passed_key(__float_as_uint(v))) << 32) |
                                       static_cast<uint32_t>(~(jl + off));
                }
            }
        }
    }
    cnt = c;
}

template <bool kSpill>
__device__ __forceinline__ void collect_step(const KTile& t, const bf16x8_t (&qf)[kIdxSlices], int j0, int lim,
                                             float tau, int row_local, int j_begin, uint64_t* seg, int& cnt,
                                             uint64_t* row_list, int* row_cnt) {
    f32x4_t acc[4];
    step_scores<1>(t, qf, acc);
    const int lane = threadIdx.x & 63;
    const int jl = j0 + 4 * (lane >> 4);
    const uint32_t base = static_cast<uint32_t>((row_local << 16) | (jl - j_begin));
    // the block limit matters only in the steps that reach some lane's limit
    if (__all(j0 + kColStep <= lim))
        collect_scan<false, kSpill>(acc, jl, lim, tau, base, seg, cnt, row_list, row_cnt);
    else
        collect_scan<true, kSpill>(acc, jl, lim, tau, base, seg, cnt, row_list, row_cnt);
}

template <int kMode, bool kPaged>
__global__ __launch_bounds__(256) void index_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos0, int tq, int n_wt, int n_cc, int cols_per_chunk, int64_t n_wg,
    float* __restrict__ scores, int64_t ld, int64_t ss, const int* __restrict__ flags, IndexCollect col,
    PageMap pm) {
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
    if (kMode == kModeScores && flags != nullptr) {       // only the row tiles holding a flagged row
        if (col.n_flagged != nullptr && *col.n_flagged == 0) return;
        const int tid = threadIdx.x;
        const bool mine = tid < n_tok_wg && flags[static_cast<int64_t>(b) * tq + t_wg + tid] != 0;
        if (!__syncthreads_or(mine)) return;
    }
    const int omin = pos0.p[b] / kBlock;
    const int jmax = (kMode == kModeSample) ? kSampleCols : (pos0.p[b] + t_wg + n_tok_wg - 1) / kBlock;
    const int j_begin = cc * cols_per_chunk;
    const int j_end = min(j_begin + cols_per_chunk, jmax);
    if (j_begin >= j_end) return;                         // whole workgroup
    if (kMode == kModeCollectRetry && col.wg_flag[wg] == 0) return;   // its lists fit in the first pass

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = t_wg + kTokTile * wave;
    const bool has_rows = t0 < tq;

    bf16x8_t qf[kIdxSlices];
    load_index_q(q_idx + b * qs, t0, tq, qf);

    // block keys of the sequence, or the page pool and the sequence's table row
    const uint16_t* kb = kPaged ? kbar : kbar + b * kbs;
    const KbPages kp{kPaged ? pm.table + b * pm.ts : nullptr, pm.shift, pm.n_pages};
    const int n_steps = (j_end - j_begin + kColStep - 1) / kColStep;
    const DmaOffsets dof = dma_offsets();

    if constexpr (kMode == kModeCollect || kMode == kModeCollectRetry) {
        constexpr bool kSpill = kMode == kModeCollectRetry;
        const int tok = t0 + (lane & 15);
        const int64_t row = static_cast<int64_t>(b) * tq + tok;
        const float tau = tok < tq ? col.tau[row] : __uint_as_float(0x7fc00000u);
        uint64_t* row_list = col.list + row * kRowCap;     // this lane's row (used only when tok < tq)
        int* row_cnt = col.row_cnt + row;
        const int lim = min((pos0.p[b] + tok) / kBlock, j_end);
        if (threadIdx.x < kWgTok) lrow[threadIdx.x] = 0;
        uint64_t* seg = lcand + wave * (kCollectCap / 4);    // this wave's list
        int cnt = 0;
        __builtin_amdgcn_s_waitcnt(0x0f70);               // q and tau in registers before the pipeline starts
        __syncthreads();
        // two LDS buffers: step s + 1 loads while step s is scored; the loop
        // issues no other vector memory op, so "all landed" is vmcnt(0)
        stage_dma<kMode, kPaged>(kb, j_begin, j_end, omin, kp, dof, tA);
        for (int s = 0; s < n_steps; s += 2) {
            wait_and_meet<0>();
            stage_dma<kMode, kPaged>(kb, j_begin + kColStep * (s + 1), j_end, omin, kp, dof, tB);
            if (has_rows)
                collect_step<kSpill>(tA, qf, j_begin + kColStep * s, lim, tau, tok - t_wg, j_begin, seg, cnt, row_list,
                                     row_cnt);
            if (s + 1 >= n_steps) break;
            wait_and_meet<0>();
            stage_dma<kMode, kPaged>(kb, j_begin + kColStep * (s + 2), j_end, omin, kp, dof, tA);
            if (has_rows)
                collect_step<kSpill>(tB, qf, j_begin + kColStep * (s + 1), lim, tau, tok - t_wg, j_begin, seg, cnt,
                                     row_list, row_cnt);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);               // no load into LDS outlives the workgroup
        __syncthreads();
        // hand the lists to the rows: count per row, one global reservation
        // per row (in the retry pass, what did not fit went to the rows already)
        if (lane == 0) lwcnt[wave] = kSpill ? min(cnt, kCollectCap / 4) : cnt;
        __syncthreads();
        if constexpr (!kSpill) {
            bool overflow = false;
#pragma unroll
            for (int w = 0; w < 4; ++w) overflow |= lwcnt[w] > kCollectCap / 4;
            if (threadIdx.x == 0) col.wg_flag[wg] = overflow ? 1 : 0;
            if (overflow) return;                         // the retry pass redoes this workgroup
        }
        int slot[kCollectCap / 256];
#pragma unroll
        for (int k = 0; k < kCollectCap / 256; ++k) {
            const int i = threadIdx.x + 256 * k;
            const bool v = (i % (kCollectCap / 4)) < lwcnt[i / (kCollectCap / 4)];
            slot[k] = v ? atomicAdd(&lrow[(lcand[i] >> 16) & 63], 1) : -1;
        }
        __syncthreads();
        if (threadIdx.x < n_tok_wg && lrow[threadIdx.x] > 0)
            lrow_base[threadIdx.x] = atomicAdd(&col.row_cnt[static_cast<int64_t>(b) * tq + t_wg + threadIdx.x], lrow[threadIdx.x]);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kCollectCap / 256; ++k) {
            const int i = threadIdx.x + 256 * k;
            if (slot[k] >= 0) {
                const uint64_t e = lcand[i];
                const int rl = static_cast<int>((e >> 16) & 63);
                const int pos = lrow_base[rl] + slot[k];
                if (pos < kRowCap) {
                    const int j = j_begin + static_cast<int>(e & 0xffffu);
                    col.list[(static_cast<int64_t>(b) * tq + t_wg + rl) * kRowCap + pos] =
                        (static_cast<uint64_t>(passed_key(static_cast<uint32_t>(e >> 32))) << 32) |
                        static_cast<uint32_t>(~j);
                }
            }
        }
    } else {
        __builtin_amdgcn_s_waitcnt(0x0f70);               // B in registers before the load pipeline starts
        float* sb = scores + b * ss;
        // three LDS buffers: step s is scored while steps s + 1 and s + 2 load
        stage_dma<kMode, kPaged>(kb, j_begin, j_end, omin, kp, dof, tA);
        stage_dma<kMode, kPaged>(kb, j_begin + kColStep, j_end, omin, kp, dof, tB);
        for (int s = 0; s < n_steps; s += 3) {
            step_sync(s, has_rows);
            stage_dma<kMode, kPaged>(kb, j_begin + kColStep * (s + 2), j_end, omin, kp, dof, tC);
            if (has_rows) store_step(tA, qf, j_begin + kColStep * s, j_end, t0, tq, sb, ld);
            if (s + 1 >= n_steps) break;
            step_sync(s + 1, has_rows);
            stage_dma<kMode, kPaged>(kb, j_begin + kColStep * (s + 3), j_end, omin, kp, dof, tA);
            if (has_rows) store_step(tB, qf, j_begin + kColStep * (s + 1), j_end, t0, tq, sb, ld);
            if (s + 2 >= n_steps) break;
            step_sync(s + 2, has_rows);
            stage_dma<kMode, kPaged>(kb, j_begin + kColStep * (s + 4), j_end, omin, kp, dof, tB);
            if (has_rows) store_step(tC, qf, j_begin + kColStep * (s + 2), j_end, t0, tq, sb, ld);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);               // no load into LDS outlives the workgroup
    }
}

// Grid: batch x column chunks x 64-row tiles, the chunk width a multiple of
// 64 blocks (at most max_cols) so that a few thousand workgroups fill the chip.
static void index_grid(int jmax, int batch, int tq, int max_cols, int* n_wt, int* n_cc, int* cols_per_chunk,
                       int64_t* n_wg) {
    *n_wt = (tq + kWgTok - 1) / kWgTok;
    const int64_t steps = (jmax + kColStep - 1) / kColStep;
    const int64_t target_wgs = 4096;
    int64_t per = (static_cast<int64_t>(batch) * *n_wt * steps) / target_wgs;
    per = per < 1 ? 1 : (per > max_cols / kColStep ? max_cols / kColStep : per);
    *cols_per_chunk = static_cast<int>(per * kColStep);
    *n_cc = max(1, static_cast<int>((jmax + *cols_per_chunk - 1) / *cols_per_chunk));
    *n_wg = static_cast<int64_t>(batch) * *n_cc * *n_wt;
}

template <int kMode>
static hipError_t launch_mode(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                              const Positions& pos0, int batch, int tq, int jmax, int max_cols, float* scores,
                              int64_t ld, int64_t ss, const int* flags, const IndexCollect& col,
                              const PageMap* pm, hipStream_t stream) {
    if (tq <= 0 || jmax <= 0) return hipSuccess;
    int n_wt, n_cc, cpc;
    int64_t n_wg;
    index_grid(jmax, batch, tq, max_cols, &n_wt, &n_cc, &cpc, &n_wg);
    const unsigned grid = static_cast<unsigned>((n_wg + 7) / 8 * 8);
    if (pm != nullptr)
        hipLaunchKernelGGL((index_kernel<kMode, true>), dim3(grid), dim3(256), 0, stream, q_idx, qs, kbar, kbs,
                           pos0, tq, n_wt, n_cc, cpc, n_wg, scores, ld, ss, flags, col, *pm);
    else
        hipLaunchKernelGGL((index_kernel<kMode, false>), dim3(grid), dim3(256), 0, stream, q_idx, qs, kbar, kbs,
                           pos0, tq, n_wt, n_cc, cpc, n_wg, scores, ld, ss, flags, col, PageMap{});
    return hipGetLastError();
}

static int max_visible_block(const Positions& pos0, int batch, int tq) {
    int jmax = 0;
    for (int b = 0; b < batch; ++b) jmax = max(jmax, (pos0.p[b] + tq - 1) / kBlock);
    return jmax;
}

hipError_t launch_index_scores(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                               int64_t kbs, const Positions& pos0, int batch, int tq,
                               float* scores, int64_t ld, int64_t ss, const int* row_flags,
                               const int* n_flagged, const PageMap* pm, hipStream_t stream) {
    IndexCollect col{};
    col.n_flagged = n_flagged;
    return launch_mode<kModeScores>(q_idx, qs, kbar, kbs, pos0, batch, tq, max_visible_block(pos0, batch, tq),
                                    4096, scores, ld, ss, row_flags, col, pm, stream);
}

hipError_t launch_index_sample(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                               const Positions& pos0, int batch, int tq, float* sample, const PageMap* pm,
                               hipStream_t stream) {
    return launch_mode<kModeSample>(q_idx, qs, kbar, kbs, pos0, batch, tq, kSampleCols, 4096, sample,
                                    kSampleCols, static_cast<int64_t>(tq) * kSampleCols, nullptr, IndexCollect{},
                                    pm, stream);
}

hipError_t launch_index_collect(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                                const Positions& pos0, int batch, int tq, int max_cols, const IndexCollect& col,
                                const PageMap* pm, hipStream_t stream) {
    const int jmax = max_visible_block(pos0, batch, tq);
    hipError_t e = launch_mode<kModeCollect>(q_idx, qs, kbar, kbs, pos0, batch, tq, jmax, max_cols, nullptr, 0, 0,
                                             nullptr, col, pm, stream);
    if (e != hipSuccess) return e;
    return launch_mode<kModeCollectRetry>(q_idx, qs, kbar, kbs, pos0, batch, tq, jmax, max_cols, nullptr, 0, 0,
                                          nullptr, col, pm, stream);
}

}  // namespace qsa
