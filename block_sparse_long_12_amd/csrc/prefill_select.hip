// Steps 2 + 3 fused for a prefill chunk: the same selection as
// index_scores_kernel followed by the selection kernels (blog "Attention:
// GDN + QSA": blocks are scored and the most relevant ones kept; model card:
// budget 512 blocks), without writing and re-reading the score matrix.
//
//  1. sample      the indexer scores a fixed sample of 4096 blocks per row (256
//                 runs of 16 spread over the blocks every row of the chunk
//                 sees);
//  2. threshold   per row, a key threshold from the sample whose expected
//                 count in the whole row is threshold_target(keep);
//  3. collect     the indexer scores every block; scores at or above the
//                 row's threshold go to the row's candidate list (a second
//                 launch redoes the workgroups whose LDS lists overflowed,
//                 sending what does not fit straight to the rows' lists);
//  4. finalize    per row: if the list holds at least `keep` entries and did
//                 not overflow, it contains the row's exact top `keep`, which
//                 an exact radix select finishes; otherwise the row is flagged;
//  5. fallback    flagged rows (if any) get full scores and the full exact
//                 selection, so every row's result is that of the unfused path.
// Chunks whose rows see fewer than kFusedMinBlocks blocks, or budgets above
// kResMaxBudget, take the unfused path directly.
#include "select_common.h"

namespace qsa {

constexpr int kThrNT = 256;
constexpr int kFinNT = 512;
constexpr int kFusedMinBlocks = 16384;

// Every field is (re)initialised by the call that uses it, so the workspace
// needs no preparation and its layout may change with the call's shape.
struct PrefillWs {
    int* n_flagged;     // rows flagged for the fallback (zeroed by threshold_kernel)
    int* flags;         // [rows] (zeroed by threshold_kernel, set by finalize)
    int* row_cnt;       // [rows] list lengths (zeroed by threshold_kernel)
    float* tau;         // [rows]
    uint64_t* list;     // [rows][kRowCap]
    float* sample;      // [rows][kSampleCols]
};

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

size_t prefill_select_ws_bytes(int batch, int tq) {
    const size_t rows = static_cast<size_t>(batch) * tq;
    return al256(rows * 4) + 256 + al256(rows * 4) + al256(rows * 4) + rows * kRowCap * 8 +
           rows * static_cast<size_t>(kSampleCols) * 4;
}

static PrefillWs carve(void* ws, int batch, int tq) {
    const size_t rows = static_cast<size_t>(batch) * tq;
    char* p = static_cast<char*>(ws);
    PrefillWs w;
    w.n_flagged = reinterpret_cast<int*>(p);
    p += 256;
    w.flags = reinterpret_cast<int*>(p);
    p += al256(rows * 4);
    w.row_cnt = reinterpret_cast<int*>(p);
    p += al256(rows * 4);
    w.tau = reinterpret_cast<float*>(p);
    p += al256(rows * 4);
    w.list = reinterpret_cast<uint64_t*>(p);
    p += rows * kRowCap * 8;
    w.sample = reinterpret_cast<float*>(p);
    return w;
}

// One workgroup per row: the threshold from the row's 4096 sampled scores.
__global__ __launch_bounds__(kThrNT) void threshold_kernel(const float* __restrict__ sample, Positions pos0, int tq,
                                                           int budget, PrefillWs ws) {
    __shared__ ResolveSmem sm;
    const int64_t row = blockIdx.x;
    const int b = static_cast<int>(row / tq);
    const int i = static_cast<int>(row % tq);
    const int o = (pos0.p[b] + i) / kBlock;
    const int keep = min(budget - 1, o);
    if (threadIdx.x == 0) {
        if (row == 0) *ws.n_flagged = 0;
        ws.flags[row] = 0;
        ws.row_cnt[row] = 0;
    }
    if (keep == 0 || keep == o) {                         // trivial rows collect nothing
        if (threadIdx.x == 0) ws.tau[row] = __uint_as_float(0x7fc00000u);
        return;
    }
    const float4* s4 = reinterpret_cast<const float4*>(sample + row * kSampleCols);
    uint32_t sk[kSampleCols / kThrNT];
#pragma unroll
    for (int it = 0; it < kSampleCols / kThrNT / 4; ++it) {
        const float4 v = s4[threadIdx.x + kThrNT * it];
        sk[4 * it + 0] = score_key(v.x);
        sk[4 * it + 1] = score_key(v.y);
        sk[4 * it + 2] = score_key(v.z);
        sk[4 * it + 3] = score_key(v.w);
    }
    const int64_t target = threshold_target(keep);
    const int r = static_cast<int>(min<int64_t>((target * kSampleCols + o - 1) / o, kSampleCols));
    const float t = sample_threshold<kThrNT, kSampleCols / kThrNT>(sk, r, sm);
    if (threadIdx.x == 0) ws.tau[row] = t;
}

// One workgroup per row: the exact finish from the row's candidate list.
__global__ __launch_bounds__(kFinNT) void prefill_finalize_kernel(Positions pos0, int tq, int budget, PrefillWs ws,
                                                                  int32_t* __restrict__ sel, int64_t sels) {
    __shared__ ResolveSmem sm;
    __shared__ uint32_t bitmap[kResBitmapWords];
    __shared__ int sh_n;
    const int64_t row = blockIdx.x;
    const int b = static_cast<int>(row / tq);
    const int i = static_cast<int>(row % tq);
    const int o = (pos0.p[b] + i) / kBlock;
    const int keep = min(budget - 1, o);
    int32_t* out = sel + b * sels + static_cast<int64_t>(i) * budget;
    if (threadIdx.x == 0) sh_n = ws.row_cnt[row];
    __syncthreads();
    const int n = sh_n;
    if (trivial_selection(keep, o, budget, out, kFinNT)) return;
    if (n < keep || n > kRowCap) {                        // short or overflowed: exact fallback
        if (threadIdx.x == 0) {
            ws.flags[row] = 1;
            atomicAdd(ws.n_flagged, 1);
        }
        return;
    }
    constexpr int K = kRowCap / kFinNT;
    uint64_t c[K];
    bool cv[K];
    const uint64_t* lst = ws.list + row * kRowCap;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = threadIdx.x + kFinNT * k;
        cv[k] = idx < n;
        c[k] = cv[k] ? lst[idx] : 0ull;
    }
    finish_from_candidates<kFinNT, K>(c, cv, n, keep, o, budget, out, sm, bitmap);
}

hipError_t launch_prefill_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                                       const Positions& pos0, int batch, int tq, int budget, float* scores,
                                       int64_t ld, int64_t ss, int32_t* sel, int64_t sels, void* ws,
                                       const PageMap* pm, hipStream_t stream) {
    if (tq <= 0) return hipSuccess;
    int omin = 0x7fffffff;
    for (int b = 0; b < batch; ++b) omin = min(omin, pos0.p[b] / kBlock);
    if (budget > kResMaxBudget || omin < kFusedMinBlocks) {
        hipError_t e = launch_index_scores(q_idx, qs, kbar, kbs, pos0, batch, tq, scores, ld, ss, nullptr, nullptr,
                                           pm, stream);
        if (e != hipSuccess) return e;
        return launch_select(scores, ld, ss, pos0, batch, tq, budget, sel, sels, nullptr, stream);
    }
    const PrefillWs w = carve(ws, batch, tq);
    const unsigned rows = static_cast<unsigned>(static_cast<int64_t>(batch) * tq);
    hipError_t e = launch_index_sample(q_idx, qs, kbar, kbs, pos0, batch, tq, w.sample, pm, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(threshold_kernel, dim3(rows), dim3(kThrNT), 0, stream, w.sample, pos0, tq, budget, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // column chunks narrow enough that a workgroup's expected candidates
    // (64 rows x width x target / blocks) stay below half its LDS list
    const int64_t target = 2 * (budget - 1) + 512;
    int64_t cols = 16 * static_cast<int64_t>(omin) / target / 64 * 64;
    cols = cols < 64 ? 64 : (cols > 4096 ? 4096 : cols);
    IndexCollect col{};
    col.tau = w.tau;
    col.row_cnt = w.row_cnt;
    col.list = w.list;
    // one byte per collect workgroup, over the sample (read by the threshold
    // kernel before the collect starts; rows x 16 KiB hold any grid's flags)
    col.wg_flag = reinterpret_cast<uint8_t*>(w.sample);
    e = launch_index_collect(q_idx, qs, kbar, kbs, pos0, batch, tq, static_cast<int>(cols), col, pm, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_finalize_kernel, dim3(rows), dim3(kFinNT), 0, stream, pos0, tq, budget, w, sel, sels);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_index_scores(q_idx, qs, kbar, kbs, pos0, batch, tq, scores, ld, ss, w.flags, w.n_flagged, pm, stream);
    if (e != hipSuccess) return e;
    return launch_select(scores, ld, ss, pos0, batch, tq, budget, sel, sels, w.flags, stream);
}

}  // namespace qsa
