// Step 3: per-token block selection -- one workgroup per query row running
// the exact radix select of select_common.h on the row's float32 scores.
#include "select_common.h"

namespace qsa {

// Rows with a zero flag are skipped when flags is given; a processed row's
// flag is cleared (every thread has read it first).
__device__ __forceinline__ bool take_flagged_row(int* flags, int64_t row, int* sh) {
    if (flags == nullptr) return true;
    if (threadIdx.x == 0) *sh = flags[row];
    __syncthreads();
    const int f = *sh;
    if (f != 0 && threadIdx.x == 0) flags[row] = 0;
    return f != 0;
}

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ scores, int64_t ld,
                                                    int64_t ss, Positions pos0, int tq, int budget,
                                                    int32_t* __restrict__ sel, int64_t sels, int* flags) {
    __shared__ SelectSmem sm;
    __shared__ int sh_flag;
    const int b = blockIdx.x / tq;
    const int i = blockIdx.x % tq;
    if (!take_flagged_row(flags, blockIdx.x, &sh_flag)) return;
    const int p = pos0.p[b] + i;
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    select_row<NT>(scores + b * ss + static_cast<int64_t>(i) * ld, o, keep, budget,
                   sel + b * sels + static_cast<int64_t>(i) * budget, sm);
}

// ---------------------------------------------------------------------------
// Single-read selection (budgets up to 1024).  The multi-pass radix select
// above reads a long row two to four times; this one reads it once in the
// common case and falls back to it otherwise, so results are identical:
//   1. a sample of 8192 scores (32 evenly spread runs of 256) gives, by a two
//      level radix select in LDS, a key threshold tau whose expected count in
//      the whole row is sqrt(keep * kSpCap) -- far from both keep and the LDS
//      capacity;
//   2. one pass over the row appends every candidate with key >= tau to its
//      wave's LDS segment (ballot + mbcnt, no atomics), as (key << 32 | ~j);
//   3. if the segments did not overflow and hold at least `keep` entries, the
//      exact top `keep` of the whole row lies among them: a radix select over
//      the 64-bit entries (descending key, then ascending j) finds it;
//      otherwise the row is redone by select_row.
// Rows with at most kSpCap candidates skip the threshold and take them all.
constexpr int kSpNT = 512;
constexpr int kSpWaves = kSpNT / 64;
constexpr int kSpCap = 4096;                  // candidates held in LDS
constexpr int kSpSeg = kSpCap / kSpWaves;     // per-wave segment
constexpr int kSpRuns = 32;                   // sample runs of 64 float4
constexpr int kSpSample = kSpRuns * 64 * 4;

struct SampledSmem {
    alignas(16) uint64_t cand[kSpCap];
    ResolveSmem res;
    int seg_cnt[kSpWaves];
};

union SelectAllSmem {
    SampledSmem s;
    SelectSmem f;
};

// Appends (key(s) << 32 | ~j) for the lanes with q to the wave's segment.
// cnt is wave-uniform; entries past the segment are counted, not written.
__device__ __forceinline__ void wave_append(bool q, float s, int j, uint64_t* seg, int& cnt) {
    const uint64_t m = __ballot(q);
    if (m != 0ull) {
        if (q) {
            const int pos = cnt + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                      static_cast<uint32_t>(m >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
            if (pos < kSpSeg)
                seg[pos] = (static_cast<uint64_t>(score_key(s)) << 32) | static_cast<uint32_t>(~j);
        }
        cnt += __popcll(m);
    }
}

__global__ __launch_bounds__(kSpNT) void select_sampled_kernel(const float* __restrict__ scores, int64_t ld,
                                                               int64_t ss, Positions pos0, int tq, int budget,
                                                               int32_t* __restrict__ sel, int64_t sels, int* flags) {
    __shared__ SelectAllSmem smu;
    __shared__ int sh_flag;
    SampledSmem& sm = smu.s;
    const int b = blockIdx.x / tq;
    const int i = blockIdx.x % tq;
    if (!take_flagged_row(flags, blockIdx.x, &sh_flag)) return;
    const int o = (pos0.p[b] + i) / kBlock;
    const int keep = min(budget - 1, o);
    const float* row = scores + b * ss + static_cast<int64_t>(i) * ld;
    int32_t* out = sel + b * sels + static_cast<int64_t>(i) * budget;
    if (trivial_selection(keep, o, budget, out, kSpNT)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int o4 = o >> 2;
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const bool take_all = o <= kSpCap;

    // ---- 1. threshold from the sample ----
    float tf = 0.0f;
    if (!take_all) {
        uint32_t sk[16];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int f = tid + kSpNT * it;
            const int run = f >> 6;
            const int start4 = static_cast<int>(static_cast<int64_t>(run) * (o4 - 64) / (kSpRuns - 1));
            const float4 v = row4[start4 + (f & 63)];
            sk[4 * it + 0] = score_key(v.x);
            sk[4 * it + 1] = score_key(v.y);
            sk[4 * it + 2] = score_key(v.z);
            sk[4 * it + 3] = score_key(v.w);
        }
        const int64_t target = threshold_target(keep);
        const int r = static_cast<int>(min<int64_t>((target * kSpSample + o - 1) / o, kSpSample));
        tf = sample_threshold<kSpNT, 16>(sk, r, sm.res);
    }

    // ---- 2. one pass: candidates (score >= tf) into per-wave segments ----
    // For a number tf whose key has zero low bits, score >= tf (IEEE) holds
    // exactly when score_key(score) >= score_key(tf): -0.0 passes with +0.0
    // and NaN never passes; a NaN tf passes nothing.
    {
        uint64_t* seg = sm.cand + wave * kSpSeg;
        int cnt = 0;
        for (int k0 = 0; k0 < o4; k0 += 4 * kSpNT) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = row4[min(k0 + u * kSpNT + tid, o4 - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = k0 + u * kSpNT + tid;
                const bool valid = k < o4;
                wave_append(valid && (take_all || v[u].x >= tf), v[u].x, 4 * k + 0, seg, cnt);
                wave_append(valid && (take_all || v[u].y >= tf), v[u].y, 4 * k + 1, seg, cnt);
                wave_append(valid && (take_all || v[u].z >= tf), v[u].z, 4 * k + 2, seg, cnt);
                wave_append(valid && (take_all || v[u].w >= tf), v[u].w, 4 * k + 3, seg, cnt);
            }
        }
        if (wave == kSpWaves - 1) {          // the o % 4 trailing scores
            const int j = 4 * o4 + lane;
            const bool valid = lane < (o & 3);
            const float s = valid ? row[j] : 0.0f;
            wave_append(valid && (take_all || s >= tf), s, j, seg, cnt);
        }
        if (lane == 0) sm.seg_cnt[wave] = cnt;
    }
    __syncthreads();
    bool fallback = false;
    int total = 0;
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) {
        const int c = sm.seg_cnt[w];
        fallback |= c > kSpSeg;
        total += c;
    }
    fallback |= total < keep;
    if (fallback) {                           // uniform: every thread read the same counts
        __syncthreads();
        select_row<kSpNT>(row, o, keep, budget, out, smu.f);
        return;
    }

    // ---- 3. exact top `keep` among the candidates ----
    uint64_t c[kSpWaves];
    bool cv[kSpWaves];
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) {
        cv[w] = tid < sm.seg_cnt[w];
        c[w] = cv[w] ? sm.cand[w * kSpSeg + tid] : 0ull;
    }
    __syncthreads();                                      // every thread holds its candidates: the list is free
    finish_from_candidates<kSpNT, kSpWaves>(c, cv, total, keep, o, budget, out, sm.res,
                                            reinterpret_cast<uint32_t*>(sm.cand));
}

hipError_t launch_select(const float* scores, int64_t ld, int64_t ss, const Positions& pos0,
                         int batch, int tq, int budget, int32_t* sel, int64_t sels, int* flags,
                         hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * tq;
    if (rows == 0) return hipSuccess;
    if (budget <= kResMaxBudget) {
        hipLaunchKernelGGL(select_sampled_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSpNT), 0, stream,
                           scores, ld, ss, pos0, tq, budget, sel, sels, flags);
    } else if (rows < 1024) {
        hipLaunchKernelGGL(select_kernel<1024>, dim3(static_cast<unsigned>(rows)), dim3(1024), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels, flags);
    } else {
        hipLaunchKernelGGL(select_kernel<256>, dim3(static_cast<unsigned>(rows)), dim3(256), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels, flags);
    }
    return hipGetLastError();
}

}  // namespace qsa
