// Step 3: per-token block selection (Qwen3.8-Flash-Next blog, "Attention:
// GDN + QSA": the most relevant blocks are selected; model card: budget 512
// blocks or 2048 tokens).  For the query at position p with own block
// o = p / 4: keep the top min(budget - 1, o) candidates j < o by (score desc,
// j asc), add o, write ascending, pad with -1.
//
// Exact radix select on ordered uint32 keys (score_key: monotone in the
// float, -0.0 == +0.0, NaN lowest).  One workgroup per query row:
//   1. histogram passes over the row (LDS atomics) on key digits of 11, 11
//      and 10 bits, each restricted to the current prefix, until the bin that
//      holds the threshold has at most kCap members (usually after one pass);
//   2. a collect pass: keys above the threshold bin are taken outright, bin
//      members go to LDS as (key << 32 | ~j) and are bitonic-sorted there, the
//      first `remaining` of them are taken;
//   3. if all 32 bits are resolved and the tied keys still exceed kCap, the
//      ties are taken in index order with a workgroup prefix count;
//   4. the chosen indices plus o are bitonic-sorted ascending and written.
// The result depends only on the score bits, never on thread timing.
#include "qsa_internal.h"

namespace qsa {

constexpr int kCap = 2048;     // threshold-bin members held in LDS

template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int t = wave_tot[w];
        before += (w < wave) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

template <int NT, typename T, bool kDescending>
__device__ void bitonic_sort(T* a, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const T x = a[i];
                    const T y = a[ixj];
                    const bool first_half_up = ((i & k) == 0) != kDescending;
                    if (first_half_up ? (x > y) : (x < y)) {
                        a[i] = y;
                        a[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ scores, int64_t ld,
                                                    int64_t ss, Positions pos0, int tq, int budget,
                                                    int32_t* __restrict__ sel, int64_t sels) {
    __shared__ uint32_t hist[2048];
    __shared__ uint64_t cand[kCap];
    __shared__ int32_t chosen[QSA_MAX_BUDGET];
    __shared__ int wave_tot[NT / 64];
    __shared__ int n_chosen, n_cand, sh_above;
    __shared__ uint32_t sh_bin;

    const int tid = threadIdx.x;
    const int b = blockIdx.x / tq;
    const int i = blockIdx.x % tq;
    const int p = pos0.p[b] + i;
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    int32_t* out = sel + b * sels + static_cast<int64_t>(i) * budget;

    if (keep == o || keep == 0) {            // every candidate, or the own block alone
        for (int k = tid; k < budget; k += NT)
            out[k] = (keep == o) ? (k <= o ? k : -1) : (k == 0 ? o : -1);
        return;
    }
    const float* row = scores + b * ss + static_cast<int64_t>(i) * ld;
    const int n4 = o >> 2;
    const float4* row4 = reinterpret_cast<const float4*>(row);

    uint32_t prefix = 0, pmask = 0;
    int remaining = keep;                    // still to take among keys matching the prefix
    int bin_count = o;
    int shift = 32;
    for (int d = 0; d < 3 && bin_count > kCap; ++d) {
        const int bits = (d < 2) ? 11 : 10;
        shift -= bits;
        const int nb = 1 << bits;
        const uint32_t dmask = static_cast<uint32_t>(nb - 1);
        for (int k = tid; k < nb; k += NT) hist[k] = 0;
        __syncthreads();
        for (int k = tid; k < n4; k += NT) {
            const float4 v = row4[k];
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(f[e]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
        }
        for (int j = 4 * n4 + tid; j < o; j += NT) {
            const uint32_t key = score_key(row[j]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        // threshold bin: walk bins from the top; thread tid owns nb / NT of them
        const int bpt = nb / NT;
        const int hi = nb - 1 - tid * bpt;
        int local = 0;
        for (int q = 0; q < bpt; ++q) local += static_cast<int>(hist[hi - q]);
        int total;
        const int above = block_exclusive_scan<NT>(local, wave_tot, &total);
        if (above < remaining && above + local >= remaining) {
            int run = above;
            for (int q = 0; q < bpt; ++q) {
                const int h = static_cast<int>(hist[hi - q]);
                if (run + h >= remaining) {
                    sh_bin = static_cast<uint32_t>(hi - q);
                    sh_above = run;
                    break;
                }
                run += h;
            }
        }
        __syncthreads();
        const uint32_t tb = sh_bin;
        remaining -= sh_above;
        prefix |= tb << shift;
        pmask |= dmask << shift;
        bin_count = static_cast<int>(hist[tb]);
        __syncthreads();
    }

    if (tid == 0) {
        n_chosen = 0;
        n_cand = 0;
    }
    __syncthreads();

    if (bin_count <= kCap) {
        for (int k = tid; k < n4; k += NT) {
            const float4 v = row4[k];
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(f[e]);
                const uint32_t mk = key & pmask;
                const int j = 4 * k + e;
                if (mk > prefix) chosen[atomicAdd(&n_chosen, 1)] = j;
                else if (mk == prefix)
                    cand[atomicAdd(&n_cand, 1)] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
            }
        }
        for (int j = 4 * n4 + tid; j < o; j += NT) {
            const uint32_t key = score_key(row[j]);
            const uint32_t mk = key & pmask;
            if (mk > prefix) chosen[atomicAdd(&n_chosen, 1)] = j;
            else if (mk == prefix)
                cand[atomicAdd(&n_cand, 1)] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
        }
        __syncthreads();
        const int nc = n_cand;
        const int base = n_chosen;           // == keep - remaining
        const int np2 = next_pow2(nc);
        for (int k = nc + tid; k < np2; k += NT) cand[k] = 0;   // below every real entry
        __syncthreads();
        bitonic_sort<NT, uint64_t, true>(cand, np2);
        for (int k = tid; k < remaining; k += NT)
            chosen[base + k] = static_cast<int32_t>(~static_cast<uint32_t>(cand[k]));
        __syncthreads();
    } else {
        // all 32 key bits fixed: key == prefix are ties, taken by ascending index
        int tie_base = 0;
        for (int base = 0; base < o; base += NT) {
            const int j = base + tid;
            const uint32_t key = (j < o) ? score_key(row[j]) : 0u;
            const bool gt = (j < o) && key > prefix;
            const bool eq = (j < o) && key == prefix;
            if (gt) chosen[atomicAdd(&n_chosen, 1)] = j;
            int total;
            const int rank = block_exclusive_scan<NT>(eq ? 1 : 0, wave_tot, &total);
            if (eq && tie_base + rank < remaining) chosen[atomicAdd(&n_chosen, 1)] = j;
            tie_base += total;
        }
        __syncthreads();
    }

    // chosen[0 .. keep) + the own block, ascending
    const int nsel = keep + 1;
    const int np2 = next_pow2(nsel);
    if (tid == 0) chosen[keep] = o;
    for (int k = nsel + tid; k < np2; k += NT) chosen[k] = 0x7fffffff;
    __syncthreads();
    bitonic_sort<NT, int32_t, false>(chosen, np2);
    for (int k = tid; k < budget; k += NT) out[k] = (k < nsel) ? chosen[k] : -1;
}

hipError_t launch_select(const float* scores, int64_t ld, int64_t ss, const Positions& pos0,
                         int batch, int tq, int budget, int32_t* sel, int64_t sels,
                         hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * tq;
    if (rows == 0) return hipSuccess;
    if (rows < 1024) {
        hipLaunchKernelGGL(select_kernel<1024>, dim3(static_cast<unsigned>(rows)), dim3(1024), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels);
    } else {
        hipLaunchKernelGGL(select_kernel<256>, dim3(static_cast<unsigned>(rows)), dim3(256), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels);
    }
    return hipGetLastError();
}

}  // namespace qsa
