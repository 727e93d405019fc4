// Exact per-row block selection, shared by the selection kernel and the
// fallback of the fused decode index-select.
//
// Row semantics (Qwen3.8-Flash-Next blog, "Attention: GDN + QSA": the most
// relevant blocks are selected; model card: budget 512 blocks): for the query
// with own block o, keep the top `keep` = min(budget - 1, o) candidates j < o
// by (score desc, j asc), add o, write ascending into out[0 .. budget),
// padded with -1.
//
// Exact radix select on ordered uint32 keys (score_key: monotone in the
// float, -0.0 == +0.0, NaN lowest), one workgroup per row:
//   1. histogram passes over the row (LDS atomics) on key digits of 11, 11
//      and 10 bits, each restricted to the current prefix, until the bin that
//      holds the threshold has at most kSelectCap members;
//   2. a collect pass: keys above the threshold bin are taken outright, bin
//      members go to LDS as (key << 32 | ~j) and are bitonic-sorted, the first
//      `remaining` are taken;
//   3. if all 32 bits are resolved and the tied keys still exceed kSelectCap,
//      the ties are taken in index order with a workgroup prefix count;
//   4. the chosen indices plus o are bitonic-sorted ascending and written.
// The result depends only on the score bits, never on thread timing.
#pragma once

#include "qsa_internal.h"

namespace qsa {

constexpr int kSelectCap = 2048;     // threshold-bin members held in LDS

struct SelectSmem {
    uint32_t hist[2048];
    alignas(16) uint64_t cand[kSelectCap];
    alignas(16) int32_t chosen[QSA_MAX_BUDGET];
    int wave_tot[16];
    int n_chosen, n_cand, sh_above;
    uint32_t sh_bin;
};

// Exclusive prefix sum of v over the workgroup; *total gets the sum.  With
// kTrailingSync false the call ends without the barrier that keeps wave_tot
// from being rewritten while slower threads still read it: for callers whose
// next write of wave_tot is behind a barrier of their own anyway.
template <int NT, bool kTrailingSync = true>
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
    lds_barrier();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int t = wave_tot[w];
        before += (w < wave) ? t : 0;
        all += t;
    }
    if (kTrailingSync) lds_barrier();
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
            lds_barrier();
        }
    }
}

__device__ __forceinline__ int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Threshold bin of a histogram walked from the top: the bin where the
// running count (from the highest bin down) first reaches `remaining`.
// Sets *sh_bin and *sh_above (count strictly above that bin).  Every thread
// of the workgroup must call it; nb must be a multiple of NT.
template <int NT>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, int nb, int remaining,
                                                   int* wave_tot, uint32_t* sh_bin, int* sh_above) {
    const int tid = threadIdx.x;
    const int bpt = nb / NT;
    const int hi = nb - 1 - tid * bpt;
    int local = 0;
    for (int q = 0; q < bpt; ++q) local += static_cast<int>(hist[hi - q]);
    int total;
    const int above = block_exclusive_scan<NT, false>(local, wave_tot, &total);   // the barrier below follows
    if (above < remaining && above + local >= remaining) {
        int run = above;
        for (int q = 0; q < bpt; ++q) {
            const int h = static_cast<int>(hist[hi - q]);
            if (run + h >= remaining) {
                *sh_bin = static_cast<uint32_t>(hi - q);
                *sh_above = run;
                break;
            }
            run += h;
        }
    }
    lds_barrier();
}

// Writes the final ascending selection: sm.chosen[0 .. keep) plus o.
template <int NT>
__device__ __forceinline__ void write_selection(SelectSmem& sm, int keep, int o, int budget,
                                                int32_t* out) {
    const int tid = threadIdx.x;
    const int nsel = keep + 1;
    const int np2 = next_pow2(nsel);
    if (tid == 0) sm.chosen[keep] = o;
    for (int k = nsel + tid; k < np2; k += NT) sm.chosen[k] = 0x7fffffff;
    lds_barrier();
    bitonic_sort<NT, int32_t, false>(sm.chosen, np2);
    for (int k = tid; k < budget; k += NT) out[k] = (k < nsel) ? sm.chosen[k] : -1;
}

// The `take` largest of cand[0 .. n) (distinct keys) by counting: entry i
// goes to dst[rank_i] (as the block index ~key) when rank_i < take, so dst
// ends in descending key order.  cand must be 16-byte aligned with room for
// an even count; the odd tail is padded with 0 (below every real key).
// Every lane reads the same 16 bytes at a time (LDS broadcast), 8 reads in
// flight.  O(n^2 / NT) work per thread: for lists of a few hundred.
template <int NT>
__device__ __forceinline__ void rank_take_desc(uint64_t* cand, int n, int take, int32_t* dst) {
    if (threadIdx.x == 0 && (n & 1)) cand[n] = 0ull;
    lds_barrier();
    const int n2 = (n + 1) >> 1;
    const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand);
    for (int i = threadIdx.x; i < n; i += NT) {
        const uint64_t x = cand[i];
        int r = 0;
#pragma unroll 8
        for (int k = 0; k < n2; ++k) {
            const ulonglong2 v = c2[k];
            r += (v.x > x ? 1 : 0) + (v.y > x ? 1 : 0);
        }
        if (r < take) dst[r] = static_cast<int32_t>(~static_cast<uint32_t>(x));
    }
}

// vals[0 .. n) (distinct, below INT32_MAX) written ascending into out[0 .. n)
// by counting; vals must be 16-byte aligned with room for n rounded up to 4
// (the tail is padded with INT32_MAX).
template <int NT>
__device__ __forceinline__ void rank_write_ascending(int32_t* vals, int n, int32_t* out) {
    const int n4 = (n + 3) >> 2;
    for (int k = n + threadIdx.x; k < 4 * n4; k += NT) vals[k] = 0x7fffffff;
    lds_barrier();
    const int4* v4 = reinterpret_cast<const int4*>(vals);
    for (int i = threadIdx.x; i < n; i += NT) {
        const int32_t x = vals[i];
        int r = 0;
#pragma unroll 8
        for (int k = 0; k < n4; ++k) {
            const int4 v = v4[k];
            r += (v.x < x ? 1 : 0) + (v.y < x ? 1 : 0) + (v.z < x ? 1 : 0) + (v.w < x ? 1 : 0);
        }
        out[r] = x;
    }
}

// Trivial rows: every candidate fits the budget, or the budget is the own block alone.
__device__ __forceinline__ bool trivial_selection(int keep, int o, int budget, int32_t* out, int nt) {
    if (keep != o && keep != 0) return false;
    for (int k = threadIdx.x; k < budget; k += nt)
        out[k] = (keep == o) ? (k <= o ? k : -1) : (k == 0 ? o : -1);
    return true;
}

// Full selection of one row held in global memory (16-byte aligned).
template <int NT>
__device__ void select_row(const float* __restrict__ row, int o, int keep, int budget,
                           int32_t* __restrict__ out, SelectSmem& sm) {
    const int tid = threadIdx.x;
    if (trivial_selection(keep, o, budget, out, NT)) return;
    const int n4 = o >> 2;
    const float4* row4 = reinterpret_cast<const float4*>(row);

    uint32_t prefix = 0, pmask = 0;
    int remaining = keep;                    // still to take among keys matching the prefix
    int bin_count = o;
    int shift = 32;
    for (int d = 0; d < 3 && bin_count > kSelectCap; ++d) {
        const int bits = (d < 2) ? 11 : 10;
        shift -= bits;
        const int nb = 1 << bits;
        const uint32_t dmask = static_cast<uint32_t>(nb - 1);
        for (int k = tid; k < nb; k += NT) sm.hist[k] = 0;
        lds_barrier();
        for (int k = tid; k < n4; k += NT) {
            const float4 v = row4[k];
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(f[e]);
                if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1u);
            }
        }
        for (int j = 4 * n4 + tid; j < o; j += NT) {
            const uint32_t key = score_key(row[j]);
            if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1u);
        }
        lds_barrier();
        find_threshold_bin<NT>(sm.hist, nb, remaining, sm.wave_tot, &sm.sh_bin, &sm.sh_above);
        const uint32_t tb = sm.sh_bin;
        remaining -= sm.sh_above;
        prefix |= tb << shift;
        pmask |= dmask << shift;
        bin_count = static_cast<int>(sm.hist[tb]);
        lds_barrier();
    }

    if (tid == 0) {
        sm.n_chosen = 0;
        sm.n_cand = 0;
    }
    lds_barrier();

    if (bin_count <= kSelectCap) {
        for (int k = tid; k < n4; k += NT) {
            const float4 v = row4[k];
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(f[e]);
                const uint32_t mk = key & pmask;
                const int j = 4 * k + e;
                if (mk > prefix) sm.chosen[atomicAdd(&sm.n_chosen, 1)] = j;
                else if (mk == prefix)
                    sm.cand[atomicAdd(&sm.n_cand, 1)] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
            }
        }
        for (int j = 4 * n4 + tid; j < o; j += NT) {
            const uint32_t key = score_key(row[j]);
            const uint32_t mk = key & pmask;
            if (mk > prefix) sm.chosen[atomicAdd(&sm.n_chosen, 1)] = j;
            else if (mk == prefix)
                sm.cand[atomicAdd(&sm.n_cand, 1)] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
        }
        lds_barrier();
        const int nc = sm.n_cand;
        const int base = sm.n_chosen;        // == keep - remaining
        const int np2 = next_pow2(nc);
        for (int k = nc + tid; k < np2; k += NT) sm.cand[k] = 0;   // below every real entry
        lds_barrier();
        bitonic_sort<NT, uint64_t, true>(sm.cand, np2);
        for (int k = tid; k < remaining; k += NT)
            sm.chosen[base + k] = static_cast<int32_t>(~static_cast<uint32_t>(sm.cand[k]));
        lds_barrier();
    } else {
        // all 32 key bits fixed: key == prefix are ties, taken by ascending index
        int tie_base = 0;
        for (int base = 0; base < o; base += NT) {
            const int j = base + tid;
            const uint32_t key = (j < o) ? score_key(row[j]) : 0u;
            const bool gt = (j < o) && key > prefix;
            const bool eq = (j < o) && key == prefix;
            if (gt) sm.chosen[atomicAdd(&sm.n_chosen, 1)] = j;
            int total;
            const int rank = block_exclusive_scan<NT>(eq ? 1 : 0, sm.wave_tot, &total);
            if (eq && tie_base + rank < remaining) sm.chosen[atomicAdd(&sm.n_chosen, 1)] = j;
            tie_base += total;
        }
        lds_barrier();
    }
    write_selection<NT>(sm, keep, o, budget, out);
}

// ---------------------------------------------------------------------------
// Pieces of the threshold-based selections (the single-read select and the
// fused prefill index-select): a key threshold estimated from a sample, and
// the exact finish among the candidates at or above it.

constexpr int kResShort = 256;        // threshold-bin members resolved by ranking
constexpr int kResMaxBudget = 1024;   // budgets the threshold paths serve

constexpr int kResBitmapWords = 8192;  // ascending output by bitmap for o <= 262144

struct ResolveSmem {
    alignas(16) uint64_t shortl[kResShort + 2];
    alignas(16) int32_t chosen[kResMaxBudget];
    uint32_t hist[2048];
    uint64_t wave_hi[16], wave_lo[16];
    int wave_tot[16];
    int n_chosen, n_short, sh_above;
    uint32_t sh_bin;
};

// float whose score_key is `key` (key must not be the image of a NaN pattern)
__device__ __forceinline__ float key_to_float(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Expected number of candidates the threshold aims at for a row keeping
// `keep`: far above keep (a short count forces the exact fallback) and far
// below the capacities of the candidate buffers.
__device__ __forceinline__ int threshold_target(int keep) { return 2 * keep + 512; }

// Key threshold from sample keys held PER per thread (1 <= r <= NT * PER):
// the lower edge of the 22-bit key prefix holding the r-th largest sample key
// (two 11-bit radix levels in LDS).
template <int NT, int PER>
__device__ uint32_t sample_threshold_key(const uint32_t (&sk)[PER], int r, ResolveSmem& sm) {
    const int tid = threadIdx.x;
    for (int k = tid; k < 2048; k += NT) sm.hist[k] = 0u;
    lds_barrier();
#pragma unroll
    for (int e = 0; e < PER; ++e) atomicAdd(&sm.hist[sk[e] >> 21], 1u);
    lds_barrier();
    find_threshold_bin<NT>(sm.hist, 2048, r, sm.wave_tot, &sm.sh_bin, &sm.sh_above);
    const uint32_t b1 = sm.sh_bin;
    const int r2 = r - sm.sh_above;
    lds_barrier();
    for (int k = tid; k < 2048; k += NT) sm.hist[k] = 0u;
    lds_barrier();
#pragma unroll
    for (int e = 0; e < PER; ++e)
        if ((sk[e] >> 21) == b1) atomicAdd(&sm.hist[(sk[e] >> 10) & 2047u], 1u);
    lds_barrier();
    find_threshold_bin<NT>(sm.hist, 2048, r2, sm.wave_tot, &sm.sh_bin, &sm.sh_above);
    const uint32_t tkey = (b1 << 21) | (sm.sh_bin << 10);
    lds_barrier();
    return tkey;
}

// The same threshold as the float to compare scores against; a quiet NaN (no
// score passes) when it would sit at or below -inf.
template <int NT, int PER>
__device__ float sample_threshold(const uint32_t (&sk)[PER], int r, ResolveSmem& sm) {
    const uint32_t tkey = sample_threshold_key<NT, PER>(sk, r, sm);
    return tkey <= 0x007fffffu ? __uint_as_float(0x7fc00000u) : key_to_float(tkey);
}

// Exact top `keep` (descending key, then ascending j) among `total` distinct
// candidates (key << 32 | ~j), K per thread in registers (valid where cv),
// that contain the row's true top `keep`; writes them and the own block o
// ascending into out[0 .. budget), padded with -1.  Radix passes over the
// 64-bit entries, the first digit placed just below the bits every candidate
// shares (from the largest and smallest entry), until the threshold bin holds
// at most kResShort, which are ranked.  The ascending output goes through a
// bitmap of the blocks when `bitmap` (kResBitmapWords words of free LDS) is
// given and o fits it, else by counting.  keep < kResMaxBudget.
template <int NT, int K>
__device__ void finish_from_candidates(const uint64_t (&c)[K], const bool (&cv)[K], int total, int keep, int o,
                                       int budget, int32_t* out, ResolveSmem& sm, uint32_t* bitmap) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // the bits all candidates share
    uint64_t hi = 0ull, lo = ~0ull;
#pragma unroll
    for (int w = 0; w < K; ++w) {
        if (cv[w]) {
            hi = c[w] > hi ? c[w] : hi;
            lo = c[w] < lo ? c[w] : lo;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t h2 = __shfl_xor(hi, off);
        const uint64_t l2 = __shfl_xor(lo, off);
        hi = h2 > hi ? h2 : hi;
        lo = l2 < lo ? l2 : lo;
    }
    if (lane == 0) {
        sm.wave_hi[wave] = hi;
        sm.wave_lo[wave] = lo;
    }
    lds_barrier();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        hi = sm.wave_hi[w] > hi ? sm.wave_hi[w] : hi;
        lo = sm.wave_lo[w] < lo ? sm.wave_lo[w] : lo;
    }
    const uint64_t diff = hi ^ lo;
    const int top = diff ? 63 - __clzll(diff) : 0;       // highest bit where candidates differ
    int sh = top > 10 ? top - 10 : 0;
    uint64_t pmask = (sh + 11 >= 64) ? 0ull : ~((1ull << (sh + 11)) - 1ull);
    uint64_t prefix = hi & pmask;
    int rem = keep;
    int bin_count = total;
    while (bin_count > kResShort) {
        for (int k = tid; k < 2048; k += NT) sm.hist[k] = 0u;
        lds_barrier();
#pragma unroll
        for (int w = 0; w < K; ++w)
            if (cv[w] && (c[w] & pmask) == prefix)
                atomicAdd(&sm.hist[static_cast<uint32_t>(c[w] >> sh) & 2047u], 1u);
        lds_barrier();
        find_threshold_bin<NT>(sm.hist, 2048, rem, sm.wave_tot, &sm.sh_bin, &sm.sh_above);
        const uint32_t tb = sm.sh_bin;
        rem -= sm.sh_above;
        prefix |= static_cast<uint64_t>(tb) << sh;
        pmask |= 2047ull << sh;
        bin_count = static_cast<int>(sm.hist[tb]);
        lds_barrier();
        if (sh == 0) break;
        sh = sh > 11 ? sh - 11 : 0;
    }
    if (tid == 0) {
        sm.n_chosen = 0;
        sm.n_short = 0;
    }
    lds_barrier();
#pragma unroll
    for (int w = 0; w < K; ++w) {
        if (cv[w]) {
            const uint64_t mk = c[w] & pmask;
            if (mk > prefix) sm.chosen[atomicAdd(&sm.n_chosen, 1)] = static_cast<int32_t>(~static_cast<uint32_t>(c[w]));
            else if (mk == prefix) sm.shortl[atomicAdd(&sm.n_short, 1)] = c[w];
        }
    }
    lds_barrier();
    rank_take_desc<NT>(sm.shortl, sm.n_short, rem, sm.chosen + (keep - rem));
    if (bitmap != nullptr && o <= 32 * kResBitmapWords) {
        constexpr int kWpt = kResBitmapWords / NT;
        for (int k = tid; k < kResBitmapWords; k += NT) bitmap[k] = 0u;
        lds_barrier();                                  // chosen complete, bitmap clear
        for (int k = tid; k < keep; k += NT) {
            const int v = sm.chosen[k];
            atomicOr(&bitmap[v >> 5], 1u << (v & 31));
        }
        if (tid == 0) out[keep] = o;                      // above every candidate
        lds_barrier();
        uint32_t wv[kWpt];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < kWpt; ++q) {
            wv[q] = bitmap[kWpt * tid + q];
            cnt += __popc(wv[q]);
        }
        int all;
        int base = block_exclusive_scan<NT, false>(cnt, sm.wave_tot, &all);   // wave_tot is not used again
#pragma unroll
        for (int q = 0; q < kWpt; ++q) {
            uint32_t bits = wv[q];
            while (bits) {
                const int bit = __ffs(bits) - 1;
                out[base++] = 32 * (kWpt * tid + q) + bit;
                bits &= bits - 1;
            }
        }
    } else {
        if (tid == 0) sm.chosen[keep] = o;
        rank_write_ascending<NT>(sm.chosen, keep + 1, out);
    }
    for (int k = keep + 1 + tid; k < budget; k += NT) out[k] = -1;
}

}  // namespace qsa
