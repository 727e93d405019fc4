// Fused index-select for decode rows (one query token per sequence, up to
// 262144 candidate blocks): the same scores and the same selection as
// index_scores_kernel followed by select_kernel, in two launches that spread
// each row over hundreds of workgroups.
//
//  decode_scan_kernel     B x G workgroups.  Scores every candidate block with
//                         the shared MFMA block_score (bit-identical to the
//                         index_scores path), stores them, and counts the top
//                         12 bits of each ordered key in an LDS histogram that
//                         is added to a per-sequence global histogram.  The
//                         last workgroup of a sequence to finish (ticket
//                         counter) finds the bin holding the threshold and
//                         clears the global histogram.  Optionally it also
//                         rotates the new K row into the cache (step 0).
//  decode_filter_kernel   B x F workgroups over the stored scores: keys above
//                         the threshold bin are appended to a list of winners,
//                         keys in the bin to a candidate list (wave-aggregated
//                         atomics).  The last workgroup of a sequence sorts the
//                         candidates in LDS, takes the ones still needed,
//                         merges, sorts ascending and writes sel; if the bin
//                         overflows LDS it runs the full radix select on the
//                         stored row instead.  It leaves the control words
//                         zeroed for the next call.
// Cross-workgroup hand-off uses the release/acquire pattern: results, then
// __threadfence(), then the ticket atomic; the last workgroup fences again
// before reading.  No workgroup ever waits on another, so nothing can hang.
#include "index_common.h"
#include "rope_common.h"
#include "select_common.h"

namespace qsa {

constexpr int kDecHistBits = 12;
constexpr int kDecHistBins = 1 << kDecHistBits;
constexpr int kDecShift = 32 - kDecHistBits;
constexpr int kDecCap = 4096;        // threshold-bin candidates sorted in LDS by the last workgroup
constexpr int kCtrl = 16;            // control words per sequence

enum { kDoneScan = 0, kDoneFilter, kNDef, kNCand, kBin, kAbove, kInBin };

struct DecodeWs {
    uint32_t* hist;     // [B][4096]
    uint32_t* ctrl;     // [B][16]
    int32_t* defl;      // [B][QSA_MAX_BUDGET]  keys above the threshold bin
    uint64_t* cand;     // [B][kDecCap]         keys in the threshold bin: key << 32 | ~j
};

size_t decode_select_ws_bytes(int batch) {
    return static_cast<size_t>(batch) *
           (kDecHistBins * 4 + kCtrl * 4 + QSA_MAX_BUDGET * 4 + kDecCap * 8);
}

static DecodeWs carve(void* ws, int batch) {
    char* p = static_cast<char*>(ws);
    DecodeWs w;
    w.hist = reinterpret_cast<uint32_t*>(p);
    p += static_cast<size_t>(batch) * kDecHistBins * 4;
    w.ctrl = reinterpret_cast<uint32_t*>(p);
    p += static_cast<size_t>(batch) * kCtrl * 4;
    w.defl = reinterpret_cast<int32_t*>(p);
    p += static_cast<size_t>(batch) * QSA_MAX_BUDGET * 4;
    w.cand = reinterpret_cast<uint64_t*>(p);
    return w;
}

__global__ __launch_bounds__(256) void decode_scan_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos, int budget, int wg_per_seq, int blocks_per_wg, float* __restrict__ scores,
    int64_t ss, DecodeWs ws, const uint16_t* __restrict__ k_new, int64_t kns,
    uint16_t* __restrict__ k_cache, int64_t kcs, InvFreq inv, int rope_k) {
    __shared__ uint32_t hist[kDecHistBins];
    __shared__ int wave_tot[4];
    __shared__ uint32_t sh_bin;
    __shared__ int sh_above, sh_last;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.x / wg_per_seq;
    const int g = blockIdx.x % wg_per_seq;
    const int p = pos.p[b];
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    const bool need_hist = keep > 0 && keep < o;

    if (rope_k && g == 0 && wave == 0)
        rope_row_wave(k_new + b * kns, k_cache + b * kcs + static_cast<int64_t>(p) * (kHkv * kD), kHkv,
                      static_cast<double>(p), inv, false);

    for (int k = tid; k < kDecHistBins; k += 256) hist[k] = 0;
    __syncthreads();

    const int c16 = lane & 15;
    const int G = lane >> 4;
    bf16x8_t a[4];
    load_index_a(q_idx + b * qs, 0, 1, a);
    const uint16_t* kb = kbar + b * kbs;
    float* sb = scores + b * ss;
    const int j_lo = g * blocks_per_wg;
    const int j_hi = min(o, j_lo + blocks_per_wg);
    for (int j0 = j_lo + wave * 64; j0 < j_hi; j0 += 256) {
        bf16x8_t bf[4][4];
#pragma unroll
        for (int n = 0; n < 4; ++n) load_index_b(kb, j0, n, j_hi, bf[n]);
        float s[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) s[n] = block_score(a, bf[n]);
        const int jj = j0 + 4 * c16;
        if (G == 0 && jj < j_hi) {
            *reinterpret_cast<float4*>(sb + jj) = make_float4(s[0], s[1], s[2], s[3]);
            if (need_hist) {
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    if (jj + n < j_hi) atomicAdd(&hist[score_key(s[n]) >> kDecShift], 1u);
            }
        }
    }
    __syncthreads();
    if (need_hist) {
        for (int k = tid; k < kDecHistBins; k += 256) {
            const uint32_t v = hist[k];
            if (v) atomicAdd(&ws.hist[static_cast<int64_t>(b) * kDecHistBins + k], v);
        }
    }
    __threadfence();
    __syncthreads();
    uint32_t* ctrl = ws.ctrl + b * kCtrl;
    if (tid == 0) sh_last = atomicAdd(&ctrl[kDoneScan], 1u) == static_cast<uint32_t>(wg_per_seq - 1);
    __syncthreads();
    if (!sh_last) return;
    __threadfence();
    if (need_hist) {
        for (int k = tid; k < kDecHistBins; k += 256)
            hist[k] = atomicExch(&ws.hist[static_cast<int64_t>(b) * kDecHistBins + k], 0u);
        __syncthreads();
        find_threshold_bin<256>(hist, kDecHistBins, keep, wave_tot, &sh_bin, &sh_above);
        if (tid == 0) {
            ctrl[kBin] = sh_bin;
            ctrl[kAbove] = static_cast<uint32_t>(sh_above);
            ctrl[kInBin] = hist[sh_bin];
        }
    }
    if (tid == 0) ctrl[kDoneScan] = 0;
}

__device__ __forceinline__ void wave_append(uint32_t* counter, bool pred, uint32_t* off_out) {
    const uint64_t m = __ballot(pred);
    const int lane = threadIdx.x & 63;
    uint32_t base = 0;
    if (m != 0) {
        if (lane == 0) base = atomicAdd(counter, static_cast<uint32_t>(__popcll(m)));
        base = __shfl(base, 0);
    }
    *off_out = base + static_cast<uint32_t>(__popcll(m & ((1ull << lane) - 1ull)));
}

struct FilterSmem {
    SelectSmem s;
    uint64_t cand[kDecCap];
    int sh_last;
};

__global__ __launch_bounds__(256) void decode_filter_kernel(
    const float* __restrict__ scores, int64_t ss, Positions pos, int budget, int wg_per_seq,
    int per_wg, DecodeWs ws, int32_t* __restrict__ sel, int64_t sels) {
    __shared__ FilterSmem sm;
    const int tid = threadIdx.x;
    const int b = blockIdx.x / wg_per_seq;
    const int g = blockIdx.x % wg_per_seq;
    const int p = pos.p[b];
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    const bool nontrivial = keep > 0 && keep < o;
    uint32_t* ctrl = ws.ctrl + b * kCtrl;
    const float* row = scores + b * ss;
    int32_t* out = sel + b * sels;

    if (nontrivial) {
        const uint32_t tbin = ctrl[kBin];
        int32_t* defl = ws.defl + static_cast<int64_t>(b) * QSA_MAX_BUDGET;
        uint64_t* cand = ws.cand + static_cast<int64_t>(b) * kDecCap;
        const int j_lo = g * per_wg;
        const int j_hi = min(o, j_lo + per_wg);
        for (int base = j_lo; base < j_hi; base += 4 * 256) {      // uniform trip count
            const int j4 = base + 4 * tid;
            const bool in = j4 < j_hi;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (in) v = *reinterpret_cast<const float4*>(row + j4);
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j4 + e;
                const bool valid = in && j < j_hi;
                const uint32_t key = score_key(f[e]);
                const uint32_t bin = key >> kDecShift;
                const bool is_def = valid && bin > tbin;
                const bool is_cand = valid && bin == tbin;
                uint32_t off;
                wave_append(&ctrl[kNDef], is_def, &off);
                if (is_def && off < static_cast<uint32_t>(QSA_MAX_BUDGET)) defl[off] = j;
                wave_append(&ctrl[kNCand], is_cand, &off);
                if (is_cand && off < static_cast<uint32_t>(kDecCap))
                    cand[off] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
            }
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) sm.sh_last = atomicAdd(&ctrl[kDoneFilter], 1u) == static_cast<uint32_t>(wg_per_seq - 1);
    __syncthreads();
    if (!sm.sh_last) return;
    __threadfence();

    if (!nontrivial) {
        trivial_selection(keep, o, budget, out, 256);
    } else {
        const int above = static_cast<int>(ctrl[kAbove]);
        const int inbin = static_cast<int>(ctrl[kInBin]);
        const int remaining = keep - above;
        if (inbin <= kDecCap) {
            const int32_t* defl = ws.defl + static_cast<int64_t>(b) * QSA_MAX_BUDGET;
            const uint64_t* cand = ws.cand + static_cast<int64_t>(b) * kDecCap;
            for (int k = tid; k < above; k += 256) sm.s.chosen[k] = defl[k];
            const int np2 = next_pow2(inbin);
            for (int k = tid; k < np2; k += 256) sm.cand[k] = (k < inbin) ? cand[k] : 0ull;
            __syncthreads();
            bitonic_sort<256, uint64_t, true>(sm.cand, np2);
            for (int k = tid; k < remaining; k += 256)
                sm.s.chosen[above + k] = static_cast<int32_t>(~static_cast<uint32_t>(sm.cand[k]));
            __syncthreads();
            write_selection<256>(sm.s, keep, o, budget, out);
        } else {
            select_row<256>(row, o, keep, budget, out, sm.s);
        }
    }
    __syncthreads();
    if (tid == 0) {
        ctrl[kNDef] = 0;
        ctrl[kNCand] = 0;
        ctrl[kDoneFilter] = 0;
    }
}

hipError_t launch_decode_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                                      int64_t kbs, const Positions& pos, int batch, int budget,
                                      float* scores, int64_t ss, int32_t* sel, int64_t sels, void* ws,
                                      const uint16_t* k_new, int64_t kns, uint16_t* k_cache,
                                      int64_t kcs, double rope_theta, hipStream_t stream) {
    int o_max = 0;
    for (int b = 0; b < batch; ++b) o_max = max(o_max, pos.p[b] / kBlock);
    // scan: ~1024 workgroups in total, ranges in whole 256-block steps
    int wg_scan = max(1, min((o_max + 255) / 256, (1024 + batch - 1) / batch));
    int per_scan = ((o_max + wg_scan - 1) / wg_scan + 255) / 256 * 256;
    if (per_scan == 0) per_scan = 256;
    wg_scan = max(1, (o_max + per_scan - 1) / per_scan);
    // filter: up to 64 workgroups per sequence, ranges in whole 1024-score steps
    int wg_filt = max(1, min((o_max + 4095) / 4096, 64));
    int per_filt = ((o_max + wg_filt - 1) / wg_filt + 1023) / 1024 * 1024;
    if (per_filt == 0) per_filt = 1024;
    wg_filt = max(1, (o_max + per_filt - 1) / per_filt);

    const DecodeWs w = carve(ws, batch);
    const InvFreq inv = make_inv_freq(rope_theta > 0.0 ? rope_theta : 1.0e7);
    hipLaunchKernelGGL(decode_scan_kernel, dim3(static_cast<unsigned>(batch * wg_scan)), dim3(256), 0, stream,
                       q_idx, qs, kbar, kbs, pos, budget, wg_scan, per_scan, scores, ss, w, k_new, kns,
                       k_cache, kcs, inv, (rope_theta > 0.0 && k_new != nullptr) ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_filter_kernel, dim3(static_cast<unsigned>(batch * wg_filt)), dim3(256), 0,
                       stream, scores, ss, pos, budget, wg_filt, per_filt, w, sel, sels);
    return hipGetLastError();
}

}  // namespace qsa
