// Fused index-select for decode rows (1 to 4 consecutive query tokens per
// sequence, up to 262144 candidate blocks each; a row is one token of one
// sequence): the same scores and the same selection as index_scores_kernel
// followed by select_kernel, spread over hundreds of workgroups per row.  The
// tokens of a sequence share one pass over its block keys (they are columns
// of the same matrix-core tiles).  Three launches; every hand-off between workgroups
// goes through a kernel boundary or a device-scope atomic, never through an
// in-kernel fence (an agent-scope fence writes back and invalidates the L2 of
// the XCD, which costs microseconds per workgroup on this part):
//
//  decode_scan_kernel      B x G workgroups, long-lived waves that stream
//                          64-block groups with the next group's loads in
//                          flight.  Scores every candidate with the shared MFMA
//                          block_scores (bit-identical to index_scores_kernel),
//                          stores the scores, counts the top 12 bits of each
//                          ordered key in an LDS histogram per token and adds
//                          them to per-row global histograms.  In a decode step
//                          it also appends the new rows (append_rows).
//  decode_filter_kernel    rows x F workgroups: each finds the threshold bin from
//                          the global histogram, then collects its slice's keys
//                          above the bin (winners) and in the bin (candidates)
//                          in LDS and appends them to per-row lists with
//                          one atomic reservation per list.
//  decode_finalize_kernel  one workgroup per row: sorts the candidates, takes the ones
//                          still needed, merges, sorts ascending and writes sel;
//                          if the bin overflowed the list it runs the full radix
//                          select on the stored row.  Leaves the histogram and
//                          counters zeroed for the next call.
#include "compress_common.h"
#include "index_common.h"
#include "rope_common.h"
#include "select_common.h"

namespace qsa {

constexpr int kDecHistBits = 12;
constexpr int kDecHistBins = 1 << kDecHistBits;
constexpr int kDecShift = 32 - kDecHistBits;
constexpr int kDecCap = 4096;        // threshold-bin candidates sorted in LDS by the last workgroup
constexpr int kCtrl = 16;            // control words per row

enum { kDoneScan = 0, kDoneFilter, kNDef, kNCand, kBin, kAbove, kInBin };

// per row r = b * tq + t (token t of sequence b, at position q_pos[b] + t)
struct DecodeWs {
    uint32_t* hist;     // [rows][4096]
    uint32_t* ctrl;     // [rows][16]
    int32_t* defl;      // [rows][QSA_MAX_BUDGET]  keys above the threshold bin
    uint64_t* cand;     // [rows][kDecCap]         keys in the threshold bin: key << 32 | ~j
};

size_t decode_select_ws_bytes(int rows) {
    return static_cast<size_t>(rows) *
           (kDecHistBins * 4 + kCtrl * 4 + QSA_MAX_BUDGET * 4 + kDecCap * 8);
}

static DecodeWs carve(void* ws, int rows) {
    char* p = static_cast<char*>(ws);
    DecodeWs w;
    w.hist = reinterpret_cast<uint32_t*>(p);
    p += static_cast<size_t>(rows) * kDecHistBins * 4;
    w.ctrl = reinterpret_cast<uint32_t*>(p);
    p += static_cast<size_t>(rows) * kCtrl * 4;
    w.defl = reinterpret_cast<int32_t*>(p);
    p += static_cast<size_t>(rows) * QSA_MAX_BUDGET * 4;
    w.cand = reinterpret_cast<uint64_t*>(p);
    return w;
}

// Device copy of DecodeAppend, with the rotary table.
struct AppendArgs {
    const uint16_t* k_new;
    int64_t kns;
    uint16_t* k_cache;
    const uint16_t* v_new;
    int64_t vns;
    uint16_t* v_cache;
    int64_t kvs;
    const uint16_t* k_idx_new;
    int64_t kins;
    uint16_t* k_idx;
    int64_t kis;
    uint16_t* kbar;
    int64_t kbs;
    InvFreq inv;
};

// The rows of one sequence's new tokens p0 .. p0 + tq - 1: wave 0 rotates the
// K rows into the cache (step 0), wave 1 copies the V rows, wave 2 copies the
// indexer key rows and, for each new token that completes its block,
// compresses the block (step 1), taking the block's new rows from the inputs
// (not back through memory).  With one token per sequence this runs in the
// first scan workgroup of the sequence: the scan reads blocks j < p0 / 4 only
// and attention runs in a later launch.  With several, a block an earlier new
// token completes is a candidate of the later ones, so it runs in its own
// launch (decode_append_kernel) before the scan.
// With kPaged the caches are page pools: token rows and block-key rows go
// through the block table (pm).
template <bool kPaged>
__device__ __forceinline__ void append_rows(const AppendArgs& ap, const PageMap& pm, int b, int p0, int tq,
                                            int wave) {
    const int lane = threadIdx.x & 63;
    // element offset of token x's row (row_elems per token) in its cache
    auto tok_off = [&](int64_t seq_stride, int x, int row_elems) -> int64_t {
        return kPaged ? phys_token(pm, b, x) * row_elems : b * seq_stride + static_cast<int64_t>(x) * row_elems;
    };
    if (wave == 0 && ap.k_new != nullptr)
        for (int t = 0; t < tq; ++t)
            rope_row_wave(ap.k_new + b * ap.kns + t * (kHkv * kD), ap.k_cache + tok_off(ap.kvs, p0 + t, kHkv * kD),
                          kHkv, static_cast<double>(p0 + t), ap.inv, false);
    if (wave == 1 && ap.v_new != nullptr)        // 2 x 256 values per row: 16 B per lane
        for (int t = 0; t < tq; ++t)
            *reinterpret_cast<uint4*>(ap.v_cache + tok_off(ap.kvs, p0 + t, kHkv * kD) + 8 * lane) =
                *reinterpret_cast<const uint4*>(ap.v_new + b * ap.vns + t * (kHkv * kD) + 8 * lane);
    if (wave == 2 && ap.k_idx != nullptr && lane < kDi / 8) {
        uint16_t* kr = ap.k_idx + 8 * lane;
        const uint16_t* kn = ap.k_idx_new != nullptr ? ap.k_idx_new + b * ap.kins + 8 * lane : nullptr;
        auto row = [&](int x) -> uint4 {           // indexer key row x of this sequence, this lane's 8 dims
            return (kn != nullptr && x >= p0) ? *reinterpret_cast<const uint4*>(kn + (x - p0) * kDi)
                                              : *reinterpret_cast<const uint4*>(kr + tok_off(ap.kis, x, kDi));
        };
        if (kn != nullptr)
            for (int t = 0; t < tq; ++t)
                *reinterpret_cast<uint4*>(kr + tok_off(ap.kis, p0 + t, kDi)) =
                    *reinterpret_cast<const uint4*>(kn + t * kDi);
        for (int t = 0; t < tq; ++t) {
            const int x = p0 + t;
            if (x % kBlock != kBlock - 1) continue;
            uint4 r[kBlock];
#pragma unroll
            for (int i = 0; i < kBlock; ++i) r[i] = row(x - (kBlock - 1) + i);
            const int64_t kb_off = kPaged ? phys_block(pm, b, x / kBlock) * kDi
                                          : b * ap.kbs + static_cast<int64_t>(x / kBlock) * kDi;
            *reinterpret_cast<uint4*>(ap.kbar + kb_off + 8 * lane) = compress_rows(r);
        }
    }
}

template <bool kPaged>
__global__ __launch_bounds__(192) void decode_append_kernel(Positions pos, int tq, AppendArgs ap, PageMap pm) {
    append_rows<kPaged>(ap, pm, blockIdx.x, pos.p[blockIdx.x], tq, threadIdx.x >> 6);
}

// hist: tq x 4096 words of dynamic LDS (one histogram per token).  kPaged:
// kbar (and the caches the append writes) are page pools behind pm.
template <int STEPS, bool kPaged>
__global__ __launch_bounds__(256) void decode_scan_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos, int budget, int tq, int wg_per_seq, float* __restrict__ scores,
    int64_t ss, int64_t sld, DecodeWs ws, AppendArgs ap, int append, PageMap pm) {
    extern __shared__ uint32_t hist[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // scalar: loop control stays uniform
    const int b = blockIdx.x / wg_per_seq;
    const int g = blockIdx.x % wg_per_seq;
    const int p0 = pos.p[b];
    const int o_last = (p0 + tq - 1) / kBlock;           // blocks below the last token's own block

    if (append && g == 0) append_rows<kPaged>(ap, pm, b, p0, tq, wave);

    for (int k = tid; k < tq * kDecHistBins; k += 256) hist[k] = 0;
    lds_barrier();          // the appended rows' stores need not land before the scan

    const int c16 = lane & 15;
    const int G = lane >> 4;
    // column c16 < tq: token c16, its candidates j < o_c; histogram only when
    // its selection is not trivial
    const int o_c = (p0 + c16) / kBlock;
    const int keep_c = min(budget - 1, o_c);
    const bool col_hist = c16 < tq && keep_c > 0 && keep_c < o_c;
    uint32_t* hist_c = hist + (c16 < tq ? c16 : 0) * kDecHistBins;
    bf16x8_t qf[kIdxSlices];
    load_index_q(q_idx + b * qs, 0, tq, qf);            // tokens 0 .. tq-1 in columns 0 .. tq-1, zero elsewhere
    const uint16_t* kb = kPaged ? kbar : kbar + b * kbs;
    float* sb = scores + b * ss + (c16 < tq ? c16 : 0) * sld;
    const int j_lo = g * (256 * STEPS);
    const int j_hi = min(o_last, j_lo + 256 * STEPS);
    auto load_tile = [&](int jt, bf16x8_t (&kf)[4]) {
        if constexpr (kPaged)
            load_index_k_paged(kb, pm, b, jt, j_hi, kf);
        else
            load_index_k(kb, jt, j_hi, kf);
    };
    // two named buffers, loop unrolled by two: one group computes while the
    // next is in flight (the next-group address is clamped, never skipped)
    auto step_of = [&](int j) { return (j < j_hi) ? j : (j_hi - 1) / 64 * 64; };
    // 4 tiles of 16 blocks; the lanes of column c < tq hold token c's scores,
    // 4 consecutive blocks each
    const int lim_c = min(j_hi, o_c);
    auto score_group = [&](const bf16x8_t (&kf)[4][4], int j0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const f32x4_t s = block_scores(kf[nt], qf);
            const int jj = j0 + 16 * nt + 4 * G;
            if (c16 < tq && jj < j_hi) {
                *reinterpret_cast<float4*>(sb + jj) = make_float4(s[0], s[1], s[2], s[3]);
                if (col_hist) {
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        if (jj + n < lim_c) atomicAdd(&hist_c[score_key(s[n]) >> kDecShift], 1u);
                }
            }
        }
    };
    // STEPS groups of 64 blocks per wave (stride 256 over the workgroup's
    // range), fully unrolled: straight-line code lets every wait count only
    // the loads it needs, so the next group is always in flight
    const int j0 = j_lo + wave * 64;
    if (j0 < j_hi) {
        bf16x8_t buf[2][4][4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) load_tile(j0 + 16 * nt, buf[0][nt]);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (st + 1 < STEPS) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    load_tile(step_of(j0 + 256 * (st + 1)) + 16 * nt, buf[(st + 1) & 1][nt]);
            }
            if (j0 + 256 * st < j_hi) score_group(buf[st & 1], j0 + 256 * st);
        }
    }
    lds_barrier();
    for (int t = 0; t < tq; ++t) {
        const int o_t = (p0 + t) / kBlock;
        const int keep_t = min(budget - 1, o_t);
        if (!(keep_t > 0 && keep_t < o_t)) continue;     // uniform
        uint32_t* gh = ws.hist + static_cast<int64_t>(b * tq + t) * kDecHistBins;
        for (int k = tid; k < kDecHistBins; k += 256) {
            const uint32_t v = hist[t * kDecHistBins + k];
            if (v) atomicAdd(&gh[k], v);
        }
    }
}

struct FilterSmem {
    alignas(16) uint32_t hist[kDecHistBins];
    int32_t def[QSA_MAX_BUDGET];
    uint64_t cand[kDecCap];
    int wave_tot[4];
    uint32_t sh_bin;
    int sh_above, n_def, n_cand, base_def, base_cand;
};

constexpr int kFiltPer = 4096;      // scores per filter workgroup: 4 float4 per thread

__global__ __launch_bounds__(256) void decode_filter_kernel(
    const float* __restrict__ scores, int64_t ss, int64_t sld, Positions pos, int budget, int tq, int wg_per_row,
    DecodeWs ws) {
    __shared__ FilterSmem sm;
    const int tid = threadIdx.x;
    const int r = blockIdx.x / wg_per_row;                 // row = token t of sequence b
    const int g = blockIdx.x % wg_per_row;
    const int b = r / tq;
    const int t = r % tq;
    const int p = pos.p[b] + t;
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    if (!(keep > 0 && keep < o)) return;                 // trivial rows need no filter
    uint32_t* ctrl = ws.ctrl + r * kCtrl;

    // the global histogram the scan completed, then this workgroup's scores
    // (independent of the threshold): all issued at once, the histogram
    // first so that waiting for it leaves the scores in flight through the
    // threshold search (the barriers below wait for LDS work only)
    const uint4* gh = reinterpret_cast<const uint4*>(ws.hist + static_cast<int64_t>(r) * kDecHistBins);
    uint4 hv[kDecHistBins / 1024];
#pragma unroll
    for (int it = 0; it < kDecHistBins / 1024; ++it) hv[it] = gh[tid + 256 * it];
    const float* row = scores + b * ss + t * sld;
    const int j_lo = g * kFiltPer;
    const int j_hi = min(o, j_lo + kFiltPer);
    float4 v[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int j4 = min(j_lo + 4 * tid + 1024 * it, (o - 1) & ~3);   // clamped: always a legal load
        v[it] = *reinterpret_cast<const float4*>(row + j4);
    }
#pragma unroll
    for (int it = 0; it < kDecHistBins / 1024; ++it) reinterpret_cast<uint4*>(sm.hist)[tid + 256 * it] = hv[it];
    if (tid == 0) {
        sm.n_def = 0;
        sm.n_cand = 0;
    }
    lds_barrier();
    find_threshold_bin<256>(sm.hist, kDecHistBins, keep, sm.wave_tot, &sm.sh_bin, &sm.sh_above);
    const uint32_t tbin = sm.sh_bin;
    if (g == 0 && tid == 0) {
        ctrl[kBin] = tbin;
        ctrl[kAbove] = static_cast<uint32_t>(sm.sh_above);
        ctrl[kInBin] = sm.hist[tbin];
    }

#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int j4 = j_lo + 4 * tid + 1024 * it;
        const float f[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j4 + e;
            if (j >= j_hi) continue;
            const uint32_t key = score_key(f[e]);
            const uint32_t bin = key >> kDecShift;
            if (bin > tbin) {
                const int k = atomicAdd(&sm.n_def, 1);
                if (k < QSA_MAX_BUDGET) sm.def[k] = j;
            } else if (bin == tbin) {
                const int k = atomicAdd(&sm.n_cand, 1);
                if (k < kDecCap) sm.cand[k] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~j);
            }
        }
    }
    lds_barrier();
    const int nd = min(sm.n_def, QSA_MAX_BUDGET);
    const int nc = sm.n_cand;
    if (tid == 0) {
        sm.base_def = nd ? static_cast<int>(atomicAdd(&ctrl[kNDef], static_cast<uint32_t>(nd))) : 0;
        sm.base_cand = nc ? static_cast<int>(atomicAdd(&ctrl[kNCand], static_cast<uint32_t>(nc))) : 0;
    }
    lds_barrier();
    int32_t* defl = ws.defl + static_cast<int64_t>(r) * QSA_MAX_BUDGET;
    uint64_t* cand = ws.cand + static_cast<int64_t>(r) * kDecCap;
    for (int k = tid; k < nd; k += 256)
        if (sm.base_def + k < QSA_MAX_BUDGET) defl[sm.base_def + k] = sm.def[k];
    for (int k = tid; k < min(nc, kDecCap); k += 256)
        if (sm.base_cand + k < kDecCap) cand[sm.base_cand + k] = sm.cand[k];
}

constexpr int kFinNT = 1024;                 // finalize threads
constexpr int kBitmapWords = 8192;           // ascending order by bitmap for candidates j < 262144

struct FinalizeSmem {
    union {
        SelectSmem s;                                        // overflow: full radix select
        struct {
            uint32_t bm[kBitmapWords];                       // one bit per candidate block
            alignas(16) int32_t chosen[QSA_MAX_BUDGET];      // selection, any order
            alignas(16) uint64_t cand[kDecCap];              // threshold-bin candidates
            uint32_t h2[kDecHistBins];                       // second radix level over them
            alignas(16) uint64_t sub[kDecCap];               // members of the cut sub-bin
            int wave_tot[16];
            uint32_t sh_bin;
            int sh_above, n_taken, n_sub;
        } m;
    } u;
};

__global__ __launch_bounds__(kFinNT) void decode_finalize_kernel(const float* __restrict__ scores, int64_t ss,
                                                                 int64_t sld, Positions pos, int budget, int tq,
                                                                 DecodeWs ws, int32_t* __restrict__ sel,
                                                                 int64_t sels) {
    __shared__ FinalizeSmem sm;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;                             // row = token t of sequence b
    const int b = r / tq;
    const int t = r % tq;
    const int p = pos.p[b] + t;
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    int32_t* out = sel + b * sels + t * budget;
    uint32_t* ctrl = ws.ctrl + r * kCtrl;
    if (trivial_selection(keep, o, budget, out, kFinNT)) return;   // nothing was accumulated

    // every load of both lists in flight at once, with the control words (the
    // lists have fixed capacities: unused tails are read and dropped)
    const int32_t* __restrict__ defl = ws.defl + static_cast<int64_t>(r) * QSA_MAX_BUDGET;
    const uint64_t* __restrict__ cg = ws.cand + static_cast<int64_t>(r) * kDecCap;
    int32_t dv[QSA_MAX_BUDGET / kFinNT];
    uint64_t cv[kDecCap / kFinNT];
#pragma unroll
    for (int it = 0; it < QSA_MAX_BUDGET / kFinNT; ++it) dv[it] = defl[tid + kFinNT * it];
#pragma unroll
    for (int it = 0; it < kDecCap / kFinNT; ++it) cv[it] = cg[tid + kFinNT * it];
    const int above = static_cast<int>(ctrl[kAbove]);
    const int inbin = static_cast<int>(ctrl[kInBin]);
    const int remaining = keep - above;
    if (inbin > kDecCap) {
        select_row<kFinNT>(scores + b * ss + t * sld, o, keep, budget, out, sm.u.s);
    } else {
        int32_t* chosen = sm.u.m.chosen;
        const bool bitmap = o <= 32 * kBitmapWords;             // every chosen j < o has a bit; o goes last
        if (bitmap)
            for (int k = tid; k < kBitmapWords; k += kFinNT) sm.u.m.bm[k] = 0u;
#pragma unroll
        for (int it = 0; it < QSA_MAX_BUDGET / kFinNT; ++it)
            if (tid + kFinNT * it < above) chosen[tid + kFinNT * it] = dv[it];
        if (tid == 0) chosen[keep] = o;
        // candidates of the threshold bin share the top 12 key bits: a second
        // radix level on the next 12 bits (LDS histogram) splits them into
        // those surely taken, the few in the sub-bin holding the cut, and the rest
        uint64_t* lc = sm.u.m.cand;
        uint32_t* h2 = sm.u.m.h2;
        for (int k = tid; k < kDecHistBins; k += kFinNT) h2[k] = 0u;
#pragma unroll
        for (int it = 0; it < kDecCap / kFinNT; ++it)
            if (tid + kFinNT * it < inbin) lc[tid + kFinNT * it] = cv[it];
        if (tid == 0) sm.u.m.n_taken = 0;
        lds_barrier();
        for (int k = tid; k < inbin; k += kFinNT)
            atomicAdd(&h2[static_cast<uint32_t>(lc[k] >> 40) & (kDecHistBins - 1)], 1u);
        lds_barrier();
        find_threshold_bin<kFinNT>(h2, kDecHistBins, remaining, sm.u.m.wave_tot, &sm.u.m.sh_bin, &sm.u.m.sh_above);
        const uint32_t t2 = sm.u.m.sh_bin;
        const int above2 = sm.u.m.sh_above;                   // taken outright
        const int need2 = remaining - above2;                 // still to take from sub-bin t2
        // members of the cut sub-bin go to a short list; the rest are decided here
        uint64_t* sub = sm.u.m.sub;
        if (tid == 0) sm.u.m.n_sub = 0;
        lds_barrier();
        for (int i = tid; i < inbin; i += kFinNT) {
            const uint64_t x = lc[i];
            const uint32_t d2 = static_cast<uint32_t>(x >> 40) & (kDecHistBins - 1);
            if (d2 > t2)
                chosen[above + atomicAdd(&sm.u.m.n_taken, 1)] = static_cast<int32_t>(~static_cast<uint32_t>(x));
            else if (d2 == t2)
                sub[atomicAdd(&sm.u.m.n_sub, 1)] = x;
        }
        lds_barrier();
        const int n_sub = sm.u.m.n_sub;
        int32_t* dst = chosen + above + above2;
        if (n_sub <= 256) {
            // rank among the few members of the sub-bin: full key, then index
            for (int i = tid; i < n_sub; i += kFinNT) {
                const uint64_t x = sub[i];
                int r = 0;
#pragma unroll 8
                for (int k = 0; k < n_sub; ++k) r += sub[k] > x ? 1 : 0;
                if (r < need2) dst[r] = static_cast<int32_t>(~static_cast<uint32_t>(x));
            }
        } else {
            const int np2 = next_pow2(n_sub);
            for (int k = n_sub + tid; k < np2; k += kFinNT) sub[k] = 0ull;
            lds_barrier();
            bitonic_sort<kFinNT, uint64_t, true>(sub, np2);
            for (int k = tid; k < need2; k += kFinNT) dst[k] = static_cast<int32_t>(~static_cast<uint32_t>(sub[k]));
        }
        lds_barrier();
        if (bitmap) {
            for (int k = tid; k < keep; k += kFinNT) {
                const int v = chosen[k];
                atomicOr(&sm.u.m.bm[v >> 5], 1u << (v & 31));
            }
            if (tid == 0) out[keep] = o;                     // above every candidate
            lds_barrier();
            // thread t owns words 8t .. 8t+7: prefix count of set bits, then emit in order
            constexpr int kWpt = kBitmapWords / kFinNT;
            uint32_t w[kWpt];
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < kWpt; ++q) {
                w[q] = sm.u.m.bm[kWpt * tid + q];
                cnt += __popc(w[q]);
            }
            int total;
            int base = block_exclusive_scan<kFinNT>(cnt, sm.u.m.wave_tot, &total);
#pragma unroll
            for (int q = 0; q < kWpt; ++q) {
                uint32_t bits = w[q];
                while (bits) {
                    const int bit = __ffs(bits) - 1;
                    out[base++] = 32 * (kWpt * tid + q) + bit;
                    bits &= bits - 1;
                }
            }
        } else {
            rank_write_ascending<kFinNT>(chosen, keep + 1, out);
        }
        for (int k = keep + 1 + tid; k < budget; k += kFinNT) out[k] = -1;
    }
    lds_barrier();
    uint32_t* gh = ws.hist + static_cast<int64_t>(r) * kDecHistBins;
    for (int k = tid; k < kDecHistBins; k += kFinNT) gh[k] = 0u;
    if (tid < kCtrl) ctrl[tid] = 0u;
}

hipError_t launch_decode_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                                      int64_t kbs, const Positions& pos, int batch, int tq, int budget,
                                      float* scores, int64_t ss, int64_t sld, int32_t* sel, int64_t sels,
                                      void* ws, const DecodeAppend* append, const PageMap* pm,
                                      hipStream_t stream) {
    const int rows = batch * tq;
    int o_max = 0;
    for (int b = 0; b < batch; ++b) o_max = max(o_max, (pos.p[b] + tq - 1) / kBlock);
    // scan: 256 * STEPS blocks per workgroup; STEPS is the largest of 8, 4, 2, 1
    // that still gives about 2 workgroups per CU
    const int64_t groups = static_cast<int64_t>(batch) * ((o_max + 255) / 256);
    const int steps = groups >= 8 * 512 ? 8 : groups >= 4 * 512 ? 4 : groups >= 2 * 512 ? 2 : 1;
    const int wg_scan = max(1, (o_max + 256 * steps - 1) / (256 * steps));
    // filter: kFiltPer scores per workgroup
    const int wg_filt = max(1, (o_max + kFiltPer - 1) / kFiltPer);

    const DecodeWs w = carve(ws, rows);
    AppendArgs ap{};
    if (append != nullptr) {
        ap.k_new = append->k_new;
        ap.kns = append->kns;
        ap.k_cache = append->k_cache;
        ap.v_new = append->v_new;
        ap.vns = append->vns;
        ap.v_cache = append->v_cache;
        ap.kvs = append->kvs;
        ap.k_idx_new = append->k_idx_new;
        ap.kins = append->kins;
        ap.k_idx = append->k_idx;
        ap.kis = append->kis;
        ap.kbar = append->kbar;
        ap.kbs = append->kbs;
        ap.inv = make_inv_freq(append->rope);
    }
    hipError_t e;
    // one token per sequence: the rows are appended by the scan; several: first,
    // because a block an earlier new token completes is scored for the later ones
    int scan_appends = append != nullptr ? 1 : 0;
    const PageMap pmv = pm != nullptr ? *pm : PageMap{};
    if (append != nullptr && tq > 1) {
        if (pm != nullptr)
            hipLaunchKernelGGL(decode_append_kernel<true>, dim3(static_cast<unsigned>(batch)), dim3(192), 0, stream,
                               pos, tq, ap, pmv);
        else
            hipLaunchKernelGGL(decode_append_kernel<false>, dim3(static_cast<unsigned>(batch)), dim3(192), 0, stream,
                               pos, tq, ap, pmv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        scan_appends = 0;
    }
    const dim3 grid(static_cast<unsigned>(batch * wg_scan));
    const size_t lds = static_cast<size_t>(tq) * kDecHistBins * 4;
#define QSA_SCAN(S, P)                                                                                       \
    hipLaunchKernelGGL((decode_scan_kernel<S, P>), grid, dim3(256), lds, stream, q_idx, qs, kbar, kbs, pos, \
                       budget, tq, wg_scan, scores, ss, sld, w, ap, scan_appends, pmv)
    if (pm != nullptr) {
        switch (steps) {
            case 8: QSA_SCAN(8, true); break;
            case 4: QSA_SCAN(4, true); break;
            case 2: QSA_SCAN(2, true); break;
            default: QSA_SCAN(1, true); break;
        }
    } else {
        switch (steps) {
            case 8: QSA_SCAN(8, false); break;
            case 4: QSA_SCAN(4, false); break;
            case 2: QSA_SCAN(2, false); break;
            default: QSA_SCAN(1, false); break;
        }
    }
#undef QSA_SCAN
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_filter_kernel, dim3(static_cast<unsigned>(rows * wg_filt)), dim3(256), 0,
                       stream, scores, ss, sld, pos, budget, tq, wg_filt, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(static_cast<unsigned>(rows)), dim3(kFinNT), 0, stream,
                       scores, ss, sld, pos, budget, tq, w, sel, sels);
    return hipGetLastError();
}

}  // namespace qsa
