// Fused index-select for decode rows (1 to 4 consecutive query tokens per
// sequence, up to 262144 candidate blocks each; a row is one token of one
// sequence): the same scores and the same selection as index_scores_kernel
// followed by select_kernel, spread over hundreds of workgroups per row.  The
// tokens of a sequence share one pass over its block keys (they are columns
// of the same matrix-core tiles).  Two launches:
//
//  decode_scan_kernel      B x G scan workgroups (plus, in a decode step, one
//                          side workgroup per sequence that appends the new
//                          rows and writes the rotated queries, off the scan's
//                          critical path).  A scan workgroup streams 64-block
//                          groups of its range with the next group's loads in
//                          flight, scores them with the shared MFMA
//                          block_scores (bit-identical to index_scores_kernel)
//                          and keeps the scores in LDS -- nothing else in the
//                          loop.  Then each wave, alone, finds a key T that at
//                          least K of its own blocks of every row reach (K a
//                          Poisson bound on its share of the selection) by a
//                          search over the key bits with ballots, and lists
//                          every candidate whose key is >= T; the workgroup
//                          writes its scores to global memory in full lines and
//                          its list entries to the row's candidate list (one
//                          reservation per workgroup and row), and max T per row.
//  decode_finalize_kernel  one workgroup per row: the exact top `keep` of the
//                          list (one radix level over the listed keys' own
//                          range, then the cut bin's members ranked), valid
//                          because every key >= max T is listed, so the list's
//                          cut is the row's when the cut key is >= max T;
//                          otherwise the list's cut is still a lower bound and
//                          the row is recovered from the listed keys above it
//                          plus the stored scores of the few waves that can
//                          hold more (or of the whole row); with tie floods or
//                          an overflowed list, the full radix select on the
//                          stored row.  Emits ascending through a block bitmap
//                          and leaves the row's control words zeroed.
// The host plans each call (scan_plan): blocks per workgroup and the list
// capacity per row, from the batch, tq, context and budget.
//
// Workspace: control words for the largest possible row count at offset 0
// (zero before the first call, left zero by every call, so one workspace
// serves calls of any shape), then the candidate lists (no initialisation).
#include "compress_common.h"
#include "index_common.h"
#include "rope_common.h"
#include "select_common.h"

namespace qsa {

constexpr int kDecCap = 4096;        // cut-bin members resolved in LDS by the finalize
constexpr int kCtrl = 16;            // control words per row
constexpr int kDecMaxRows = QSA_MAX_BATCH * QSA_MAX_DECODE_TQ;
constexpr int kListCap = 6144;       // candidates listed per row: the smallest capacity
constexpr int kListCapMax = 4 * kListCap;
constexpr int kListRowsMin = 32;     // the workspace lists at least this many rows' worth

enum { kNList = 0, kMaxT, kOverflow };

// per row r = b * tq + t (token t of sequence b, at position q_pos[b] + t)
struct DecodeWs {
    uint32_t* ctrl;     // [kDecMaxRows][kCtrl]   zero between calls
    uint64_t* list;     // [rows][cap]            key << 32 | ~j, any order
    int cap;            // list entries per row in this call: kListCap, 2 kListCap or 4 kListCap
    int steps;          // scan geometry: 256 * steps blocks per workgroup,
    int wg;             // wg workgroups per sequence (4 waves each)
};

// The lists take max(rows, kListRowsMin) x kListCap entries, so a call with
// fewer rows may give each row a longer list (2x up to 16 rows, 4x up to 8).
size_t decode_select_ws_bytes(int rows) {
    return static_cast<size_t>(kDecMaxRows) * kCtrl * 4 +
           static_cast<size_t>(max(rows, kListRowsMin)) * kListCap * 8;
}

// The largest list capacity per row the workspace holds for `rows` rows.
static int list_cap_avail(int rows) {
    int c = kListCap;
    while (2 * c <= kListCapMax && static_cast<int64_t>(rows) * 2 * c <= int64_t{max(rows, kListRowsMin)} * kListCap)
        c *= 2;
    return c;
}

static DecodeWs carve(void* ws, int cap, int steps, int wg) {
    char* p = static_cast<char*>(ws);
    DecodeWs w;
    w.ctrl = reinterpret_cast<uint32_t*>(p);
    w.list = reinterpret_cast<uint64_t*>(p + static_cast<size_t>(kDecMaxRows) * kCtrl * 4);
    w.cap = cap;
    w.steps = steps;
    w.wg = wg;
    return w;
}

// Candidates a wave lists for a row keeping `keep` of o candidates, n_w of
// them among the wave's blocks: with blocks ranked at random the wave holds
// about Poisson(m) of the selection, m = keep n_w / o, and m + 5.5 sqrt(m) + 4
// bounds that count except with probability below 1e-7 (checked against the
// Poisson quantiles for m from 0.01 to 400; at most 3 above them).  The cut
// is exact whatever the count: more only costs list space, fewer sends skewed
// rows to the slower exact path.
__host__ __device__ inline int wave_keep(int keep, int o, int n_w) {
    const float m = static_cast<float>(keep) * static_cast<float>(n_w) / static_cast<float>(o);
    return min(n_w, static_cast<int>(ceilf(m + 5.5f * sqrtf(m) + 4.f)));
}

constexpr int kLaneMaxKeep = 64;     // largest kw whose threshold comes from the lanes' two largest keys

// Entries a wave of n_w blocks lists for a row, bounded from above for blocks
// ranked at random: only a lane's third or later key can reach T without
// being one of the 128 values T is taken from, which keeps the count within
// kw (1 + (kw / 64)^2) (simulated means: 11.02 for kw = 11 and 8 keys per
// lane, 19.2 for 19 and 8, 28.6 for 28 and 16, 44.3 for 42 and 32); with the
// exact search, kw.
static double wave_listed(int kw, int n_w) {
    if (kw >= n_w) return n_w;
    if (kw > kLaneMaxKeep) return kw;
    return kw * (1.0 + (kw / 64.0) * (kw / 64.0));
}

// Queries of a decode step rotated for attention (q_rot [B][tq][24][256]).
struct QrotArgs {
    const uint16_t* q;      // unrotated [B][tq][24][256], sequence stride qs (null: not written)
    int64_t qs;
    uint16_t* q_rot;        // [B * tq][24][256]
};

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

constexpr int kEmitPerRow = 512;     // candidates one scan workgroup lists per row (LDS)

struct ScanSmem {
    uint64_t emit[kMaxDecodeTq][kEmitPerRow];
    int n_emit[kMaxDecodeTq];
    uint32_t max_t[kMaxDecodeTq];
    int base[kMaxDecodeTq];
};

// Grid: n_side side workgroups first (one per sequence when the step appends
// rows or rotates queries, else none), then B x wg_per_seq scan workgroups.
// Dynamic LDS: tq x (256 * STEPS) scores.  kPaged: kbar (and the caches the
// append writes) are page pools behind pm.
template <int STEPS, bool kPaged>
__global__ __launch_bounds__(256) void decode_scan_kernel(
    const uint16_t* __restrict__ q_idx, int64_t qs, const uint16_t* __restrict__ kbar, int64_t kbs,
    Positions pos, int budget, int tq, int n_side, int wg_per_seq, float* __restrict__ scores,
    int64_t ss, int64_t sld, DecodeWs ws, AppendArgs ap, int append, QrotArgs qr, PageMap pm) {
    constexpr int R = 256 * STEPS;                      // blocks per scan workgroup
    extern __shared__ float lds_sc[];                   // [tq][R]
    __shared__ ScanSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // scalar: loop control stays uniform

    if (static_cast<int>(blockIdx.x) < n_side) {
        // side workgroup of sequence b: append the new rows, rotate the queries
        const int b = blockIdx.x;
        const int p0 = pos.p[b];
        if (append) append_rows<kPaged>(ap, pm, b, p0, tq, wave);
        if (qr.q != nullptr)
            for (int t = 0; t < tq; ++t)
                rope_row_wave(qr.q + b * qr.qs + (t * kHq + 6 * wave) * kD,
                              qr.q_rot + (static_cast<int64_t>(b * tq + t) * kHq + 6 * wave) * kD, 6,
                              static_cast<double>(p0 + t), ap.inv, false);
        return;
    }
    const int bid = blockIdx.x - n_side;
    const int b = bid / wg_per_seq;
    const int g = bid % wg_per_seq;
    const int p0 = pos.p[b];
    const int o_last = (p0 + tq - 1) / kBlock;           // blocks below the last token's own block

    const int c16 = lane & 15;
    const int G = lane >> 4;
    if (tid < kMaxDecodeTq) {
        sm.n_emit[tid] = 0;
        sm.max_t[tid] = 0u;
    }
    lds_barrier();
    bf16x8_t qf[kIdxSlices];
    load_index_q(q_idx + b * qs, 0, tq, qf);            // tokens 0 .. tq-1 in columns 0 .. tq-1, zero elsewhere
    const uint16_t* kb = kPaged ? kbar : kbar + b * kbs;
    float* lb = lds_sc + (c16 < tq ? c16 : 0) * R;
    const int j_lo = g * R;
    const int j_hi = min(o_last, j_lo + R);
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
    // 4 consecutive blocks each, kept in LDS
    auto score_group = [&](const bf16x8_t (&kf)[4][4], int j0) {
        f32x4_t acc[4];
        block_scores4(kf, qf, acc);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int jj = j0 + 16 * nt + 4 * G;
            if (c16 < tq && jj < j_hi)
                *reinterpret_cast<float4*>(lb + (jj - j_lo)) = make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
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
    // Per row, this wave's candidates: its blocks j0 + 256 st + lane (one per
    // step) -- it reads back only what it wrote, so no workgroup barrier.
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // this wave's LDS stores done
    for (int t = 0; t < tq; ++t) {
        const int o_t = (p0 + t) / kBlock;
        const int keep_t = min(budget - 1, o_t);
        if (!(keep_t > 0 && keep_t < o_t)) continue;     // uniform
        const int lim = min(j_hi, o_t);
        uint32_t key[STEPS];
        bool ok[STEPS];
        int n_w = 0;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int j = j0 + 256 * st + lane;
            ok[st] = j < lim;
            key[st] = ok[st] ? score_key(lds_sc[t * R + (j - j_lo)]) : 0u;
            n_w += __popcll(__ballot(ok[st]));
        }
        if (n_w == 0) continue;                          // uniform
        const int kw = wave_keep(keep_t, o_t, n_w);
        // T with at least kw of the wave's keys >= T (0: every candidate
        // listed), built from the top bit down, keeping a bit while enough
        // keys reach the prefix.  For kw <= kLaneMaxKeep it is the kw-th
        // largest of the 128 values made of each lane's two largest keys (at
        // most the kw-th largest key: kw distinct keys reach it), two ballots
        // per bit; else the kw-th largest key itself, STEPS ballots per bit.
        uint32_t T = 0u;
        if (kw < n_w) {
            if (kw <= kLaneMaxKeep) {
                uint32_t l1 = 0u, l2 = 0u;                   // the lane's two largest keys
#pragma unroll
                for (int st = 0; st < STEPS; ++st) {
                    l2 = max(l2, min(l1, key[st]));
                    l1 = max(l1, key[st]);
                }
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = T | (1u << bit);
                    if (__popcll(__ballot(l1 >= c)) + __popcll(__ballot(l2 >= c)) >= kw) T = c;
                }
            } else {
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = T | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int st = 0; st < STEPS; ++st) cnt += __popcll(__ballot(ok[st] && key[st] >= c));
                    if (cnt >= kw) T = c;
                }
            }
        }
        // list every candidate with key >= T (at least kw of them)
        int my = 0;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) my += (ok[st] && key[st] >= T) ? 1 : 0;
        int tot = my;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(tot, off);
            if (lane >= off) tot += y;
        }
        const int excl = tot - my;
        const int wave_n = __shfl(tot, 63);
        int wbase = 0;
        if (lane == 0) {
            wbase = atomicAdd(&sm.n_emit[t], wave_n);
            if (T != 0u) atomicMax(&sm.max_t[t], T);
        }
        wbase = __shfl(wbase, 0);
        int k = wbase + excl;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (ok[st] && key[st] >= T) {
                if (k < kEmitPerRow)
                    sm.emit[t][k] = (static_cast<uint64_t>(key[st]) << 32) |
                                    static_cast<uint32_t>(~(j0 + 256 * st + lane));
                ++k;
            }
        }
    }
    // the scores of this wave's own blocks (j0 + 256 st .. + 63) in full
    // lines from LDS, issued before the workgroup meets: the wave reads back
    // only what it wrote
    {
        const int n = j_hi - j_lo;
        for (int t = 0; t < tq; ++t) {
            float* sb = scores + b * ss + t * sld + j_lo;
            for (int st = lane >> 4; st < STEPS; st += 4) {
                const int i = 64 * wave + 256 * st + 4 * (lane & 15);
                if (i < n) *reinterpret_cast<float4*>(sb + i) = *reinterpret_cast<const float4*>(lds_sc + t * R + i);
            }
        }
    }
    lds_barrier();
    if (tid < tq) {
        const int ne = sm.n_emit[tid];
        uint32_t* ctrl = ws.ctrl + (b * tq + tid) * kCtrl;
        sm.base[tid] = ne ? static_cast<int>(atomicAdd(&ctrl[kNList], static_cast<uint32_t>(min(ne, kEmitPerRow)))) : 0;
        if (sm.max_t[tid] != 0u) atomicMax(&ctrl[kMaxT], sm.max_t[tid]);
        if (ne > kEmitPerRow) atomicOr(&ctrl[kOverflow], 1u);
    }
    lds_barrier();
    for (int t = 0; t < tq; ++t) {
        const int nl = min(sm.n_emit[t], kEmitPerRow);
        const int base = sm.base[t];
        uint64_t* list = ws.list + static_cast<int64_t>(b * tq + t) * ws.cap;
        for (int k = tid; k < nl; k += 256)
            if (base + k < ws.cap) list[base + k] = sm.emit[t][k];
    }
}

constexpr int kFinNT = 1024;                 // finalize threads
constexpr int kRankMax = 1024;               // cut-bin members ranked directly
constexpr int kFinBins = 2048;               // radix bins over the listed keys' range
constexpr int kFinBits = 11;
constexpr int kBitmapWords = 8192;           // ascending order by bitmap for candidates j < 262144

struct FinalizeSmem {
    union {
        SelectSmem s;                                        // fallback: full radix select
        struct {
            alignas(16) int32_t chosen[QSA_MAX_BUDGET + 4];  // selection, any order
            alignas(16) uint64_t cand[kDecCap];              // cut-bin members
            uint32_t h[kFinBins];                            // radix level
            uint32_t bm[kBitmapWords];                       // one bit per candidate block
            int wave_tot[16];
            uint32_t wave_min[16], wave_max[16];
            uint32_t sh_bin, kstar;
            int sh_above, n_taken, n_cand;
        } m;
    } u;
};

// set bits of the wave mask m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

// entries x of cand[0 .. n) ranked by (key, ~j) descending: those with rank
// < take go to dst[rank] (and set their block's bit in bm, if given); the one
// of rank take - 1 (the cut) leaves its key in *kstar.  Every thread must call it.
template <int NT>
__device__ __forceinline__ void rank_cut(const uint64_t* cand, int n, int take, int32_t* dst, uint32_t* kstar,
                                         uint32_t* bm) {
    for (int i = threadIdx.x; i < n; i += NT) {
        const uint64_t x = cand[i];
        int rk = 0;
#pragma unroll 8
        for (int k = 0; k < n; ++k) rk += cand[k] > x ? 1 : 0;
        if (rk < take) {
            const int32_t v = static_cast<int32_t>(~static_cast<uint32_t>(x));
            dst[rk] = v;
            if (bm != nullptr) atomicOr(&bm[v >> 5], 1u << (v & 31));
        }
        if (rk == take - 1) *kstar = static_cast<uint32_t>(x >> 32);
    }
}

// kPer list entries per thread: ws.cap = kPer * kFinNT.
// The top `keep` of entries e by (key, ~j) -- thread tid holds entries
// tid + kFinNT i, i < P, the first n of all valid -- into sm.u.m.chosen (any
// order), leaving the keep-th largest key in sm.u.m.kstar: one radix level over
// the entries' own key range, keys above the cut bin taken, the bin's members
// ranked.  False (nothing decided) when the cut bin holds more than kDecCap.
// With set_bits (candidates below 32 kBitmapWords) each chosen block also sets
// its bit in sm.u.m.bm, which must be clear: the ascending emission then needs
// no pass of its own.  Every thread must call it.
template <int P>
__device__ __forceinline__ bool take_top(const uint64_t (&e)[P], int n, int keep, bool set_bits, FinalizeSmem& sm) {
    const int tid = threadIdx.x;
    uint32_t* h = sm.u.m.h;
    int32_t* chosen = sm.u.m.chosen;
    uint32_t* bm = set_bits ? sm.u.m.bm : nullptr;
    // one radix level over the entries' own key range [kmin, kmax]: bin =
    // (key - kmin) >> shift < 4096 (the entries all sit in the tail, so the
    // top key bits would crowd them into a few bins and serialize the LDS
    // atomics)
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (tid + kFinNT * i < n) {
            const uint32_t k = static_cast<uint32_t>(e[i] >> 32);
            kmin = min(kmin, k);
            kmax = max(kmax, k);
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), off)));
        kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), off)));
    }
    if ((tid & 63) == 0) {
        sm.u.m.wave_min[tid >> 6] = kmin;
        sm.u.m.wave_max[tid >> 6] = kmax;
    }
    for (int k = tid; k < kFinBins; k += kFinNT) h[k] = 0u;
    if (tid == 0) {
        sm.u.m.n_taken = 0;
        sm.u.m.n_cand = 0;
        sm.u.m.kstar = 0u;
    }
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kFinNT / 64; ++w) {
        kmin = min(kmin, sm.u.m.wave_min[w]);
        kmax = max(kmax, sm.u.m.wave_max[w]);
    }
    const uint32_t span = kmax - kmin;
    const int shift = span < kFinBins ? 0 : 32 - __clz(static_cast<int>(span >> kFinBits));
    auto bin_of = [&](uint64_t x) { return (static_cast<uint32_t>(x >> 32) - kmin) >> shift; };
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (tid + kFinNT * i < n) atomicAdd(&h[bin_of(e[i])], 1u);
    lds_barrier();
    find_threshold_bin<kFinNT>(h, kFinBins, keep, sm.u.m.wave_tot, &sm.u.m.sh_bin, &sm.u.m.sh_above);
    const uint32_t tbin = sm.u.m.sh_bin;
    const int above = sm.u.m.sh_above;
    const int inbin = static_cast<int>(h[tbin]);
    if (inbin > kDecCap) return false;                    // uniform
    {
        // keys above the cut bin are taken; the cut bin's members go to cand
        // (positions by ballot and lane count: one LDS atomic per wave and
        // pass, not one per entry on a single counter)
        uint64_t* lc = sm.u.m.cand;
        uint64_t m_up[P], m_in[P];
        int n_up = 0, n_in = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const bool ok = tid + kFinNT * i < n;
            const uint32_t d1 = bin_of(e[i]);
            m_up[i] = __ballot(ok && d1 > tbin);
            m_in[i] = __ballot(ok && d1 == tbin);
            n_up += __popcll(m_up[i]);
            n_in += __popcll(m_in[i]);
        }
        int b_up = 0, b_in = 0;
        if ((tid & 63) == 0) {
            b_up = n_up ? atomicAdd(&sm.u.m.n_taken, n_up) : 0;
            b_in = n_in ? atomicAdd(&sm.u.m.n_cand, n_in) : 0;
        }
        b_up = __shfl(b_up, 0);
        b_in = __shfl(b_in, 0);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int lane = tid & 63;
            if ((m_up[i] >> lane) & 1ull) {
                const int32_t v = static_cast<int32_t>(~static_cast<uint32_t>(e[i]));
                chosen[b_up + lanes_below(m_up[i])] = v;
                if (bm != nullptr) atomicOr(&bm[v >> 5], 1u << (v & 31));
            }
            if ((m_in[i] >> lane) & 1ull) lc[b_in + lanes_below(m_in[i])] = e[i];
            b_up += __popcll(m_up[i]);
            b_in += __popcll(m_in[i]);
        }
        lds_barrier();
        const int remaining = keep - above;
        if (inbin <= kRankMax) {
            rank_cut<kFinNT>(lc, inbin, remaining, chosen + above, &sm.u.m.kstar, bm);
        } else {
            // many members (tie floods): sorted, the first `remaining` taken
            const int np2 = next_pow2(inbin);
            for (int k = inbin + tid; k < np2; k += kFinNT) lc[k] = 0ull;
            lds_barrier();
            bitonic_sort<kFinNT, uint64_t, true>(lc, np2);
            for (int k = tid; k < remaining; k += kFinNT) {
                const int32_t v = static_cast<int32_t>(~static_cast<uint32_t>(lc[k]));
                chosen[above + k] = v;
                if (bm != nullptr) atomicOr(&bm[v >> 5], 1u << (v & 31));
            }
            if (tid == 0) sm.u.m.kstar = static_cast<uint32_t>(lc[remaining - 1] >> 32);
        }
        lds_barrier();
    }
    return true;
}

constexpr int kIncMax = 32;          // incomplete waves re-read before a whole-row pass is cheaper

// Appends the entries whose `in` is set to sm.u.m.cand: one LDS reservation
// per wave (a wave-uniform call).
__device__ __forceinline__ void append_cand(bool in, uint64_t entry, FinalizeSmem& sm) {
    const uint64_t m = __ballot(in);
    if (m == 0ull) return;
    int wb = 0;
    if ((threadIdx.x & 63) == 0) wb = atomicAdd(&sm.u.m.n_cand, __popcll(m));
    const int pos = __shfl(wb, 0) + lanes_below(m);
    if (in && pos < kDecCap) sm.u.m.cand[pos] = entry;
}

// A row whose list missed part of its selection (some scan wave held more of
// it than it listed: scores far from random order, such as a run of recent
// blocks that all score high).  The list's own cut kl (its keep-th largest
// key) is at most the row's, so the row's selection lies among its keys >= kl;
// these are collected into sm.u.m.cand and the same radix cut as the list
// path decides the row (false: it could not, nothing decided).
//
// First from the list and the waves: a wave listed every one of its keys
// >= its threshold T, and its smallest listed key m is >= T, so a wave with
// m <= kl listed all of its keys >= kl; only the waves with m > kl (a few,
// when high scores cluster) are re-read from the stored row, for their keys
// in [kl, m) -- none of them listed.  m comes from the list itself (the wave
// of an entry follows from its block).  With more than kIncMax such waves,
// one pass over the whole stored row instead.  More than kDecCap keys >= kl
// (tie floods): false.
__device__ __forceinline__ bool recover(int n, const float* __restrict__ row, int o, int keep, const DecodeWs& ws,
                                        int r, FinalizeSmem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const uint32_t kl = sm.u.m.kstar;
    const uint64_t* __restrict__ list = ws.list + static_cast<int64_t>(r) * ws.cap;
    const int n_waves = ws.wg * 4;
    const int R = 256 * ws.steps;
    uint32_t* wmin = sm.u.m.bm;                           // per wave: its smallest listed key (the bitmap is free here)
    int* inc = reinterpret_cast<int*>(sm.u.m.h);          // the waves to re-read (the histogram is free here)
    auto wave_of = [&](int j) { return (j / R) * 4 + ((j % R) >> 6) % 4; };
    lds_barrier();                                        // every thread has read kstar
    bool whole_row = n_waves > kBitmapWords;              // uniform
    if (!whole_row) {
        for (int w = tid; w < n_waves; w += kFinNT) wmin[w] = 0xffffffffu;
        if (tid == 0) {
            sm.u.m.n_cand = 0;
            sm.u.m.n_taken = 0;                           // count of waves to re-read
        }
        lds_barrier();
        for (int i = tid; i < n; i += kFinNT) {
            const uint64_t x = list[i];
            atomicMin(&wmin[wave_of(static_cast<int>(~static_cast<uint32_t>(x)))], static_cast<uint32_t>(x >> 32));
        }
        lds_barrier();
        for (int w = tid; w < n_waves; w += kFinNT)
            if (wmin[w] > kl && (w >> 2) * R + 64 * (w & 3) < o) {   // a wave with blocks below o
                const int k = atomicAdd(&sm.u.m.n_taken, 1);
                if (k < kIncMax) inc[k] = w;
            }
        lds_barrier();
        whole_row = sm.u.m.n_taken > kIncMax;             // uniform
    } else {
        if (tid == 0) sm.u.m.n_cand = 0;
        lds_barrier();
    }
    if (!whole_row) {
        for (int i0 = 0; i0 < n; i0 += kFinNT) {          // uniform
            const uint64_t x = i0 + tid < n ? list[i0 + tid] : 0ull;
            append_cand(i0 + tid < n && static_cast<uint32_t>(x >> 32) >= kl, x, sm);
        }
        const int n_inc = sm.u.m.n_taken;
        for (int k = 0; k < n_inc; ++k) {                 // uniform
            const int w = inc[k];
            const uint32_t T = wmin[w];
            const int j_w = (w >> 2) * R + 64 * (w & 3);  // the wave's blocks: j_w + 256 st + lane
            for (int q = tid; q < 64 * ws.steps; q += kFinNT) {
                const int j = j_w + 256 * (q >> 6) + (q & 63);
                const uint32_t key = j < o ? score_key(row[j]) : 0u;
                append_cand(j < o && key >= kl && key < T, (static_cast<uint64_t>(key) << 32) | ~static_cast<uint32_t>(j),
                            sm);
            }
        }
    } else {
        constexpr int kIn = 8;                            // float4 loads in flight per thread
        for (int j0 = 4 * tid; j0 < o; j0 += 4 * kFinNT * kIn) {
            float4 v[kIn];
#pragma unroll
            for (int u = 0; u < kIn; ++u) {
                const int j = j0 + 4 * kFinNT * u;      // rows are padded to a multiple of 4 floats
                v[u] = j < o ? *reinterpret_cast<const float4*>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            // this lane's keys >= kl among its 4 kIn values, then one LDS
            // reservation per wave: the lane's count (<= 32) by its 6 bits, each
            // a ballot, so the lane's offset is a sum of shifted lane counts
            auto val = [&](int u, int e) { return e == 0 ? v[u].x : e == 1 ? v[u].y : e == 2 ? v[u].z : v[u].w; };
            uint32_t pass = 0u;                           // bit 4u + e: value e of load u passes
#pragma unroll
            for (int u = 0; u < kIn; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + 4 * kFinNT * u + e < o && score_key(val(u, e)) >= kl) pass |= 1u << (4 * u + e);
            const int my = __popc(pass);
            int off = 0, tot = 0;
#pragma unroll
            for (int bit = 0; bit < 6; ++bit) {
                const uint64_t m = __ballot((my >> bit) & 1);
                off += lanes_below(m) << bit;
                tot += __popcll(m) << bit;
            }
            if (tot != 0) {                               // wave-uniform
                int wb = 0;
                if (lane == 0) wb = atomicAdd(&sm.u.m.n_cand, tot);
                int pos = __shfl(wb, 0) + off;
#pragma unroll
                for (int u = 0; u < kIn; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if ((pass >> (4 * u + e)) & 1u) {
                            const uint32_t j = static_cast<uint32_t>(j0 + 4 * kFinNT * u + e);
                            if (pos < kDecCap) sm.u.m.cand[pos] = (static_cast<uint64_t>(score_key(val(u, e))) << 32) | ~j;
                            ++pos;
                        }
            }
        }
    }
    lds_barrier();
    const int n2 = sm.u.m.n_cand;
    if (n2 > kDecCap) return false;                       // uniform
    constexpr int kP = kDecCap / kFinNT;
    uint64_t e2[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) e2[i] = tid + kFinNT * i < n2 ? sm.u.m.cand[tid + kFinNT * i] : 0ull;
    lds_barrier();                                        // cand and its count are reused below
    const bool bits = o <= 32 * kBitmapWords;
    if (bits)                                             // the first cut's bits, then wmin, were here
        for (int k = tid; k < kBitmapWords; k += kFinNT) sm.u.m.bm[k] = 0u;
    return take_top<kP>(e2, n2, keep, bits, sm);
}

template <int kPer>
__global__ __launch_bounds__(kFinNT) void decode_finalize_kernel(const float* __restrict__ scores, int64_t ss,
                                                                 int64_t sld, Positions pos, int budget, int tq,
                                                                 DecodeWs ws, int32_t* __restrict__ sel,
                                                                 int64_t sels, uint32_t* fallback_count) {
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
    if (trivial_selection(keep, o, budget, out, kFinNT)) return;   // nothing was listed

    // the list, every load in flight at once with the control words (fixed
    // capacity: entries past the count are read and dropped)
    const uint64_t* __restrict__ lg = ws.list + static_cast<int64_t>(r) * (kPer * kFinNT);
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) e[i] = lg[tid + kFinNT * i];
    const int n = static_cast<int>(ctrl[kNList]);
    const uint32_t max_t = ctrl[kMaxT];
    // the block bitmap of the ascending emission, cleared while the list is in
    // flight; the cut sets the chosen blocks' bits as it takes them
    const bool bits = o <= 32 * kBitmapWords;
    if (bits)
        for (int k = tid; k < kBitmapWords; k += kFinNT) sm.u.m.bm[k] = 0u;
    const bool listed = ctrl[kOverflow] == 0u && n <= kPer * kFinNT && n >= keep;
    int32_t* chosen = sm.u.m.chosen;
    bool exact = false;
    bool cut_known = false;                               // sm.u.m.kstar holds the list's own cut
    if (listed) {
        cut_known = take_top<kPer>(e, n, keep, bits, sm);
        // every key >= max T is listed: the cut is exact if the cut key reaches max T
        exact = cut_known && sm.u.m.kstar >= max_t;
    }
    if (!exact && fallback_count != nullptr && tid == 0) atomicAdd(fallback_count, 1u);
    if (__builtin_expect(!exact && cut_known, 0)) exact = recover(n, scores + b * ss + t * sld, o, keep, ws, r, sm);
    if (!exact) {
        select_row<kFinNT>(scores + b * ss + t * sld, o, keep, budget, out, sm.u.s);
    } else {
        if (bits) {
            // ascending through the bitmap of the chosen blocks (every chosen
            // j < o set its bit in the cut, behind a barrier since); thread t
            // owns words kWpt t .. kWpt t + kWpt - 1
            uint32_t* bm = sm.u.m.bm;
            if (tid == 0) out[keep] = o;                     // above every candidate
            constexpr int kWpt = kBitmapWords / kFinNT;
            uint32_t w[kWpt];
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < kWpt; ++q) {
                w[q] = bm[kWpt * tid + q];
                cnt += __popc(w[q]);
            }
            int total;
            int base = block_exclusive_scan<kFinNT, false>(cnt, sm.u.m.wave_tot, &total);   // wave_tot not used again
#pragma unroll
            for (int q = 0; q < kWpt; ++q) {
                uint32_t wq = w[q];
                while (wq) {
                    const int bit = __ffs(wq) - 1;
                    out[base++] = 32 * (kWpt * tid + q) + bit;
                    wq &= wq - 1;
                }
            }
        } else {
            if (tid == 0) chosen[keep] = o;              // above every candidate
            rank_write_ascending<kFinNT>(chosen, keep + 1, out);
        }
        for (int k = keep + 1 + tid; k < budget; k += kFinNT) out[k] = -1;
    }
    if (tid < kCtrl) ctrl[tid] = 0u;
}

// Scan granularity (256 * steps blocks per workgroup, 64 * steps per wave) and
// list capacity per row.  A row's list holds about wave_listed entries per
// wave, so longer waves give shorter lists but fewer workgroups.  Measured
// at 1M context, budget 512: one sequence scanned by 128 workgroups instead
// of 256 takes about 5 us longer, by 64 about 19 us; doubling the list
// capacity costs the finalize about 2.5 us; with 4 tokens per sequence,
// 256 workgroups instead of 512 cost about 11 us.  So the plan takes the
// longest steps that still give every CU a workgroup (two when tq > 1; the
// steps start at the largest of 8, 4, 2, 1 that gives about two), then,
// going down to the starting steps, the first whose expected list plus 4
// standard deviations fits a capacity the workspace holds (kListCap,
// 2 kListCap, 4 kListCap: the smallest that fits) with the thresholds taken
// from the lanes' two largest keys; if none, longer steps; then the exact
// threshold search.  The dynamic LDS (tq x 256 x steps floats) stays within
// 64 KiB.  A list that still overflows sends its row to the exact path.
static void scan_plan(int batch, int tq, int o, int keep, int* steps, int* cap) {
    const int64_t groups = static_cast<int64_t>(batch) * ((o + 255) / 256);
    const int s0 = groups >= 8 * 512 ? 8 : groups >= 4 * 512 ? 4 : groups >= 2 * 512 ? 2 : 1;
    const int s_max = tq <= 2 ? 32 : 16;
    if (keep <= 0 || keep >= o) {                         // trivial rows list nothing
        *steps = s0;
        *cap = kListCap;
        return;
    }
    const int avail = list_cap_avail(batch * tq);
    auto wgs = [&](int st) { return static_cast<int64_t>(batch) * ((o + 256 * st - 1) / (256 * st)); };
    // the longest steps that give every CU a workgroup (two with several
    // tokens per sequence: the per-row listing after the stream grows with tq,
    // and a second workgroup per CU overlaps it)
    const int64_t min_wgs = tq > 1 ? 512 : 256;
    int s_full = s0;
    while (2 * s_full <= s_max && wgs(2 * s_full) >= min_wgs) s_full *= 2;
    auto lane_max = [&](int st) { return wave_keep(keep, o, min(64 * st, o)) <= kLaneMaxKeep; };
    // the smallest capacity that holds the expected list (per-wave spread
    // about sqrt(listed - kw + 1)), or 0
    auto cap_for = [&](int st) {
        const int n_w = min(64 * st, o);
        const int kw = wave_keep(keep, o, n_w);
        const double per = wave_listed(kw, n_w);
        const double waves = (o + n_w - 1) / n_w;
        const double need = waves * per + 4.0 * sqrt(waves * (per - kw + 1.0));
        for (int c = kListCap; c <= avail; c *= 2)
            if (need <= c) return c;
        return 0;
    };
    auto take = [&](int st) {
        const int c = cap_for(st);
        if (c == 0) return false;
        *steps = st;
        *cap = c;
        return true;
    };
    for (int st = s_full; st >= s0; st /= 2)
        if (lane_max(st) && take(st)) return;
    for (int st = 2 * s_full; st <= s_max; st *= 2)
        if (lane_max(st) && take(st)) return;
    for (int st = s_full; st >= s0; st /= 2)
        if (take(st)) return;
    for (int st = 2 * s_full; st <= s_max; st *= 2)
        if (take(st)) return;
    *steps = s0;                                             // rows that overflow take the exact path
    *cap = avail;
}

hipError_t launch_decode_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                                      int64_t kbs, const Positions& pos, int batch, int tq, int budget,
                                      float* scores, int64_t ss, int64_t sld, int32_t* sel, int64_t sels,
                                      void* ws, const DecodeAppend* append, const DecodeQrot* qrot,
                                      const PageMap* pm, hipStream_t stream) {
    const int rows = batch * tq;
    int o_max = 0;
    for (int b = 0; b < batch; ++b) o_max = max(o_max, (pos.p[b] + tq - 1) / kBlock);
    int steps, cap;
    scan_plan(batch, tq, o_max, min(budget - 1, o_max), &steps, &cap);
    const int wg_scan = max(1, (o_max + 256 * steps - 1) / (256 * steps));

    const DecodeWs w = carve(ws, cap, steps, wg_scan);
    AppendArgs ap{};
    qsa_rope_t rope{1.0e7, 1.0, 0};
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
        rope = append->rope;
    }
    QrotArgs qr{};
    if (qrot != nullptr) {
        qr.q = qrot->q;
        qr.qs = qrot->qs;
        qr.q_rot = qrot->q_rot;
        rope = qrot->rope;
    }
    ap.inv = make_inv_freq(rope);
    hipError_t e;
    // one token per sequence: the rows are appended by the scan's side
    // workgroups; several: first, because a block an earlier new token
    // completes is scored for the later ones
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
    const int n_side = (scan_appends || qr.q != nullptr) ? batch : 0;
    const dim3 grid(static_cast<unsigned>(n_side + batch * wg_scan));
    const size_t lds = static_cast<size_t>(tq) * 256 * steps * 4;
    const ScanTiming timing = scan_timing();
    if (timing.begin != nullptr && (e = hipEventRecord(timing.begin, stream)) != hipSuccess) return e;
#define QSA_SCAN(S, P)                                                                                       \
    hipLaunchKernelGGL((decode_scan_kernel<S, P>), grid, dim3(256), lds, stream, q_idx, qs, kbar, kbs, pos, \
                       budget, tq, n_side, wg_scan, scores, ss, sld, w, ap, scan_appends, qr, pmv)
    if (pm != nullptr) {
        switch (steps) {
            case 32: QSA_SCAN(32, true); break;
            case 16: QSA_SCAN(16, true); break;
            case 8: QSA_SCAN(8, true); break;
            case 4: QSA_SCAN(4, true); break;
            case 2: QSA_SCAN(2, true); break;
            default: QSA_SCAN(1, true); break;
        }
    } else {
        switch (steps) {
            case 32: QSA_SCAN(32, false); break;
            case 16: QSA_SCAN(16, false); break;
            case 8: QSA_SCAN(8, false); break;
            case 4: QSA_SCAN(4, false); break;
            case 2: QSA_SCAN(2, false); break;
            default: QSA_SCAN(1, false); break;
        }
    }
#undef QSA_SCAN
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (timing.end != nullptr && (e = hipEventRecord(timing.end, stream)) != hipSuccess) return e;
#define QSA_FIN(P)                                                                                            \
    hipLaunchKernelGGL(decode_finalize_kernel<P>, dim3(static_cast<unsigned>(rows)), dim3(kFinNT), 0, stream, \
                       scores, ss, sld, pos, budget, tq, w, sel, sels, decode_fallback_counter())
    switch (cap) {
        case 4 * kListCap: QSA_FIN(4 * kListCap / kFinNT); break;
        case 2 * kListCap: QSA_FIN(2 * kListCap / kFinNT); break;
        default: QSA_FIN(kListCap / kFinNT); break;
    }
#undef QSA_FIN
    return hipGetLastError();
}

}  // namespace qsa
