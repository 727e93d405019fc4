// Internal declarations shared by the libqsa kernels and the C-ABI shim.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 matrix-core (MFMA) tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kBlock = 4;     // tokens per micro-block
constexpr int kHq = 24;       // attention query heads
constexpr int kHkv = 2;       // attention KV heads
constexpr int kGroup = kHq / kHkv;
constexpr int kD = 256;       // attention head dim
constexpr int kRot = 64;      // rotary slice
constexpr int kHi = 4;        // indexer query heads
constexpr int kDi = 128;      // indexer head dim

// host positions travel by value inside the kernel arguments
struct Positions {
    int32_t p[QSA_MAX_BATCH];
};

// Paged caches (block table): token n of sequence b sits in page
// table[b * ts + (n >> shift)], row n & (P - 1) of it, P = 1 << shift tokens per
// page (a multiple of 64, so a page holds whole micro-blocks and whole
// 16-block tiles of block keys: block j sits in the page of token 4j, row
// j & (P/4 - 1)).  Page ids read from the table are clamped to
// [0, n_pages), so every access stays inside the pools whatever the table
// holds.
struct PageMap {
    const int32_t* table;
    int64_t ts;
    int shift;
    int n_pages;
};

__device__ __forceinline__ int page_of(const PageMap& pm, int b, int64_t n) {
    const int pg = pm.table[b * pm.ts + (n >> pm.shift)];
    return min(max(pg, 0), pm.n_pages - 1);
}

// physical token row of token n, and physical block-key row of block j
__device__ __forceinline__ int64_t phys_token(const PageMap& pm, int b, int64_t n) {
    return (static_cast<int64_t>(page_of(pm, b, n)) << pm.shift) | (n & ((int64_t{1} << pm.shift) - 1));
}
__device__ __forceinline__ int64_t phys_block(const PageMap& pm, int b, int64_t j) {
    return (static_cast<int64_t>(page_of(pm, b, j * 4)) << (pm.shift - 2)) |
           (j & ((int64_t{1} << (pm.shift - 2)) - 1));
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16, round to nearest, ties to even (NaN -> quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// float64 -> bf16 in ONE rounding step (nearest, ties to even): round the
// 52-bit mantissa to 7 bits on the integer pattern (add half of the 45
// dropped bits' range minus one, plus the kept lsb, then truncate), so the
// result is an exact float32 whose upper half is the bf16 pattern.  Finite
// inputs in bf16's normal range (or zero) are assumed.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    u += 0x0fffffffffffull + ((u >> 45) & 1ull);
    u &= ~0x1fffffffffffull;
    float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
    return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// Workgroup barrier for data exchanged through LDS only: waits for this wave's
// LDS operations (not its global loads and stores, which stay in flight), then
// meets the other waves.  __syncthreads() carries a workgroup release fence,
// which also waits for every global load and store in flight; this does not.
// The empty asm statements keep the compiler from moving memory accesses
// across it.  Not for data one thread of the workgroup passes to another
// through global memory.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0); vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Monotone map of float32 onto uint32 for selection: larger score -> larger
// key; -0.0 and +0.0 share a key; every NaN maps to 0, below all numbers.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) == 0) return 0x80000000u;
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace qsa

// ---- launchers (one per kernel file); arguments are already validated ----
namespace qsa {

hipError_t launch_rope(const uint16_t* x, int64_t xs, int64_t xt, uint16_t* y, int64_t ys,
                       int64_t yt, int batch, int n_tokens, int n_heads, const Positions& pos0,
                       const qsa_rope_t& rope, bool in_place, hipStream_t stream);

hipError_t launch_compress(const uint16_t* k_idx, int64_t ks, int batch, int block_begin,
                           int block_end, uint16_t* kbar, int64_t kbs, hipStream_t stream);

// row_flags (may be null): only the 64-row tiles holding a row with a nonzero flag are
// scored, and nothing while *n_flagged (if given) is zero.  pm (may be null):
// kbar is a page pool addressed through the block table (here and below).
hipError_t launch_index_scores(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                               int64_t kbs, const Positions& pos0, int batch, int tq,
                               float* scores, int64_t ld, int64_t ss, const int* row_flags,
                               const int* n_flagged, const PageMap* pm, hipStream_t stream);

// row_flags (may be null): only rows with a nonzero flag are selected; their flags are cleared
hipError_t launch_select(const float* scores, int64_t ld, int64_t ss, const Positions& pos0,
                         int batch, int tq, int budget, int32_t* sel, int64_t sels, int* row_flags,
                         hipStream_t stream);

// ---- fused prefill index-select (threshold from a sample, candidate lists) ----
constexpr int kSampleRuns = 256;                  // sample runs per sequence
constexpr int kSampleRunLen = 16;                 // blocks per run: one 16-block tile
constexpr int kSampleCols = kSampleRuns * kSampleRunLen;    // sampled scores per row
constexpr int kCollectCap = 2048;                 // candidates listed in LDS per workgroup
constexpr int kRowCap = 4096;                     // candidates kept per row

struct IndexCollect {
    const float* tau;           // [rows] threshold per row
    int* row_cnt;               // [rows] candidates appended (zero before the launch)
    uint64_t* list;             // [rows][kRowCap] key << 32 | ~j
    const int* n_flagged;       // scores mode with row flags: nothing to do while *n_flagged == 0
    uint8_t* wg_flag;           // collect: per workgroup, its LDS lists overflowed (the retry pass redoes it)
};

hipError_t launch_index_sample(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                               const Positions& pos0, int batch, int tq, float* sample, const PageMap* pm,
                               hipStream_t stream);
hipError_t launch_index_collect(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                                const Positions& pos0, int batch, int tq, int max_cols, const IndexCollect& col,
                                const PageMap* pm, hipStream_t stream);

size_t prefill_select_ws_bytes(int batch, int tq);
// whole index-select of a prefill chunk; scores [B][tq][ld] is used only by rows
// that need the exact fallback (or by every row when the fused path does not apply)
hipError_t launch_prefill_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar, int64_t kbs,
                                       const Positions& pos0, int batch, int tq, int budget, float* scores,
                                       int64_t ld, int64_t ss, int32_t* sel, int64_t sels, void* ws,
                                       const PageMap* pm, hipStream_t stream);

hipError_t launch_attn_prefill(const uint16_t* q, int64_t qs, const uint16_t* k,
                               const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                               const Positions& pos0, int batch, int tq, int budget, float scale,
                               uint16_t* out, int64_t os, float* lse, int64_t lss, const uint16_t* gate,
                               int64_t gs, const PageMap* pm, hipStream_t stream);

// Decode rows: tq (1 .. kMaxDecodeTq) consecutive query tokens per sequence,
// token t of sequence b at position pos[b] + t; row r = b * tq + t.  Per
// sequence, q / out are [tq][24][256], q_idx [tq][4][128], sel [tq][budget],
// scores [tq][sld]; lse is [B * tq][24].
constexpr int kMaxDecodeTq = QSA_MAX_DECODE_TQ;

size_t decode_workspace_bytes(int rows, int budget);
// decode attention with optional rotation of q on load (rope non-null);
// gate (nullable, laid out as out with sequence stride gs): the output gate;
// pm (nullable): k / v are page pools addressed through the block table
hipError_t launch_attn_decode_ex(const uint16_t* q, int64_t qs, const uint16_t* k,
                                 const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                                 const Positions& pos, int batch, int tq, int budget, float scale,
                                 uint16_t* out, int64_t os, float* lse, const uint16_t* gate, int64_t gs,
                                 void* ws, const qsa_rope_t* rope, const PageMap* pm, hipStream_t stream);

// fused decode index-select (scores + selection of the decode rows); the
// workspace starts with control words laid out for the largest row count,
// which must be zero before the first use and are left zero by each call
// (so one workspace serves calls of any shape)
size_t decode_select_ws_bytes(int rows);
// Events the decode index-select records around its scan launch (both null:
// none); per host thread, set through qsa_set_scan_timing_events.
struct ScanTiming {
    hipEvent_t begin, end;
};
ScanTiming& scan_timing();
// Device counter of decode rows that take the exact path (null: not counted);
// per host thread, set through qsa_set_decode_fallback_counter.
uint32_t*& decode_fallback_counter();
// Rows a decode step appends at each sequence's new positions p0 .. p0+tq-1
// before it scores (every pointer may be null: then that part is not done).
struct DecodeAppend {
    const uint16_t* k_new;       // [B][tq][2][256] unrotated: rotated into k_cache[b][p0 + t]
    int64_t kns;
    uint16_t* k_cache;
    const uint16_t* v_new;       // [B][tq][2][256]: copied into v_cache[b][p0 + t]
    int64_t vns;
    uint16_t* v_cache;
    int64_t kvs;                 // sequence stride of both KV caches
    const uint16_t* k_idx_new;   // [B][tq][128]: copied into k_idx[b][p0 + t]
    int64_t kins;
    uint16_t* k_idx;             // indexer key cache; with it, a block that a new token
    int64_t kis;                 // completes (p % 4 == 3) is compressed into kbar[b][p / 4]
    uint16_t* kbar;
    int64_t kbs;
    qsa_rope_t rope;             // rotary parameters of the K rows
};

// Queries of a decode step rotated once for its attention, by side
// workgroups of the scan: q [B][tq][24][256] (sequence stride qs) rotated
// into q_rot [B * tq][24][256] with `rope`, as qsa_rope_apply would.
struct DecodeQrot {
    const uint16_t* q;
    int64_t qs;
    uint16_t* q_rot;
    qsa_rope_t rope;
};

hipError_t launch_decode_index_select(const uint16_t* q_idx, int64_t qs, const uint16_t* kbar,
                                      int64_t kbs, const Positions& pos, int batch, int tq, int budget,
                                      float* scores, int64_t ss, int64_t sld, int32_t* sel, int64_t sels,
                                      void* ws, const DecodeAppend* append, const DecodeQrot* qrot,
                                      const PageMap* pm, hipStream_t stream);
// Paged caches: the new tokens [pos0[b], pos0[b] + n_tokens) of every sequence
// are written into their pages (K rotated, V, indexer keys; null inputs are
// skipped), then the key of every block they complete (when kbar is given).
hipError_t launch_paged_append(const PageMap& pm, uint16_t* k, uint16_t* v, uint16_t* k_idx, uint16_t* kbar,
                               const uint16_t* k_new, const uint16_t* v_new, int64_t kvns,
                               const uint16_t* k_idx_new, int64_t kins, const Positions& pos0, int batch,
                               int n_tokens, const qsa_rope_t& rope, hipStream_t stream);

// Gated DeltaNet token mixer: inputs and outputs of one call (T tokens per
// sequence; decode: T = 1).
struct GdnIn {
    const uint16_t* q;   // [B][T][16][128]
    const uint16_t* k;
    int64_t qks;         // sequence stride of q and k
    const uint16_t* v;   // [B][T][48][128]
    int64_t vs;
    const float* g;      // [B][T][48]
    const float* beta;
    int64_t gs;
    float* state;        // [B][48][128][128], updated in place
    uint16_t* out;       // [B][T][48][128]
    int64_t os;
};
size_t gdn_prefill_ws_bytes(int batch, int n_tokens);
hipError_t launch_gdn_prefill(const GdnIn& in, int batch, int n_tokens, void* ws, hipStream_t stream);
hipError_t launch_gdn_decode(const GdnIn& in, int batch, hipStream_t stream);

hipError_t launch_attn_decode(const uint16_t* q, int64_t qs, const uint16_t* k,
                              const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                              const Positions& pos, int batch, int tq, int budget, float scale,
                              uint16_t* out, int64_t os, float* lse, const uint16_t* gate, int64_t gs,
                              void* ws, hipStream_t stream);

}  // namespace qsa
