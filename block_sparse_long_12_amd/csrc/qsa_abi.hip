// C ABI of libqsa: argument validation, then one launch sequence per call on
// the caller's stream.  Validation touches no device memory and makes no HIP
// call, so every rejected call returns before anything is launched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "qsa_internal.h"

// Scratch of qsa_decode_step_noalloc: one copy per GPU the library runs on,
// held until the process ends.  Host code never uses this name as an address
// (on the host it only stands for the symbol); it takes each device's address
// from hipGetSymbolAddress, once, with that device current.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];


namespace {

thread_local char g_err[512] = "";
thread_local qsa::ScanTiming g_scan_timing{nullptr, nullptr};
thread_local uint32_t* g_fallback_counter = nullptr;

qsa_status_t fail(qsa_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

qsa_status_t ok() {
    g_err[0] = '\0';
    return QSA_OK;
}

qsa_status_t hip_result(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(QSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s) { return s > 0 && (s % 8) == 0; }

#define CHECK(cond, ...)                                            \
    do {                                                            \
        if (!(cond)) return fail(QSA_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
    } while (0)

// Copies host positions into the by-value kernel argument; every position
// plus `span` must stay representable and non-negative.
qsa_status_t take_positions(const int32_t* pos, int32_t batch, int32_t span, const char* name,
                            qsa::Positions& out) {
    CHECK(pos != nullptr, "%s is NULL", name);
    for (int b = 0; b < batch; ++b) {
        CHECK(pos[b] >= 0, "%s[%d] = %d is negative", name, b, pos[b]);
        CHECK(static_cast<int64_t>(pos[b]) + span < (int64_t{1} << 30), "%s[%d] = %d too large", name,
              b, pos[b]);
        out.p[b] = pos[b];
    }
    for (int b = batch; b < QSA_MAX_BATCH; ++b) out.p[b] = 0;
    return QSA_OK;
}

qsa_status_t check_batch(int32_t batch) {
    CHECK(batch >= 1 && batch <= QSA_MAX_BATCH, "batch = %d outside [1, %d]", batch, QSA_MAX_BATCH);
    return QSA_OK;
}

// Rotary parameters: NULL means the model card's plain rotary (theta 1e7).
qsa_status_t take_rope(const qsa_rope_t* rope, qsa_rope_t& out) {
    out = rope != nullptr ? *rope : qsa_rope_t{1.0e7, 1.0, 0};
    CHECK(isfinite(out.theta) && out.theta > 1.0, "rope theta must be finite and > 1");
    CHECK(isfinite(out.yarn_factor) && out.yarn_factor >= 1.0, "yarn_factor must be finite and >= 1");
    CHECK(out.yarn_factor == 1.0 || out.yarn_original_max >= 1, "yarn_original_max must be >= 1 with YaRN");
    return QSA_OK;
}

// Paged cache: geometry and table checks; the pools a call uses are checked
// by the caller (need_*).  Every sequence's table row must reach the page of
// its last token pos[b] + span - 1.
qsa_status_t take_paged(const qsa_paged_cache_t* c, const qsa::Positions& p, int32_t batch, int32_t span,
                        bool need_kv, bool need_k_idx, bool need_kbar, qsa::PageMap& pm) {
    CHECK(c != nullptr, "cache is NULL");
    CHECK(c->block_table != nullptr && (reinterpret_cast<uintptr_t>(c->block_table) & 3u) == 0,
          "block_table must be non-NULL and 4-byte aligned");
    const int32_t P = c->page_tokens;
    CHECK(P >= 64 && P <= 65536 && (P & (P - 1)) == 0, "page_tokens = %d must be a power of two in [64, 65536]", P);
    CHECK(c->n_pages >= 1, "n_pages = %d must be >= 1", c->n_pages);
    CHECK(int64_t{c->n_pages} * P <= INT32_MAX, "n_pages * page_tokens must stay below 2^31 rows");
    CHECK(!need_kv || (c->k != nullptr && c->v != nullptr && aligned16(c->k) && aligned16(c->v)),
          "cache k and v must be non-NULL and 16-byte aligned");
    CHECK(!need_k_idx || (c->k_idx != nullptr && aligned16(c->k_idx)),
          "cache k_idx must be non-NULL and 16-byte aligned");
    CHECK(!need_kbar || (c->kbar != nullptr && aligned16(c->kbar)), "cache kbar must be non-NULL and 16-byte aligned");
    int64_t pages = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t n = (int64_t{p.p[b]} + span + P - 1) / P;
        pages = n > pages ? n : pages;
    }
    CHECK(batch == 1 || c->table_stride >= pages, "table_stride = %lld smaller than the %lld pages a row reaches",
          static_cast<long long>(c->table_stride), static_cast<long long>(pages));
    pm.table = c->block_table;
    pm.ts = c->table_stride;
    pm.shift = __builtin_ctz(static_cast<unsigned>(P));
    pm.n_pages = c->n_pages;
    return QSA_OK;
}

#define TRY(expr)                          \
    do {                                   \
        qsa_status_t _s = (expr);          \
        if (_s != QSA_OK) return _s;       \
    } while (0)

// ---- per-device state of the static scratch

constexpr int kMaxDevices = 64;

struct ScratchSlot {
    void* ptr = nullptr;     // device address of `scratch` on this device
    bool clean = false;      // zero-filled, and every call since has left its control words zeroed
};

std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
    for (size_t i = blockIdx.x * size_t{256} + threadIdx.x; i < n16; i += size_t{gridDim.x} * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch; on its first use there (or after a call that
// failed part-way) the whole array is zero-filled on `stream` by a kernel
// (no memset node, so the call may sit in a captured graph).
qsa_status_t scratch_for_current_device(hipStream_t stream, ScratchSlot** slot_out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_result(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ERR_UNSUPPORTED, "device %d beyond the %d the static scratch serves", dev, kMaxDevices);
    ScratchSlot& s = g_scratch[dev];
    if (s.ptr == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) return hip_result(e, "hipGetSymbolAddress(scratch)");
        s.ptr = ptr;
    }
    if (!s.clean) {
        hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(s.ptr),
                           size_t{QSA_NOALLOC_SCRATCH_BYTES} / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_result(e, "scratch zero-fill launch");
        s.clean = true;
    }
    *slot_out = &s;
    return QSA_OK;
}

}  // namespace

namespace qsa {
ScanTiming& scan_timing() { return g_scan_timing; }
uint32_t*& decode_fallback_counter() { return g_fallback_counter; }
}  // namespace qsa

extern "C" {

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

qsa_status_t qsa_get_dims(qsa_dims_t* out) {
    CHECK(out != nullptr, "out is NULL");
    *out = qsa_dims_t{qsa::kBlock, qsa::kHq, qsa::kHkv, qsa::kD, qsa::kRot, qsa::kHi, qsa::kDi};
    return ok();
}

const char* qsa_status_string(qsa_status_t s) {
    switch (s) {
        case QSA_OK: return "ok";
        case QSA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case QSA_ERR_UNSUPPORTED: return "unsupported";
        case QSA_ERR_WORKSPACE: return "workspace too small";
        case QSA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* qsa_last_error(void) { return g_err; }

qsa_status_t qsa_set_scan_timing_events(void* begin_event, void* end_event) {
    g_scan_timing = qsa::ScanTiming{static_cast<hipEvent_t>(begin_event), static_cast<hipEvent_t>(end_event)};
    return QSA_OK;
}

qsa_status_t qsa_set_decode_fallback_counter(uint32_t* counter) {
    g_fallback_counter = counter;
    return QSA_OK;
}

qsa_status_t qsa_rope_apply(const uint16_t* x, int64_t x_seq_stride, int64_t x_tok_stride,
                            uint16_t* y, int64_t y_seq_stride, int64_t y_tok_stride,
                            int32_t batch, int32_t n_tokens, int32_t n_heads,
                            const int32_t* pos0, const qsa_rope_t* rope, hipStream_t stream) {
    TRY(check_batch(batch));
    CHECK(x != nullptr && y != nullptr, "x or y is NULL");
    CHECK(aligned16(x) && aligned16(y), "x and y must be 16-byte aligned");
    CHECK(n_tokens >= 0, "n_tokens = %d is negative", n_tokens);
    CHECK(n_heads >= 1 && n_heads <= 64, "n_heads = %d outside [1, 64]", n_heads);
    CHECK(stride_ok(x_tok_stride) && stride_ok(y_tok_stride), "token strides must be positive multiples of 8");
    CHECK(x_tok_stride >= int64_t{n_heads} * qsa::kD && y_tok_stride >= int64_t{n_heads} * qsa::kD,
          "token stride smaller than n_heads * 256");
    CHECK(batch == 1 || (stride_ok(x_seq_stride) && stride_ok(y_seq_stride)),
          "sequence strides must be positive multiples of 8");
    qsa_rope_t rp;
    TRY(take_rope(rope, rp));
    qsa::Positions p;
    TRY(take_positions(pos0, batch, n_tokens, "pos0", p));
    const bool in_place = (x == y);
    CHECK(!in_place || (x_seq_stride == y_seq_stride && x_tok_stride == y_tok_stride),
          "in-place rotation needs identical strides");
    if (n_tokens == 0) return ok();
    return hip_result(qsa::launch_rope(x, x_seq_stride, x_tok_stride, y, y_seq_stride, y_tok_stride,
                                       batch, n_tokens, n_heads, p, rp, in_place, stream),
                      "rope_apply launch");
}

qsa_status_t qsa_compress_block_keys(const uint16_t* k_idx, int64_t k_idx_seq_stride,
                                     int32_t batch, int32_t block_begin, int32_t block_end,
                                     uint16_t* kbar, int64_t kbar_seq_stride, hipStream_t stream) {
    TRY(check_batch(batch));
    CHECK(k_idx != nullptr && kbar != nullptr, "k_idx or kbar is NULL");
    CHECK(aligned16(k_idx) && aligned16(kbar), "k_idx and kbar must be 16-byte aligned");
    CHECK(block_begin >= 0 && block_end >= block_begin, "bad block range [%d, %d)", block_begin, block_end);
    CHECK(block_end < (1 << 28), "block_end = %d too large", block_end);
    CHECK(batch == 1 || (stride_ok(k_idx_seq_stride) && stride_ok(kbar_seq_stride)),
          "sequence strides must be positive multiples of 8");
    CHECK(batch == 1 || k_idx_seq_stride >= int64_t{block_end} * qsa::kBlock * qsa::kDi,
          "k_idx_seq_stride too small for block_end");
    CHECK(batch == 1 || kbar_seq_stride >= int64_t{block_end} * qsa::kDi, "kbar_seq_stride too small for block_end");
    if (block_end == block_begin) return ok();
    return hip_result(qsa::launch_compress(k_idx, k_idx_seq_stride, batch, block_begin, block_end,
                                           kbar, kbar_seq_stride, stream),
                      "compress_block_keys launch");
}

static qsa_status_t check_scores_layout(const void* scores, int64_t ld, int64_t ss, int32_t batch,
                                        int32_t tq, const qsa::Positions& p) {
    CHECK(scores != nullptr, "scores is NULL");
    CHECK(aligned16(scores), "scores must be 16-byte aligned");
    CHECK(ld > 0 && ld % 4 == 0, "scores_ld = %lld must be a positive multiple of 4", (long long)ld);
    int64_t need = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t o_last = (static_cast<int64_t>(p.p[b]) + tq - 1) / qsa::kBlock;
        if (o_last > need) need = o_last;
    }
    CHECK(ld >= need, "scores_ld = %lld < %lld blocks seen by the last row", (long long)ld, (long long)need);
    CHECK(batch == 1 || (ss % 4 == 0 && ss >= ld * tq), "scores_seq_stride must be a multiple of 4 and >= tq * ld");
    return QSA_OK;
}

qsa_status_t qsa_index_scores(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                              const uint16_t* kbar, int64_t kbar_seq_stride,
                              const int32_t* q_pos0, int32_t batch, int32_t tq,
                              float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                              hipStream_t stream) {
    TRY(check_batch(batch));
    CHECK(q_idx != nullptr && kbar != nullptr, "q_idx or kbar is NULL");
    CHECK(aligned16(q_idx) && aligned16(kbar), "q_idx and kbar must be 16-byte aligned");
    CHECK(tq >= 0, "tq = %d is negative", tq);
    qsa::Positions p;
    TRY(take_positions(q_pos0, batch, tq, "q_pos0", p));
    if (tq == 0) return ok();
    CHECK(batch == 1 || (stride_ok(q_idx_seq_stride) && q_idx_seq_stride >= int64_t{tq} * qsa::kHi * qsa::kDi),
          "q_idx_seq_stride must be a multiple of 8 and >= tq * 4 * 128");
    CHECK(batch == 1 || stride_ok(kbar_seq_stride), "kbar_seq_stride must be a positive multiple of 8");
    TRY(check_scores_layout(scores, scores_ld, scores_seq_stride, batch, tq, p));
    return hip_result(qsa::launch_index_scores(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch,
                                               tq, scores, scores_ld, scores_seq_stride, nullptr, nullptr, nullptr,
                                               stream),
                      "index_scores launch");
}

size_t qsa_select_workspace_bytes(int32_t batch, int32_t tq, int32_t budget) {
    (void)batch;
    (void)tq;
    (void)budget;
    return 0;
}

qsa_status_t qsa_select_topk(const float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                             const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                             int32_t* sel, int64_t sel_seq_stride,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    (void)workspace;
    (void)workspace_bytes;
    TRY(check_batch(batch));
    CHECK(tq >= 0, "tq = %d is negative", tq);
    CHECK(budget >= 1 && budget <= QSA_MAX_BUDGET, "budget = %d outside [1, %d]", budget, QSA_MAX_BUDGET);
    CHECK(sel != nullptr, "sel is NULL");
    CHECK((reinterpret_cast<uintptr_t>(sel) & 3u) == 0, "sel must be 4-byte aligned");
    qsa::Positions p;
    TRY(take_positions(q_pos0, batch, tq, "q_pos0", p));
    if (tq == 0) return ok();
    TRY(check_scores_layout(scores, scores_ld, scores_seq_stride, batch, tq, p));
    CHECK(batch == 1 || sel_seq_stride >= int64_t{tq} * budget, "sel_seq_stride < tq * budget");
    return hip_result(qsa::launch_select(scores, scores_ld, scores_seq_stride, p, batch, tq, budget, sel,
                                         sel_seq_stride, nullptr, stream),
                      "select_topk launch");
}

size_t qsa_index_select_prefill_workspace_bytes(int32_t batch, int32_t tq) {
    if (batch < 1 || batch > QSA_MAX_BATCH || tq < 0) return 0;
    return qsa::prefill_select_ws_bytes(batch, tq);
}

// kbar is contiguous [B][*][128] with kbar_seq_stride, or (cache non-NULL)
// the paged block-key pool of `cache`
static qsa_status_t index_select_prefill_impl(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                              const uint16_t* kbar, int64_t kbar_seq_stride,
                                              const qsa_paged_cache_t* cache,
                                              const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                                              float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                              int32_t* sel, int64_t sel_seq_stride,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    TRY(check_batch(batch));
    if (cache != nullptr) kbar = cache->kbar;
    CHECK(q_idx != nullptr && kbar != nullptr, "q_idx or kbar is NULL");
    CHECK(aligned16(q_idx) && aligned16(kbar), "q_idx and kbar must be 16-byte aligned");
    CHECK(tq >= 0, "tq = %d is negative", tq);
    CHECK(budget >= 1 && budget <= QSA_MAX_BUDGET, "budget = %d outside [1, %d]", budget, QSA_MAX_BUDGET);
    CHECK(sel != nullptr, "sel is NULL");
    CHECK((reinterpret_cast<uintptr_t>(sel) & 3u) == 0, "sel must be 4-byte aligned");
    qsa::Positions p;
    TRY(take_positions(q_pos0, batch, tq, "q_pos0", p));
    if (tq == 0) return ok();
    CHECK(batch == 1 || (stride_ok(q_idx_seq_stride) && q_idx_seq_stride >= int64_t{tq} * qsa::kHi * qsa::kDi),
          "q_idx_seq_stride must be a multiple of 8 and >= tq * 4 * 128");
    qsa::PageMap pm{};
    if (cache != nullptr)
        TRY(take_paged(cache, p, batch, tq, false, false, true, pm));
    else
        CHECK(batch == 1 || stride_ok(kbar_seq_stride), "kbar_seq_stride must be a positive multiple of 8");
    TRY(check_scores_layout(scores, scores_ld, scores_seq_stride, batch, tq, p));
    CHECK(batch == 1 || sel_seq_stride >= int64_t{tq} * budget, "sel_seq_stride < tq * budget");
    const size_t need = qsa::prefill_select_ws_bytes(batch, tq);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "index-select workspace needs %zu bytes, got %zu", need,
                    workspace == nullptr ? size_t{0} : workspace_bytes);
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "workspace must be 256-byte aligned");
    return hip_result(qsa::launch_prefill_index_select(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch, tq,
                                                       budget, scores, scores_ld, scores_seq_stride, sel,
                                                       sel_seq_stride, workspace, cache != nullptr ? &pm : nullptr,
                                                       stream),
                      "index_select_prefill launch");
}

qsa_status_t qsa_index_select_prefill(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                      const uint16_t* kbar, int64_t kbar_seq_stride,
                                      const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                                      float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                      int32_t* sel, int64_t sel_seq_stride,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return index_select_prefill_impl(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, nullptr, q_pos0, batch, tq,
                                     budget, scores, scores_ld, scores_seq_stride, sel, sel_seq_stride, workspace,
                                     workspace_bytes, stream);
}

qsa_status_t qsa_index_select_prefill_paged(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                            const qsa_paged_cache_t* cache,
                                            const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                                            float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                            int32_t* sel, int64_t sel_seq_stride,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    CHECK(cache != nullptr, "cache is NULL");
    return index_select_prefill_impl(q_idx, q_idx_seq_stride, nullptr, 0, cache, q_pos0, batch, tq, budget, scores,
                                     scores_ld, scores_seq_stride, sel, sel_seq_stride, workspace, workspace_bytes,
                                     stream);
}

static qsa_status_t check_attn_common(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const int32_t* sel, const uint16_t* out, int32_t budget,
                                      float scale) {
    CHECK(q != nullptr && k != nullptr && v != nullptr && sel != nullptr && out != nullptr,
          "q, k_cache, v_cache, sel and out must be non-NULL");
    CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out),
          "q, k_cache, v_cache and out must be 16-byte aligned");
    CHECK((reinterpret_cast<uintptr_t>(sel) & 3u) == 0, "sel must be 4-byte aligned");
    CHECK(budget >= 1 && budget <= QSA_MAX_BUDGET, "budget = %d outside [1, %d]", budget, QSA_MAX_BUDGET);
    CHECK(isfinite(scale) && scale > 0.f, "softmax_scale must be finite and > 0");
    return QSA_OK;
}

// k_cache / v_cache contiguous with kv_seq_stride, or (cache non-NULL) the
// paged pools of `cache`
static qsa_status_t sparse_attn_prefill_impl(const uint16_t* q, int64_t q_seq_stride,
                                             const uint16_t* k_cache, const uint16_t* v_cache,
                                             int64_t kv_seq_stride, const qsa_paged_cache_t* cache,
                                             const int32_t* sel, int64_t sel_seq_stride,
                                             const int32_t* q_pos0, int32_t batch, int32_t tq,
                                             int32_t budget, float softmax_scale,
                                             uint16_t* out, int64_t out_seq_stride, float* lse,
                                             int64_t lse_seq_stride, const uint16_t* gate, int64_t gate_seq_stride,
                                             hipStream_t stream) {
    TRY(check_batch(batch));
    if (cache != nullptr) {
        k_cache = cache->k;
        v_cache = cache->v;
    }
    TRY(check_attn_common(q, k_cache, v_cache, sel, out, budget, softmax_scale));
    CHECK(tq >= 0, "tq = %d is negative", tq);
    CHECK(lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u) == 0, "lse must be 4-byte aligned");
    CHECK(gate == nullptr || aligned16(gate), "gate must be 16-byte aligned");
    qsa::Positions p;
    TRY(take_positions(q_pos0, batch, tq, "q_pos0", p));
    if (tq == 0) return ok();
    qsa::PageMap pm{};
    if (cache != nullptr) TRY(take_paged(cache, p, batch, tq, true, false, false, pm));
    if (batch > 1) {
        int64_t max_len = 0;
        for (int b = 0; b < batch; ++b) max_len = p.p[b] + tq > max_len ? p.p[b] + tq : max_len;
        CHECK(stride_ok(q_seq_stride) && q_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD, "q_seq_stride too small");
        CHECK(stride_ok(out_seq_stride) && out_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD, "out_seq_stride too small");
        CHECK(cache != nullptr || (stride_ok(kv_seq_stride) && kv_seq_stride >= max_len * qsa::kHkv * qsa::kD),
              "kv_seq_stride smaller than the rows the queries reach");
        CHECK(sel_seq_stride >= int64_t{tq} * budget, "sel_seq_stride < tq * budget");
        CHECK(lse == nullptr || lse_seq_stride >= int64_t{tq} * qsa::kHq, "lse_seq_stride < tq * 24");
        CHECK(gate == nullptr || (stride_ok(gate_seq_stride) && gate_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD),
              "gate_seq_stride too small");
    }
    return hip_result(qsa::launch_attn_prefill(q, q_seq_stride, k_cache, v_cache, kv_seq_stride, sel,
                                               sel_seq_stride, p, batch, tq, budget, softmax_scale, out,
                                               out_seq_stride, lse, lse_seq_stride, gate, gate_seq_stride,
                                               cache != nullptr ? &pm : nullptr, stream),
                      "sparse_attn_prefill launch");
}

qsa_status_t qsa_sparse_attn_prefill(const uint16_t* q, int64_t q_seq_stride,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     int64_t kv_seq_stride,
                                     const int32_t* sel, int64_t sel_seq_stride,
                                     const int32_t* q_pos0, int32_t batch, int32_t tq,
                                     int32_t budget, float softmax_scale,
                                     uint16_t* out, int64_t out_seq_stride, float* lse,
                                     int64_t lse_seq_stride, const uint16_t* gate, int64_t gate_seq_stride,
                                     hipStream_t stream) {
    return sparse_attn_prefill_impl(q, q_seq_stride, k_cache, v_cache, kv_seq_stride, nullptr, sel, sel_seq_stride,
                                    q_pos0, batch, tq, budget, softmax_scale, out, out_seq_stride, lse,
                                    lse_seq_stride, gate, gate_seq_stride, stream);
}

qsa_status_t qsa_sparse_attn_prefill_paged(const uint16_t* q, int64_t q_seq_stride,
                                           const qsa_paged_cache_t* cache,
                                           const int32_t* sel, int64_t sel_seq_stride,
                                           const int32_t* q_pos0, int32_t batch, int32_t tq,
                                           int32_t budget, float softmax_scale,
                                           uint16_t* out, int64_t out_seq_stride, float* lse,
                                           int64_t lse_seq_stride, const uint16_t* gate, int64_t gate_seq_stride,
                                           hipStream_t stream) {
    CHECK(cache != nullptr, "cache is NULL");
    return sparse_attn_prefill_impl(q, q_seq_stride, nullptr, nullptr, 0, cache, sel, sel_seq_stride, q_pos0, batch,
                                    tq, budget, softmax_scale, out, out_seq_stride, lse, lse_seq_stride, gate,
                                    gate_seq_stride, stream);
}

static bool tq_ok(int32_t tq) { return tq >= 1 && tq <= qsa::kMaxDecodeTq; }
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t qsa_decode_workspace_bytes(int32_t batch, int32_t tq, int32_t budget) {
    if (batch < 1 || batch > QSA_MAX_BATCH || !tq_ok(tq) || budget < 1 || budget > QSA_MAX_BUDGET) return 0;
    return qsa::decode_workspace_bytes(batch * tq, budget);
}

// decode rows: per sequence q / out [tq][24][256], sel [tq][budget], lse [B*tq][24]
static qsa_status_t check_decode_attn(const qsa::Positions& p, int32_t batch, int32_t tq, int32_t budget,
                                      int64_t q_seq_stride, int64_t kv_seq_stride, int64_t sel_seq_stride,
                                      int64_t out_seq_stride, const float* lse, const uint16_t* gate,
                                      int64_t gate_seq_stride, bool paged = false) {
    CHECK(tq_ok(tq), "tq = %d outside [1, %d]", tq, qsa::kMaxDecodeTq);
    CHECK(gate == nullptr || aligned16(gate), "gate must be 16-byte aligned");
    CHECK(gate == nullptr || batch == 1 ||
              (stride_ok(gate_seq_stride) && gate_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD),
          "gate_seq_stride too small");
    CHECK(lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u) == 0, "lse must be 4-byte aligned");
    if (batch > 1) {
        int64_t max_len = 0;
        for (int b = 0; b < batch; ++b) max_len = p.p[b] + tq > max_len ? p.p[b] + tq : max_len;
        CHECK(stride_ok(q_seq_stride) && q_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD, "q_seq_stride too small");
        CHECK(stride_ok(out_seq_stride) && out_seq_stride >= int64_t{tq} * qsa::kHq * qsa::kD,
              "out_seq_stride too small");
        CHECK(paged || (stride_ok(kv_seq_stride) && kv_seq_stride >= max_len * qsa::kHkv * qsa::kD),
              "kv_seq_stride smaller than the rows the queries reach");
        CHECK(sel_seq_stride >= int64_t{tq} * budget, "sel_seq_stride < tq * budget");
    }
    return QSA_OK;
}

qsa_status_t qsa_sparse_attn_decode(const uint16_t* q, int64_t q_seq_stride,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int64_t kv_seq_stride,
                                    const int32_t* sel, int64_t sel_seq_stride,
                                    const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                    float softmax_scale, uint16_t* out, int64_t out_seq_stride,
                                    float* lse, const uint16_t* gate, int64_t gate_seq_stride,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    TRY(check_batch(batch));
    TRY(check_attn_common(q, k_cache, v_cache, sel, out, budget, softmax_scale));
    CHECK(tq_ok(tq), "tq = %d outside [1, %d]", tq, qsa::kMaxDecodeTq);
    qsa::Positions p;
    TRY(take_positions(q_pos, batch, tq, "q_pos", p));
    TRY(check_decode_attn(p, batch, tq, budget, q_seq_stride, kv_seq_stride, sel_seq_stride, out_seq_stride, lse,
                          gate, gate_seq_stride));
    const size_t need = qsa::decode_workspace_bytes(batch * tq, budget);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                    workspace == nullptr ? size_t{0} : workspace_bytes);
    CHECK(aligned16(workspace), "workspace must be 16-byte aligned");
    return hip_result(qsa::launch_attn_decode(q, q_seq_stride, k_cache, v_cache, kv_seq_stride, sel,
                                              sel_seq_stride, p, batch, tq, budget, softmax_scale, out,
                                              out_seq_stride, lse, gate, gate_seq_stride, workspace, stream),
                      "sparse_attn_decode launch");
}

size_t qsa_index_select_decode_workspace_bytes(int32_t batch, int32_t tq) {
    if (batch < 1 || batch > QSA_MAX_BATCH || !tq_ok(tq)) return 0;
    return qsa::decode_select_ws_bytes(batch * tq);
}

// per sequence q_idx [tq][4][128], scores [tq][scores_ld], sel [tq][budget]
static qsa_status_t check_index_select_decode(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                              const uint16_t* kbar, int64_t kbar_seq_stride,
                                              const qsa::Positions& p, int32_t batch, int32_t tq, int32_t budget,
                                              const float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                              const int32_t* sel, int64_t sel_seq_stride, bool paged = false) {
    CHECK(tq_ok(tq), "tq = %d outside [1, %d]", tq, qsa::kMaxDecodeTq);
    CHECK(q_idx != nullptr && kbar != nullptr && scores != nullptr && sel != nullptr,
          "q_idx, kbar, scores and sel must be non-NULL");
    CHECK(aligned16(q_idx) && aligned16(kbar) && aligned16(scores), "q_idx, kbar and scores must be 16-byte aligned");
    CHECK((reinterpret_cast<uintptr_t>(sel) & 3u) == 0, "sel must be 4-byte aligned");
    CHECK(budget >= 1 && budget <= QSA_MAX_BUDGET, "budget = %d outside [1, %d]", budget, QSA_MAX_BUDGET);
    int64_t o_max = 0;
    for (int b = 0; b < batch; ++b)
        o_max = (p.p[b] + tq - 1) / qsa::kBlock > o_max ? (p.p[b] + tq - 1) / qsa::kBlock : o_max;
    CHECK(scores_ld % 4 == 0 && scores_ld >= (o_max + 3) / 4 * 4,
          "scores_ld must be a multiple of 4 and >= (q_pos + tq - 1) / 4 rounded up to 4");
    if (batch > 1) {
        CHECK(stride_ok(q_idx_seq_stride) && q_idx_seq_stride >= int64_t{tq} * qsa::kHi * qsa::kDi,
              "q_idx_seq_stride too small");
        CHECK(paged || (stride_ok(kbar_seq_stride) && kbar_seq_stride >= o_max * qsa::kDi),
              "kbar_seq_stride too small");
        CHECK(scores_seq_stride % 4 == 0 && scores_seq_stride >= int64_t{tq} * scores_ld,
              "scores_seq_stride must be a multiple of 4 and >= tq * scores_ld");
        CHECK(sel_seq_stride >= int64_t{tq} * budget, "sel_seq_stride < tq * budget");
    }
    return QSA_OK;
}

qsa_status_t qsa_index_select_decode(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                     const uint16_t* kbar, int64_t kbar_seq_stride,
                                     const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                     float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                     int32_t* sel, int64_t sel_seq_stride,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    TRY(check_batch(batch));
    CHECK(tq_ok(tq), "tq = %d outside [1, %d]", tq, qsa::kMaxDecodeTq);
    qsa::Positions p;
    TRY(take_positions(q_pos, batch, tq, "q_pos", p));
    TRY(check_index_select_decode(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch, tq, budget, scores,
                                  scores_ld, scores_seq_stride, sel, sel_seq_stride));
    const size_t need = qsa::decode_select_ws_bytes(batch * tq);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "index-select workspace needs %zu bytes, got %zu", need,
                    workspace == nullptr ? size_t{0} : workspace_bytes);
    CHECK(aligned16(workspace), "workspace must be 16-byte aligned");
    return hip_result(qsa::launch_decode_index_select(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch, tq,
                                                      budget, scores, scores_seq_stride, scores_ld, sel,
                                                      sel_seq_stride, workspace, nullptr, nullptr, nullptr, stream),
                      "index_select_decode launch");
}

// decode step workspace: index-select part | attention partials | rotated
// queries.  The partials region holds max(256, rows) (row, split) slots, an
// upper bound for every budget (a row is split at most 256 / rows ways), so
// the total grows with the row count and a workspace sized for the largest
// call serves every smaller one.
static size_t step_attn_offset(int32_t rows) { return align256(qsa::decode_select_ws_bytes(rows)); }
static size_t step_qrot_offset(int32_t rows) {
    const size_t slots = rows > 256 ? static_cast<size_t>(rows) : size_t{256};
    return step_attn_offset(rows) + align256(slots * qsa::kHq * (2 + qsa::kD) * sizeof(float));
}

size_t qsa_decode_step_workspace_bytes(int32_t batch, int32_t tq, int32_t budget) {
    if (batch < 1 || batch > QSA_MAX_BATCH || !tq_ok(tq) || budget < 1 || budget > QSA_MAX_BUDGET) return 0;
    const int32_t rows = batch * tq;
    return step_qrot_offset(rows) + static_cast<size_t>(rows) * qsa::kHq * qsa::kD * 2;
}

// caches contiguous (per-sequence strides), or (cache non-NULL) the paged
// pools of `cache`
static qsa_status_t decode_step_impl(const uint16_t* q, int64_t q_seq_stride,
                                     const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                                     const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                     const uint16_t* k_idx_new,
                                     uint16_t* k_cache, uint16_t* v_cache, int64_t kv_seq_stride,
                                     uint16_t* k_idx, int64_t k_idx_seq_stride,
                                     uint16_t* kbar, int64_t kbar_seq_stride, const qsa_paged_cache_t* cache,
                                     const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                     float softmax_scale, const qsa_rope_t* rope,
                                     float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                     int32_t* sel, int64_t sel_seq_stride,
                                     uint16_t* out, int64_t out_seq_stride, float* lse,
                                     const uint16_t* gate, int64_t gate_seq_stride,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     bool validate_only = false) {
    TRY(check_batch(batch));
    CHECK(tq_ok(tq), "tq = %d outside [1, %d]", tq, qsa::kMaxDecodeTq);
    qsa::Positions p;
    TRY(take_positions(q_pos, batch, tq, "q_pos", p));
    const bool paged = cache != nullptr;
    qsa::PageMap pm{};
    if (paged) {
        TRY(take_paged(cache, p, batch, tq, true, false, true, pm));
        k_cache = cache->k;
        v_cache = cache->v;
        k_idx = cache->k_idx;
        kbar = cache->kbar;
    }
    TRY(check_index_select_decode(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch, tq, budget, scores,
                                  scores_ld, scores_seq_stride, sel, sel_seq_stride, paged));
    TRY(check_attn_common(q, k_cache, v_cache, sel, out, budget, softmax_scale));
    TRY(check_decode_attn(p, batch, tq, budget, q_seq_stride, kv_seq_stride, sel_seq_stride, out_seq_stride, lse,
                          gate, gate_seq_stride, paged));
    CHECK(k_new != nullptr && aligned16(k_new), "k_new must be non-NULL and 16-byte aligned");
    CHECK(v_new == nullptr || aligned16(v_new), "v_new must be 16-byte aligned");
    CHECK(k_idx_new == nullptr || k_idx != nullptr, "k_idx_new needs the k_idx cache");
    CHECK(k_idx_new == nullptr || aligned16(k_idx_new), "k_idx_new must be 16-byte aligned");
    CHECK(k_idx == nullptr || aligned16(k_idx), "k_idx must be 16-byte aligned");
    qsa_rope_t rp;
    TRY(take_rope(rope, rp));
    if (batch > 1) {
        int64_t max_len = 0;
        for (int b = 0; b < batch; ++b) max_len = p.p[b] + tq > max_len ? p.p[b] + tq : max_len;
        CHECK(stride_ok(kv_new_seq_stride) && kv_new_seq_stride >= int64_t{tq} * qsa::kHkv * qsa::kD,
              "kv_new_seq_stride too small");
        CHECK(paged || k_idx == nullptr ||
                  (stride_ok(k_idx_seq_stride) && k_idx_seq_stride >= max_len * qsa::kDi),
              "k_idx_seq_stride smaller than the rows the new tokens reach");
        CHECK(paged || k_idx == nullptr || kbar_seq_stride >= (max_len / qsa::kBlock) * qsa::kDi,
              "kbar_seq_stride smaller than the blocks the new tokens complete");
    }
    if (validate_only) return QSA_OK;
    const size_t need = qsa_decode_step_workspace_bytes(batch, tq, budget);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "decode step workspace needs %zu bytes, got %zu", need,
                    workspace == nullptr ? size_t{0} : workspace_bytes);
    CHECK(aligned16(workspace), "workspace must be 16-byte aligned");
    char* wsb = static_cast<char*>(workspace);
    uint16_t* q_rot = reinterpret_cast<uint16_t*>(wsb + step_qrot_offset(batch * tq));
    qsa::DecodeAppend ap{};
    ap.k_new = k_new;
    ap.kns = kv_new_seq_stride;
    ap.k_cache = k_cache;
    ap.v_new = v_new;
    ap.vns = kv_new_seq_stride;
    ap.v_cache = v_cache;
    ap.kvs = kv_seq_stride;
    ap.k_idx_new = k_idx_new;
    ap.kins = int64_t{tq} * qsa::kDi;
    ap.k_idx = k_idx;
    ap.kis = k_idx_seq_stride;
    ap.kbar = kbar;
    ap.kbs = kbar_seq_stride;
    ap.rope = rp;
    const qsa::DecodeQrot qr{q, q_seq_stride, q_rot, rp};
    hipError_t e = qsa::launch_decode_index_select(q_idx, q_idx_seq_stride, kbar, kbar_seq_stride, p, batch, tq,
                                                   budget, scores, scores_seq_stride, scores_ld, sel, sel_seq_stride,
                                                   workspace, &ap, &qr, paged ? &pm : nullptr, stream);
    if (e != hipSuccess) return hip_result(e, "decode_step index-select launch");
    return hip_result(qsa::launch_attn_decode_ex(q_rot, int64_t{tq} * qsa::kHq * qsa::kD, k_cache, v_cache,
                                                 kv_seq_stride, sel, sel_seq_stride, p, batch, tq, budget,
                                                 softmax_scale, out, out_seq_stride, lse, gate, gate_seq_stride,
                                                 wsb + step_attn_offset(batch * tq), nullptr, paged ? &pm : nullptr,
                                                 stream),
                      "decode_step attention launch");
}

qsa_status_t qsa_decode_step(const uint16_t* q, int64_t q_seq_stride,
                             const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                             const uint16_t* q_idx, int64_t q_idx_seq_stride,
                             const uint16_t* k_idx_new,
                             uint16_t* k_cache, uint16_t* v_cache, int64_t kv_seq_stride,
                             uint16_t* k_idx, int64_t k_idx_seq_stride,
                             uint16_t* kbar, int64_t kbar_seq_stride,
                             const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                             float softmax_scale, const qsa_rope_t* rope,
                             float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                             int32_t* sel, int64_t sel_seq_stride,
                             uint16_t* out, int64_t out_seq_stride, float* lse,
                             const uint16_t* gate, int64_t gate_seq_stride,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_step_impl(q, q_seq_stride, k_new, v_new, kv_new_seq_stride, q_idx, q_idx_seq_stride, k_idx_new,
                            k_cache, v_cache, kv_seq_stride, k_idx, k_idx_seq_stride, kbar, kbar_seq_stride, nullptr,
                            q_pos, batch, tq, budget, softmax_scale, rope, scores, scores_ld, scores_seq_stride, sel,
                            sel_seq_stride, out, out_seq_stride, lse, gate, gate_seq_stride, workspace,
                            workspace_bytes, stream);
}

qsa_status_t qsa_decode_step_paged(const uint16_t* q, int64_t q_seq_stride,
                                   const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                                   const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                   const uint16_t* k_idx_new, const qsa_paged_cache_t* cache,
                                   const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                   float softmax_scale, const qsa_rope_t* rope,
                                   float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                   int32_t* sel, int64_t sel_seq_stride,
                                   uint16_t* out, int64_t out_seq_stride, float* lse,
                                   const uint16_t* gate, int64_t gate_seq_stride,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    CHECK(cache != nullptr, "cache is NULL");
    return decode_step_impl(q, q_seq_stride, k_new, v_new, kv_new_seq_stride, q_idx, q_idx_seq_stride, k_idx_new,
                            nullptr, nullptr, 0, nullptr, 0, nullptr, 0, cache, q_pos, batch, tq, budget,
                            softmax_scale, rope, scores, scores_ld, scores_seq_stride, sel, sel_seq_stride, out,
                            out_seq_stride, lse, gate, gate_seq_stride, workspace, workspace_bytes, stream);
}

qsa_status_t qsa_decode_step_noalloc(const uint16_t* q, int64_t q_seq_stride,
                                     const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                                     const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                     const uint16_t* k_idx_new,
                                     uint16_t* k_cache, uint16_t* v_cache, int64_t kv_seq_stride,
                                     uint16_t* k_idx, int64_t k_idx_seq_stride,
                                     uint16_t* kbar, int64_t kbar_seq_stride,
                                     const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                     float softmax_scale, const qsa_rope_t* rope,
                                     float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                     int32_t* sel, int64_t sel_seq_stride,
                                     uint16_t* out, int64_t out_seq_stride, float* lse,
                                     const uint16_t* gate, int64_t gate_seq_stride, hipStream_t stream) {
    const size_t need = qsa_decode_step_workspace_bytes(batch, tq, budget);
    if (need == 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "batch = %d, tq = %d or budget = %d out of range", batch, tq, budget);
    if (need > QSA_NOALLOC_SCRATCH_BYTES)
        return fail(QSA_ERR_WORKSPACE, "decode step needs %zu bytes of scratch; the static buffer holds %zu", need,
                    size_t{QSA_NOALLOC_SCRATCH_BYTES});
    // every argument check first (no HIP call): a rejected call leaves the scratch as it was
    TRY(decode_step_impl(q, q_seq_stride, k_new, v_new, kv_new_seq_stride, q_idx, q_idx_seq_stride, k_idx_new,
                         k_cache, v_cache, kv_seq_stride, k_idx, k_idx_seq_stride, kbar, kbar_seq_stride, nullptr,
                         q_pos, batch, tq, budget, softmax_scale, rope, scores, scores_ld, scores_seq_stride, sel,
                         sel_seq_stride, out, out_seq_stride, lse, gate, gate_seq_stride, nullptr, 0, stream,
                         /*validate_only=*/true));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchSlot* slot = nullptr;
    TRY(scratch_for_current_device(stream, &slot));
    const qsa_status_t st = decode_step_impl(q, q_seq_stride, k_new, v_new, kv_new_seq_stride, q_idx,
                                             q_idx_seq_stride, k_idx_new, k_cache, v_cache, kv_seq_stride, k_idx,
                                             k_idx_seq_stride, kbar, kbar_seq_stride, nullptr, q_pos, batch, tq,
                                             budget, softmax_scale, rope, scores, scores_ld, scores_seq_stride, sel,
                                             sel_seq_stride, out, out_seq_stride, lse, gate, gate_seq_stride,
                                             slot->ptr, QSA_NOALLOC_SCRATCH_BYTES, stream);
    if (st != QSA_OK) slot->clean = false;       // launched part-way: zero-fill again on the next call
    return st;
}

qsa_status_t qsa_paged_append(const qsa_paged_cache_t* cache,
                              const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                              const uint16_t* k_idx_new, int64_t k_idx_new_seq_stride,
                              const int32_t* pos0, int32_t batch, int32_t n_tokens, const qsa_rope_t* rope,
                              hipStream_t stream) {
    TRY(check_batch(batch));
    CHECK(n_tokens >= 0, "n_tokens = %d is negative", n_tokens);
    CHECK(k_new == nullptr || aligned16(k_new), "k_new must be 16-byte aligned");
    CHECK(v_new == nullptr || aligned16(v_new), "v_new must be 16-byte aligned");
    CHECK(k_idx_new == nullptr || aligned16(k_idx_new), "k_idx_new must be 16-byte aligned");
    qsa::Positions p;
    TRY(take_positions(pos0, batch, n_tokens, "pos0", p));
    qsa_rope_t rp;
    TRY(take_rope(rope, rp));
    qsa::PageMap pm{};
    CHECK(cache != nullptr, "cache is NULL");
    const bool compress = cache->kbar != nullptr;
    TRY(take_paged(cache, p, batch, n_tokens, k_new != nullptr || v_new != nullptr,
                   k_idx_new != nullptr || compress, compress, pm));
    if (n_tokens == 0) return ok();
    if (batch > 1) {
        CHECK((k_new == nullptr && v_new == nullptr) ||
                  (stride_ok(kv_new_seq_stride) && kv_new_seq_stride >= int64_t{n_tokens} * qsa::kHkv * qsa::kD),
              "kv_new_seq_stride too small");
        CHECK(k_idx_new == nullptr ||
                  (stride_ok(k_idx_new_seq_stride) && k_idx_new_seq_stride >= int64_t{n_tokens} * qsa::kDi),
              "k_idx_new_seq_stride too small");
    }
    return hip_result(qsa::launch_paged_append(pm, cache->k, cache->v, cache->k_idx, cache->kbar, k_new, v_new,
                                               kv_new_seq_stride, k_idx_new, k_idx_new_seq_stride, p, batch,
                                               n_tokens, rp, stream),
                      "paged_append launch");
}

size_t qsa_gdn_prefill_workspace_bytes(int32_t batch, int32_t n_tokens) {
    if (batch < 1 || batch > QSA_MAX_BATCH || n_tokens < 0) return 0;
    return qsa::gdn_prefill_ws_bytes(batch, n_tokens);
}

static qsa_status_t check_gdn_common(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                                     const float* beta, const float* state, const uint16_t* out) {
    CHECK(q != nullptr && k != nullptr && v != nullptr && g != nullptr && beta != nullptr && state != nullptr &&
              out != nullptr,
          "q, k, v, g, beta, state and out must be non-NULL");
    CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(state),
          "q, k, v, out and state must be 16-byte aligned");
    CHECK((reinterpret_cast<uintptr_t>(g) & 3u) == 0 && (reinterpret_cast<uintptr_t>(beta) & 3u) == 0,
          "g and beta must be 4-byte aligned");
    return QSA_OK;
}

qsa_status_t qsa_gdn_prefill(const uint16_t* q, const uint16_t* k, int64_t qk_seq_stride,
                             const uint16_t* v, int64_t v_seq_stride,
                             const float* g, const float* beta, int64_t gate_seq_stride,
                             float* state, int32_t batch, int32_t n_tokens,
                             uint16_t* out, int64_t out_seq_stride,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    TRY(check_batch(batch));
    TRY(check_gdn_common(q, k, v, g, beta, state, out));
    CHECK(n_tokens >= 0 && n_tokens <= (1 << 30), "n_tokens = %d outside [0, 2^30]", n_tokens);
    if (n_tokens == 0) return ok();
    if (batch > 1) {
        const int64_t T = n_tokens;
        CHECK(stride_ok(qk_seq_stride) && qk_seq_stride >= T * 16 * 128, "qk_seq_stride too small");
        CHECK(stride_ok(v_seq_stride) && v_seq_stride >= T * 48 * 128, "v_seq_stride too small");
        CHECK(stride_ok(out_seq_stride) && out_seq_stride >= T * 48 * 128, "out_seq_stride too small");
        CHECK(gate_seq_stride >= T * 48, "gate_seq_stride too small");
    }
    const size_t need = qsa::gdn_prefill_ws_bytes(batch, n_tokens);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "gdn prefill workspace needs %zu bytes, got %zu", need,
                    workspace == nullptr ? size_t{0} : workspace_bytes);
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "workspace must be 256-byte aligned");
    const qsa::GdnIn in{q, k, qk_seq_stride, v, v_seq_stride, g, beta, gate_seq_stride, state, out, out_seq_stride};
    return hip_result(qsa::launch_gdn_prefill(in, batch, n_tokens, workspace, stream), "gdn_prefill launch");
}

qsa_status_t qsa_gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                            const float* beta, float* state, int32_t batch, uint16_t* out, hipStream_t stream) {
    TRY(check_batch(batch));
    TRY(check_gdn_common(q, k, v, g, beta, state, out));
    const qsa::GdnIn in{q, k, 16 * 128, v, 48 * 128, g, beta, 48, state, out, 48 * 128};
    return hip_result(qsa::launch_gdn_decode(in, batch, stream), "gdn_decode launch");
}

}  // extern "C"
