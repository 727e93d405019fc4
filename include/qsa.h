/*
 * qsa.h -- C ABI of libqsa: one layer of Qwen Sparse Attention (QSA) on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages state it (Qwen3.8-Flash-Next blog, section
 * "Attention: GDN + QSA"): a lightweight indexer aggregates the sequence into
 * micro-blocks, estimates importance per block, selects the most relevant
 * blocks, and attention runs over the selected regions only.  Shapes (model
 * card, "Model Overview" -> "Qwen Sparse Attention"): 24 query heads, 2 KV
 * heads, head dim 256, rotary dim 64, indexer = MQA with 4 query heads and 1
 * shared key head of dim 128, budget 512 blocks or 2048 tokens, hence 4 tokens
 * per micro-block.  The calls below are those steps, in that order:
 *
 *   qsa_rope_apply           rotary embedding of Q / K rows     (step 0)
 *   qsa_compress_block_keys  indexer keys -> block keys          (step 1)
 *   qsa_index_scores         block scores of the MQA indexer     (step 2)
 *   qsa_select_topk          per-token top-(budget-1) + own block (step 3)
 *   qsa_index_select_prefill steps 2 + 3 for a prefill chunk, no score matrix
 *   qsa_sparse_attn_prefill  attention over the selected tokens  (step 4)
 *   qsa_sparse_attn_decode   the same for one new token per sequence
 *   qsa_decode_step          a whole serving decode step in one call
 *   qsa_*_paged              the same on paged caches (block table)
 *   qsa_gdn_prefill / _decode the Gated DeltaNet token mixer of the other layers
 *
 * Conventions shared by every call
 *   - bf16 tensors are passed as uint16_t bit patterns; every tensor pointer
 *     is caller-owned DEVICE memory, 16-byte aligned; strides are in
 *     elements and must be multiples of 8 (16 bytes).
 *   - Layouts are token-major with the last dimension contiguous:
 *       Q       [B][T][24][256]      K, V caches [B][L][2][256]
 *       q_idx   [B][T][4][128]       k_idx       [B][L][128]
 *       kbar    [B][L/4][128]        scores      [B][T][ld] float
 *       sel     [B][T][budget] int32
 *     "seq_stride" is the distance between sequences b and b+1.
 *   - Positions are HOST int32 arrays of length `batch` (at most
 *     QSA_MAX_BATCH), so validation and grid sizing never wait on the GPU.
 *     Query row i of sequence b sits at absolute position q_pos0[b] + i; its
 *     own block is o = position / 4.
 *   - Every call is asynchronous on `stream`, never synchronises, never
 *     allocates, and launches nothing when validation fails.  Errors come
 *     back as a status; qsa_last_error() gives the message (thread-local).
 *   - Calls on one stream run in order; calls on different streams that
 *     share output buffers race.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 4
#define QSA_MAX_BATCH 256
#define QSA_MAX_BUDGET 2048

typedef enum {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or stride */
    QSA_ERR_UNSUPPORTED = 2,      /* legal but outside what the library handles */
    QSA_ERR_WORKSPACE = 3,        /* workspace missing or too small             */
    QSA_ERR_HIP = 4               /* a HIP runtime call or launch failed        */
} qsa_status_t;

/* Fixed head geometry (model card "Model Overview"): block 4 tokens, 24 Q
 * heads, 2 KV heads, head dim 256, rotary dim 64, 4 indexer heads of dim 128. */
typedef struct {
    int32_t block, hq, hkv, d, rot_dim, hi, di;
} qsa_dims_t;

int32_t      qsa_abi_version(void);
qsa_status_t qsa_get_dims(qsa_dims_t* out);
const char*  qsa_status_string(qsa_status_t s);
const char*  qsa_last_error(void);

/*
 * Measurement hook, not part of the method: while set on the calling host
 * thread, every decode index-select (qsa_index_select_decode and the decode
 * steps, which run it) records `begin_event` on its stream right before it
 * launches the block-key scan kernel and `end_event` right after, so the
 * caller can time that kernel alone with hipEventElapsedTime.  The events are
 * caller-owned hipEvent_t handles (created with timing enabled, on the device
 * of the calls); NULL, NULL turns the hook off.  Only stores the two
 * handles; always returns QSA_OK.
 */
qsa_status_t qsa_set_scan_timing_events(void* begin_event, void* end_event);

/*
 * Diagnostic hook, not part of the method: while set on the calling host
 * thread, every decode index-select adds 1 to the device uint32 at `counter`
 * for each row that takes its exact path over the stored scores instead of
 * the candidate list (the list overflowed, or its cut fell below a scan
 * wave's threshold: score patterns far from random order, such as large tie
 * groups).  The selection is the same either way; the exact path is slower.
 * `counter` is caller-owned device memory on the device of the calls; the
 * caller zeroes and reads it.  NULL turns the hook off.  Only stores the
 * pointer; always returns QSA_OK.
 */
qsa_status_t qsa_set_decode_fallback_counter(uint32_t* counter);

/*
 * Rotary parameters (model card, "Processing Ultra-Long Texts",
 * rope_parameters): rope_theta (1e7 for this model) and optional static YaRN
 * (rope_type "yarn": scale factor s over original_max_position_embeddings L;
 * the card gives s = 4, L = 262144 for contexts past 262144, s = 2 for about
 * 512K).  Passed by HOST pointer, read during the call; NULL means
 * {1e7, 1, 0}.  theta must be finite and > 1, yarn_factor finite and >= 1
 * (1: plain rotary), yarn_original_max >= 1 when yarn_factor > 1; otherwise
 * QSA_ERR_INVALID_ARGUMENT.
 */
typedef struct {
    double  theta;
    double  yarn_factor;
    int64_t yarn_original_max;
} qsa_rope_t;

/*
 * Step 0 -- rotary embedding (model card, "Processing Ultra-Long Texts",
 * rope_parameters: rope_theta 1e7, partial_rotary_factor 0.25, i.e. the first
 * 64 of 256 dims; mRoPE sections [11, 11, 10] reduce to 1-D rotary for text).
 * For every row (b, i) and head h of x [B][n_tokens][n_heads][256]:
 * pair (d, d + 32), d < 32, is turned by angle p * w_d with
 * p = pos0[b] + i:  (a, c) -> (a cos - c sin, c cos + a sin) * m.  Plain
 * rotary: w_d = theta^(-d/32), m = 1.  Static YaRN (YaRN paper, Peng et al.
 * 2023, NTK-by-parts interpolation and attention temperature; the same table
 * at every length): pair d turns L w_d / (2 pi) times over the original
 * context; with i(rho) = 32 ln(L / (2 pi rho)) / ln theta the pair index
 * turning rho times, lo = floor(i(32)) (>= 0), hi = ceil(i(1)) (<= 63),
 * g_d = clamp((d - lo) / (hi - lo), 0, 1): w_d becomes
 * (w_d / s) g_d + w_d (1 - g_d), and m = 1 + 0.1 ln s.  Angles, sines and
 * the rotation are evaluated in float64, the result rounded once to bf16;
 * dims 64..255 are copied unchanged.  y may equal x (same strides) for an
 * in-place update; otherwise x and y must not overlap.
 */
qsa_status_t qsa_rope_apply(const uint16_t* x, int64_t x_seq_stride, int64_t x_tok_stride,
                            uint16_t* y, int64_t y_seq_stride, int64_t y_tok_stride,
                            int32_t batch, int32_t n_tokens, int32_t n_heads,
                            const int32_t* pos0, const qsa_rope_t* rope, hipStream_t stream);

/*
 * Step 1 -- block keys (blog, "Attention: GDN + QSA": aggregate into
 * micro-blocks).  For blocks j in [block_begin, block_end) of every sequence:
 *   kbar[b][j][d] = bf16( ((k[4j][d] + k[4j+1][d]) + k[4j+2][d]) + k[4j+3][d]) * 0.25 )
 * with the additions in float32 in token order and round-to-nearest-even.
 * k_idx [B][>= 4*block_end][128], kbar [B][>= block_end][128].
 */
qsa_status_t qsa_compress_block_keys(const uint16_t* k_idx, int64_t k_idx_seq_stride,
                                     int32_t batch, int32_t block_begin, int32_t block_end,
                                     uint16_t* kbar, int64_t kbar_seq_stride, hipStream_t stream);

/*
 * Step 2 -- block scores of the MQA indexer (model card: 4 query heads share
 * 1 key head of dim 128).  For query row i of sequence b at position
 * p = q_pos0[b] + i and every complete block j < p / 4:
 *   scores[b][i][j] = sum_h sum_d q_idx[b][i][h][d] * kbar[b][j][d]
 * computed as sum_d (sum_h q_idx[b][i][h][d]) * kbar[b][j][d]: the head sum
 * in float32, split exactly into three bf16 terms, whose 384 exact products
 * with kbar accumulate in float32 (matrix-core tiles); every entry point that
 * scores blocks produces the same bits.
 * Entries j >= p / 4 of a row are left unspecified (not written, or written
 * with values the selection never reads).  Needs scores_ld >= (q_pos0[b] +
 * tq - 1) / 4 for all b, scores_ld % 4 == 0, and kbar holding those blocks.
 */
qsa_status_t qsa_index_scores(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                              const uint16_t* kbar, int64_t kbar_seq_stride,
                              const int32_t* q_pos0, int32_t batch, int32_t tq,
                              float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                              hipStream_t stream);

/*
 * Step 3 -- block selection (blog: select the most relevant regions; model
 * card: budget 512 blocks).  For query row i at position p, own block
 * o = p / 4: keep min(budget - 1, o) of the candidates j < o ordered by
 * (score descending, j ascending), with -0.0 equal to +0.0 and NaN below
 * every number, add o, and write the set ascending into sel[b][i][0..budget),
 * padded with -1.  The selection is exact: it depends only on the float32
 * score bits.  workspace may be NULL when qsa_select_workspace_bytes() is 0.
 */
size_t       qsa_select_workspace_bytes(int32_t batch, int32_t tq, int32_t budget);
qsa_status_t qsa_select_topk(const float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                             const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                             int32_t* sel, int64_t sel_seq_stride,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Steps 2 + 3 fused for a prefill chunk (blog "Attention: GDN + QSA": blocks
 * are scored and the most relevant kept): the same selection as
 * qsa_index_scores followed by qsa_select_topk, bit for bit, without
 * materialising the score matrix when the chunk is long.  The indexer first
 * scores a fixed sample of 4096 blocks per row to set a per-row threshold,
 * then scores every block keeping only those at or above it, and an exact
 * radix select finishes each row from that list.  Rows whose list is short
 * or overflows are redone exactly from full scores, so the result never
 * depends on the threshold.  The fused path is taken when budget <= 1024 and
 * every sequence's first row sees at least 16384 blocks; otherwise the call
 * runs qsa_index_scores + qsa_select_topk.
 * scores [B][tq][ld] float, laid out as for qsa_index_scores, is scratch for
 * those exact paths (its contents are unspecified afterwards); sel
 * [B][tq][budget].  The workspace (qsa_index_select_prefill_workspace_bytes,
 * about 64 KiB per query row, 256-byte aligned) needs no initialisation;
 * calls that share a workspace must not overlap.
 */
size_t       qsa_index_select_prefill_workspace_bytes(int32_t batch, int32_t tq);
qsa_status_t qsa_index_select_prefill(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                      const uint16_t* kbar, int64_t kbar_seq_stride,
                                      const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                                      float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                      int32_t* sel, int64_t sel_seq_stride,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Step 4 -- sparse grouped-query attention (model card: 24 Q heads, 2 KV
 * heads, dim 256).  For query row i at position p and head h, with KV head
 * g = h / 12: softmax over the tokens n of the selected blocks (4 per block,
 * n <= p) of scale * q[h] . k[n][g], times v[n][g]; float32 accumulation,
 * online softmax.  out [B][tq][24][256] bf16; lse [B][tq][24] float (natural
 * log of the softmax denominator, including the scale; sequence stride
 * lse_seq_stride elements), may be NULL.
 * k_cache / v_cache rows must hold positions 0 .. q_pos0[b] + tq - 1; q and K
 * are expected already rotated.  sel entries outside [0, p/4] are skipped.
 * gate (may be NULL; bf16, laid out as out with sequence stride
 * gate_seq_stride): the attention output gate (blog, "Training stability":
 * the attention output gating mechanism is retained) -- each output value is
 * multiplied by 1 / (1 + exp(-g)) of its gate logit before rounding; lse is
 * not gated.  The decode entries below take the same optional gate.
 */
qsa_status_t qsa_sparse_attn_prefill(const uint16_t* q, int64_t q_seq_stride,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     int64_t kv_seq_stride,
                                     const int32_t* sel, int64_t sel_seq_stride,
                                     const int32_t* q_pos0, int32_t batch, int32_t tq,
                                     int32_t budget, float softmax_scale,
                                     uint16_t* out, int64_t out_seq_stride, float* lse,
                                     int64_t lse_seq_stride, const uint16_t* gate,
                                     int64_t gate_seq_stride, hipStream_t stream);

/*
 * Decode rows.  The decode entries below take tq = 1 .. QSA_MAX_DECODE_TQ
 * consecutive query tokens per sequence (one for plain decoding, several for
 * multi-token prediction or speculative verification): token t of sequence b
 * sits at position q_pos[b] + t and attends causally, so it sees the earlier
 * new tokens.  Each (sequence, token) is a row with its own selection.  Per
 * sequence: q and out [tq][24][256], q_idx [tq][4][128], sel [tq][budget],
 * scores [tq][scores_ld]; lse is [batch * tq][24].  The tokens of a sequence
 * share one pass over its block keys (they are columns of the same
 * matrix-core tiles).
 */
#define QSA_MAX_DECODE_TQ 4

/*
 * Step 4, decode form, for decode rows.  The selected blocks of every row are
 * split over many workgroups whose partial softmax states (max, sum, weighted
 * V) go to `workspace` and are merged by a final reduction.  workspace must
 * hold qsa_decode_workspace_bytes(batch, tq, budget).
 */
size_t       qsa_decode_workspace_bytes(int32_t batch, int32_t tq, int32_t budget);
qsa_status_t qsa_sparse_attn_decode(const uint16_t* q, int64_t q_seq_stride,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int64_t kv_seq_stride,
                                    const int32_t* sel, int64_t sel_seq_stride,
                                    const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                    float softmax_scale, uint16_t* out, int64_t out_seq_stride,
                                    float* lse, const uint16_t* gate, int64_t gate_seq_stride,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Steps 2 + 3 fused for decode rows: writes the same scores as
 * qsa_index_scores (q_pos0 = q_pos, the same tq) and the same selection as
 * qsa_select_topk, bit for bit, in two launches that spread each row over
 * many workgroups (a scan whose workgroups each list their own top
 * candidates of every row, then a per-row exact finish over the lists, with
 * the full radix select of the stored row where a list cannot decide).  The
 * scan's workgroup size in blocks and each row's list capacity are chosen
 * per call from batch, tq, the longest context and the budget, so that
 * randomly ordered scores fit the lists (qsa_set_decode_fallback_counter
 * counts the rows that do not); the workspace holds lists for at least 8
 * rows, which calls with fewer rows use as longer lists.
 * scores [B][tq][scores_ld] float with scores_ld >= (q_pos + tq - 1)/4
 * rounded up to a multiple of 4 (entries past a row's own block are
 * scratch), 16-byte aligned.  The workspace
 * (qsa_index_select_decode_workspace_bytes) starts with control words laid
 * out for the largest row count: it must be zero-filled before its first
 * use, and every call leaves them zeroed again, so one workspace serves
 * calls of any shape it is large enough for.  Calls that share a workspace
 * must not overlap.
 */
size_t       qsa_index_select_decode_workspace_bytes(int32_t batch, int32_t tq);
qsa_status_t qsa_index_select_decode(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                     const uint16_t* kbar, int64_t kbar_seq_stride,
                                     const int32_t* q_pos, int32_t batch, int32_t tq, int32_t budget,
                                     float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                     int32_t* sel, int64_t sel_seq_stride,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One whole decode step of the layer for decode rows: tq new tokens per
 * sequence at positions q_pos[b] .. q_pos[b] + tq - 1 (steps 0 to 4;
 * positions may differ per sequence).  In order, as one asynchronous call:
 *  - appends the new tokens' rows: the unrotated key rows k_new
 *    [B][tq][2][256] are rotated into k_cache[b][q_pos[b] + t]; v_new
 *    [B][tq][2][256] (NULL: the rows are already in v_cache) is copied to
 *    v_cache; k_idx_new [B][tq][128] contiguous (NULL: the rows are already in
 *    k_idx) is copied to k_idx;
 *  - when a new token completes its block (position % 4 == 3) and k_idx is
 *    given, writes that block's key into kbar exactly as
 *    qsa_compress_block_keys would (the later new tokens of the step score it;
 *    a block the last token completes serves the next steps);
 *  - scores the candidate blocks of each row and selects as
 *    qsa_index_select_decode does;
 *  - attends with q (unrotated; rotated once, exactly as qsa_rope_apply
 *    would with the same rope parameters, into the workspace) over each
 *    row's selection and own block.
 * k_idx NULL: no indexer-key append and no compression.  k_new / v_new share
 * kv_new_seq_stride; k_cache and v_cache share kv_seq_stride; k_idx is
 * [B][L][128] with k_idx_seq_stride.  Equals the chain rope_apply + row
 * copies + compress_block_keys + index_scores + select_topk +
 * sparse_attn_decode bit for bit.  The workspace
 * (qsa_decode_step_workspace_bytes) must be zero-filled before its first use;
 * every call leaves the control words at its start zeroed again (the rest is
 * scratch), so it serves calls of any shape it is large enough for.
 */
size_t       qsa_decode_step_workspace_bytes(int32_t batch, int32_t tq, int32_t budget);
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
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged caches with a block table (Qwen3.8-Flash-Next blog, section
 * "Attention: GDN + QSA": online serving with high prefix-cache reuse, a 90%
 * prefix-cache hit rate).  The four caches are pools of pages of P tokens:
 *   k, v    [n_pages][P][2][256]   (K rotated, as in the contiguous caches)
 *   k_idx   [n_pages][P][128]
 *   kbar    [n_pages][P/4][128]
 * block_table is DEVICE int32 [batch][table_stride]: token n of sequence b
 * sits in page block_table[b][n / P], row n % P of it (block j in the page
 * of token 4j, row j % (P/4)).  One table serves all four pools.  P is a power
 * of two in [64, 65536]; each sequence's table row must hold the pages of
 * its tokens up to the last position a call touches (checked against
 * table_stride when batch > 1; the entries themselves live on the device and
 * are not read by the host).  Page ids are clamped to [0, n_pages) on the
 * device, so a bad table gives wrong values, never an access outside the
 * pools.  Sequences may share pages (a common prefix); pages that a call
 * writes must belong to one sequence only.  Results are bit-identical to the
 * contiguous entry points on the same logical contents.
 */
typedef struct {
    uint16_t*      k;
    uint16_t*      v;
    uint16_t*      k_idx;
    uint16_t*      kbar;
    const int32_t* block_table;
    int64_t        table_stride;
    int32_t        page_tokens;
    int32_t        n_pages;
} qsa_paged_cache_t;

/*
 * Steps 0 + 1 on a paged cache: the new tokens pos0[b] .. pos0[b] + n_tokens - 1
 * of every sequence are written into their pages -- the unrotated key rows
 * k_new [B][T][2][256] rotated as qsa_rope_apply would, v_new [B][T][2][256]
 * copied (k_new and v_new share kv_new_seq_stride), k_idx_new [B][T][128]
 * copied; a NULL input is skipped.  Then, when cache->kbar is non-NULL, the
 * key of every block the new tokens complete (4j + 3 in the range) is written
 * exactly as qsa_compress_block_keys would, from the block's rows in k_idx.
 */
qsa_status_t qsa_paged_append(const qsa_paged_cache_t* cache,
                              const uint16_t* k_new, const uint16_t* v_new, int64_t kv_new_seq_stride,
                              const uint16_t* k_idx_new, int64_t k_idx_new_seq_stride,
                              const int32_t* pos0, int32_t batch, int32_t n_tokens, const qsa_rope_t* rope,
                              hipStream_t stream);

/* qsa_index_select_prefill with the block keys read from cache->kbar through
 * the block table (workspace: qsa_index_select_prefill_workspace_bytes). */
qsa_status_t qsa_index_select_prefill_paged(const uint16_t* q_idx, int64_t q_idx_seq_stride,
                                            const qsa_paged_cache_t* cache,
                                            const int32_t* q_pos0, int32_t batch, int32_t tq, int32_t budget,
                                            float* scores, int64_t scores_ld, int64_t scores_seq_stride,
                                            int32_t* sel, int64_t sel_seq_stride,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* qsa_sparse_attn_prefill with K and V gathered from cache->k / cache->v
 * through the block table. */
qsa_status_t qsa_sparse_attn_prefill_paged(const uint16_t* q, int64_t q_seq_stride,
                                           const qsa_paged_cache_t* cache,
                                           const int32_t* sel, int64_t sel_seq_stride,
                                           const int32_t* q_pos0, int32_t batch, int32_t tq,
                                           int32_t budget, float softmax_scale,
                                           uint16_t* out, int64_t out_seq_stride, float* lse,
                                           int64_t lse_seq_stride, const uint16_t* gate, int64_t gate_seq_stride,
                                           hipStream_t stream);

/*
 * qsa_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as qsa_decode_step (bit for bit), without the
 * workspace: its kernels use a static device buffer of
 * QSA_NOALLOC_SCRATCH_BYTES per GPU instead, which the library holds from the
 * first call on that GPU until the process ends (on that first call the
 * buffer is zero-filled by a kernel on `stream`; no memset).  The call makes
 * no hipMalloc/hipFree and no allocating library call.  Shapes whose
 * qsa_decode_step_workspace_bytes exceeds the buffer (more than 168 rows of
 * batch x tq, at any budget) are rejected with QSA_ERR_WORKSPACE before
 * anything runs.  All
 * calls on one GPU share its buffer, which keeps the last call's contents:
 * calls that overlap on one GPU (other streams or threads) race and must be
 * serialised by the caller.
 */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)
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
                                     const uint16_t* gate, int64_t gate_seq_stride, hipStream_t stream);

/* qsa_decode_step on a paged cache: the new rows go to their pages, the block
 * keys and the K / V rows are read through the block table
 * (workspace: qsa_decode_step_workspace_bytes).  cache->k_idx may be NULL
 * (then k_idx_new must be NULL and no block key is written). */
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
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gated DeltaNet token mixer of the hybrid layers (Qwen3.8-Flash-Next blog,
 * section "Attention: GDN + QSA": three of every four layers compress the
 * history into a fixed-size state; model card, "Model Overview": 48 V heads,
 * 16 Q/K heads, head dim 128).  The rule is the Gated DeltaNet paper's gated
 * delta rule; per V head h, on Q/K head h / 3, with the state S (128 x 128,
 * rows indexed by key dims):
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 * q and k L2-normalised per head, q then scaled by 1/sqrt(128).  Layouts
 * (bf16 as uint16_t bits, device memory, 16-byte aligned):
 *   q, k  [B][T][16][128]  (sequence stride qk_seq_stride)
 *   v     [B][T][48][128]  (v_seq_stride),  out like v (out_seq_stride)
 *   g, beta float32 [B][T][48] (gate_seq_stride): log decay (<= 0) and
 *         writing strength per V head and token
 *   state float32 [B][48][128][128], read as S_0 and overwritten with S_T.
 * qsa_gdn_prefill takes T tokens per sequence in chunks of 64 (the recurrence
 * rewritten chunk-parallel: bf16 matrix-core products, fp32 accumulation, an
 * fp32 inverse of each chunk's triangular system, the state in fp32); its
 * workspace (qsa_gdn_prefill_workspace_bytes, 256-byte aligned: the operands
 * of up to 512 chunks per sequence, twice over when T spans more than 512
 * chunks) needs no initialisation, and a workspace sized for T serves any
 * shorter call.  qsa_gdn_decode takes one token per sequence with fixed
 * contiguous layouts q, k [B][16][128], v and out [B][48][128], g and beta
 * [B][48], and applies the recurrence directly in fp32.
 */
size_t       qsa_gdn_prefill_workspace_bytes(int32_t batch, int32_t n_tokens);
qsa_status_t qsa_gdn_prefill(const uint16_t* q, const uint16_t* k, int64_t qk_seq_stride,
                             const uint16_t* v, int64_t v_seq_stride,
                             const float* g, const float* beta, int64_t gate_seq_stride,
                             float* state, int32_t batch, int32_t n_tokens,
                             uint16_t* out, int64_t out_seq_stride,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
qsa_status_t qsa_gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, float* state, int32_t batch,
                            uint16_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
