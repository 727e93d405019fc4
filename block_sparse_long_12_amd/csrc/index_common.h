// Block score of the MQA indexer on the matrix cores, shared by every kernel
// that scores blocks so that all of them produce the same bits.
//
// v_mfma_f32_16x16x32_bf16, A rows = 4 tokens x 4 indexer heads (row
// 4*token + head), B columns = 16 blocks.  The accumulator of lane l holds rows
// 4*(l/16) + r, r < 4, i.e. the 4 heads of one token for one block, so the
// head sum ((h0 + h1) + h2) + h3 is an in-lane add.  Products of bf16 pairs are
// exact in float32 and the 4 k-steps (32 dims each) accumulate in float32.
#pragma once

#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ float block_score(const bf16x8_t (&a)[4], const bf16x8_t (&b)[4]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b[ks], acc, 0, 0, 0);
    return ((acc[0] + acc[1]) + acc[2]) + acc[3];
}

// A operand for 4 tokens starting at row `tok0` of one sequence's q_idx
// [T][4][128]: lane row c16 = 4 * (token) + head, k slice 8 * (lane / 16).
__device__ __forceinline__ void load_index_a(const uint16_t* qb, int tok0, int n_tok, bf16x8_t (&a)[4]) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int tok = tok0 + (c16 >> 2);
    const uint16_t* qr = qb + (static_cast<int64_t>(tok) * kHi + (c16 & 3)) * kDi + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (tok < n_tok) a[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks);
        else a[ks] = bf16x8_t{};
    }
}

// B operand of column tile n for the 64 blocks starting at j0: lane column
// c16 is block j0 + 4 * c16 + n.  Columns at or past j_end (>= 1) read block
// j_end - 1 instead, so every load is issued unconditionally (the loop stays
// branch-free and the next step's loads can stay in flight); their scores
// land only where the result is unspecified and are never used.
__device__ __forceinline__ void load_index_b(const uint16_t* kb, int j0, int n, int j_end, bf16x8_t (&b)[4]) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int j = min(j0 + 4 * c16 + n, j_end - 1);
    const uint16_t* kr = kb + static_cast<int64_t>(j) * kDi + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b[ks] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * ks);
}

}  // namespace qsa
