// Block scores of the MQA indexer on the matrix cores, shared by every kernel
// that scores blocks so that all of them produce the same bits.
//
// The head sum is folded into the contraction: with K = 4 heads x 128 dims,
//   s[t][j] = sum_{k<512} q_idx[t][k] * kbar'[j][k],  kbar'[j][h*128 + d] = kbar[j][d],
// so one chain of 16 v_mfma_f32_16x16x32_bf16 (k-slices of 32 in increasing k,
// i.e. head-major) yields finished scores: 512 exact bf16 products summed in
// float32, no per-head partial sums.
//   A (16 x 32): rows are 16 consecutive blocks; the k-slice of head h and
//                dims 32q .. 32q + 31 is the same kbar slice q for every h;
//   B (32 x 16): columns are 16 query tokens;
//   D (16 x 16): lane l holds blocks 4*(l/16) .. 4*(l/16) + 3 for token l%16,
//                i.e. 4 consecutive scores of one row (a float4 store).
#pragma once

#include "qsa_internal.h"

namespace qsa {

// kf[q]: this lane's 8 dims of kbar slice q (dims 32q + 8*(lane/16) ..) of its
// block row; qf[ks]: its token's 8 dims of k-slice ks (head ks/4, dims
// 32*(ks%4) + 8*(lane/16) ..).
__device__ __forceinline__ f32x4_t block_scores(const bf16x8_t (&kf)[4], const bf16x8_t (&qf)[16]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks & 3], qf[ks], acc, 0, 0, 0);
    return acc;
}

// B operand for the 16 tokens t0 .. t0 + 15 of one sequence's q_idx
// [T][4][128] (512 contiguous values per token): lane column l%16 is token
// t0 + l%16; tokens at or past n_tok are zero columns.
__device__ __forceinline__ void load_index_q(const uint16_t* qb, int t0, int n_tok, bf16x8_t (&qf)[16]) {
    const int lane = threadIdx.x & 63;
    const int tok = t0 + (lane & 15);
    const uint16_t* qr = qb + static_cast<int64_t>(tok) * (kHi * kDi) + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
        if (tok < n_tok) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks);
        else qf[ks] = bf16x8_t{};
    }
}

// A operand from global memory: lane row l%16 is block j0 + l%16; blocks at
// or past j_end (>= 1) read block j_end - 1 instead, so every load is issued
// unconditionally; their scores land only where the result is unspecified.
__device__ __forceinline__ void load_index_k(const uint16_t* kb, int j0, int j_end, bf16x8_t (&kf)[4]) {
    const int lane = threadIdx.x & 63;
    const int j = min(j0 + (lane & 15), j_end - 1);
    const uint16_t* kr = kb + static_cast<int64_t>(j) * kDi + 8 * (lane >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) kf[q] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * q);
}

}  // namespace qsa
