// Block scores of the MQA indexer on the matrix cores, shared by every kernel
// that scores blocks so that all of them produce the same bits.
//
// The head sum is taken on the query side: for each dim d the 4 heads'
// values are added in float32, ((q0 + q1) + q2) + q3 (exact unless their
// exponents are very far apart), and the sum is split exactly into three
// bf16 terms hi + mid + lo.  The score is then
//   s[t][j] = sum over 3 terms x 128 dims of term[t][d] * kbar[j][d],
// 384 exact bf16 products accumulated in float32 by one chain of 12
// v_mfma_f32_16x16x32_bf16 (k-slices of 32 dims, term-major), with no
// per-head partial sums.
//   A (16 x 32): rows are 16 consecutive blocks; k-slice ks uses kbar dims
//                32 (ks % 4) ..  + 31 (the same slice for every term);
//   B (32 x 16): columns are 16 query tokens;
//   D (16 x 16): lane l holds blocks 4*(l/16) .. 4*(l/16) + 3 for token l%16,
//                i.e. 4 consecutive scores of one row (a float4 store).
#pragma once

#include "qsa_internal.h"

namespace qsa {

constexpr int kIdxSlices = 12;   // k-slices: 3 terms x 4 groups of 32 dims

// kf[q]: this lane's 8 dims of kbar slice q (dims 32q + 8*(lane/16) ..) of its
// block row; qf[ks]: its token's 8 dims of k-slice ks (term ks/4, dims
// 32*(ks%4) + 8*(lane/16) ..).
__device__ __forceinline__ f32x4_t block_scores(const bf16x8_t (&kf)[4], const bf16x8_t (&qf)[kIdxSlices]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kIdxSlices; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks & 3], qf[ks], acc, 0, 0, 0);
    return acc;
}

// The same scores for 4 tiles at once: the tiles' chains interleaved
// slice by slice, so consecutive MFMAs never wait on each other's result
// (each tile still accumulates in block_scores' order: the same bits).
__device__ __forceinline__ void block_scores4(const bf16x8_t (&kf)[4][4], const bf16x8_t (&qf)[kIdxSlices],
                                              f32x4_t (&acc)[4]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kIdxSlices; ++ks)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[nt][ks & 3], qf[ks], acc[nt], 0, 0, 0);
}

// B operand for the 16 tokens t0 .. t0 + 15 of one sequence's q_idx
// [T][4][128] (512 contiguous values per token): lane column l%16 is token
// t0 + l%16, whose 4 heads are summed and split into the three terms;
// tokens at or past n_tok (>= 1) are zero columns.  All 16 loads of a lane
// are issued before any is used (columns past n_tok read row n_tok - 1 and
// are zeroed afterwards), so the set-up costs one memory round trip.
__device__ __forceinline__ void load_index_q(const uint16_t* qb, int t0, int n_tok, bf16x8_t (&qf)[kIdxSlices]) {
    const int lane = threadIdx.x & 63;
    const int tok = t0 + (lane & 15);
    const bool ok = tok < n_tok;
    const uint16_t* qr = qb + static_cast<int64_t>(min(tok, n_tok - 1)) * (kHi * kDi) + 8 * (lane >> 4);
    uint4 raw[4][kHi];
#pragma unroll
    for (int dq = 0; dq < 4; ++dq)
#pragma unroll
        for (int hh = 0; hh < kHi; ++hh) raw[dq][hh] = *reinterpret_cast<const uint4*>(qr + hh * kDi + 32 * dq);
#pragma unroll
    for (int dq = 0; dq < 4; ++dq) {
        uint16_t h[kHi][8];
#pragma unroll
        for (int hh = 0; hh < kHi; ++hh)
            *reinterpret_cast<uint4*>(h[hh]) = ok ? raw[dq][hh] : make_uint4(0u, 0u, 0u, 0u);
        uint16_t t_hi[8], t_mid[8], t_lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
            const float s = ((bf16_to_f32(h[0][e]) + bf16_to_f32(h[1][e])) + bf16_to_f32(h[2][e])) + bf16_to_f32(h[3][e]);
            t_hi[e] = f32_to_bf16(s);
            const float r1 = s - bf16_to_f32(t_hi[e]);
            t_mid[e] = f32_to_bf16(r1);
            t_lo[e] = f32_to_bf16(r1 - bf16_to_f32(t_mid[e]));
        }
        qf[dq] = *reinterpret_cast<const bf16x8_t*>(t_hi);
        qf[4 + dq] = *reinterpret_cast<const bf16x8_t*>(t_mid);
        qf[8 + dq] = *reinterpret_cast<const bf16x8_t*>(t_lo);
    }
}

// This lane's part of an A operand row from global memory: its 8 dims of each
// slice of block j.
__device__ __forceinline__ void load_index_k_row(const uint16_t* kb, int j, bf16x8_t (&kf)[4]) {
    const int lane = threadIdx.x & 63;
    const uint16_t* kr = kb + static_cast<int64_t>(j) * kDi + 8 * (lane >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) kf[q] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * q);
}

// A operand from global memory: lane row l%16 is block j0 + l%16; blocks at
// or past j_end (>= 1) read block j_end - 1 instead, so every load is issued
// unconditionally; their scores land only where the result is unspecified.
__device__ __forceinline__ void load_index_k(const uint16_t* kb, int j0, int j_end, bf16x8_t (&kf)[4]) {
    load_index_k_row(kb, min(j0 + static_cast<int>(threadIdx.x & 15), j_end - 1), kf);
}

// The same tile from a paged block-key pool: j0 is a multiple of 16 and a
// page holds a multiple of 16 blocks, so the tile's rows (clamped ones fall in
// the tile of j_end - 1) share one page, read once per wave (scalar load).
__device__ __forceinline__ void load_index_k_paged(const uint16_t* pool, const PageMap& pm, int b, int j0,
                                                   int j_end, bf16x8_t (&kf)[4]) {
    const int jr = min(j0, j_end - 1);
    const int pg = page_of(pm, b, static_cast<int64_t>(jr) * kBlock);
    const int j = min(j0 + static_cast<int>(threadIdx.x & 15), j_end - 1);
    const int64_t row = (static_cast<int64_t>(pg) << (pm.shift - 2)) | (j & ((1 << (pm.shift - 2)) - 1));
    load_index_k_row(pool + row * kDi, 0, kf);
}

}  // namespace qsa
