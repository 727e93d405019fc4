// Block-key arithmetic of step 1, shared by every kernel that compresses a
// block so that all of them produce the same bits (Qwen3.8-Flash-Next blog,
// "Attention: GDN + QSA": the indexer aggregates the sequence into
// micro-blocks; model card: 512 blocks = 2048 tokens, so 4 tokens per block).
// The block key is the mean of the block's 4 indexer keys: float32 sum in
// token order, ((k0 + k1) + k2) + k3, times 0.25, rounded to bf16 (nearest,
// ties to even).
#pragma once

#include "qsa_internal.h"

namespace qsa {

// 8 dims of one block: r[t] holds dims 8c .. 8c + 7 of token row t of the
// block (one 16-byte load per row); returns the same 8 dims of the key.
__device__ __forceinline__ uint4 compress_rows(const uint4 (&r)[kBlock]) {
#pragma clang fp contract(off)
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t packed = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int sh = 16 * half;
            const uint32_t w0 = (&r[0].x)[w], w1 = (&r[1].x)[w], w2 = (&r[2].x)[w], w3 = (&r[3].x)[w];
            float s = bf16_to_f32(static_cast<uint16_t>(w0 >> sh));
            s = s + bf16_to_f32(static_cast<uint16_t>(w1 >> sh));
            s = s + bf16_to_f32(static_cast<uint16_t>(w2 >> sh));
            s = s + bf16_to_f32(static_cast<uint16_t>(w3 >> sh));
            s = s * 0.25f;
            packed |= static_cast<uint32_t>(f32_to_bf16(s)) << sh;
        }
        out[w] = packed;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace qsa
