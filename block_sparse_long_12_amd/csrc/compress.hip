// Step 1: micro-block key compression (Qwen3.8-Flash-Next blog, "Attention:
// GDN + QSA": the indexer aggregates the sequence into micro-blocks; model
// card: 512 blocks = 2048 tokens, so 4 tokens per block).  The block key is
// the mean of the block's 4 indexer keys: float32 sum in token order, times
// 0.25, rounded to bf16 (nearest, ties to even).
//
// HBM-bound: reads 1 KiB and writes 256 B per block.  16 lanes per block,
// each lane owns 8 dims (one 16-byte load per token row, one 16-byte store).
#include "qsa_internal.h"

namespace qsa {

__global__ __launch_bounds__(256) void compress_kernel(const uint16_t* __restrict__ k, int64_t ks,
                                                       int batch, int block_begin, int n_blocks,
                                                       uint16_t* __restrict__ kbar, int64_t kbs) {
#pragma clang fp contract(off)
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= static_cast<int64_t>(batch) * n_blocks * 16) return;
    const int c = static_cast<int>(gid & 15);
    const int64_t bj = gid >> 4;
    const int b = static_cast<int>(bj / n_blocks);
    const int64_t j = block_begin + bj % n_blocks;
    const uint16_t* src = k + b * ks + j * (kBlock * kDi) + c * 8;
    uint4 r[kBlock];
#pragma unroll
    for (int t = 0; t < kBlock; ++t) r[t] = *reinterpret_cast<const uint4*>(src + t * kDi);
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
    *reinterpret_cast<uint4*>(kbar + b * kbs + j * kDi + c * 8) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_compress(const uint16_t* k_idx, int64_t ks, int batch, int block_begin,
                           int block_end, uint16_t* kbar, int64_t kbs, hipStream_t stream) {
    const int n_blocks = block_end - block_begin;
    if (n_blocks <= 0) return hipSuccess;
    const int64_t threads = static_cast<int64_t>(batch) * n_blocks * 16;
    const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
    hipLaunchKernelGGL(compress_kernel, dim3(grid), dim3(256), 0, stream, k_idx, ks, batch,
                       block_begin, n_blocks, kbar, kbs);
    return hipGetLastError();
}

}  // namespace qsa
