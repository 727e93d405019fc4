// Step 1: micro-block key compression over a range of blocks (the arithmetic
// is compress_rows in compress_common.h).
//
// HBM-bound: reads 1 KiB and writes 256 B per block.  16 lanes per block,
// each lane owns 8 dims (one 16-byte load per token row, one 16-byte store).
#include "compress_common.h"

namespace qsa {

__global__ __launch_bounds__(256) void compress_kernel(const uint16_t* __restrict__ k, int64_t ks,
                                                       int batch, int block_begin, int n_blocks,
                                                       uint16_t* __restrict__ kbar, int64_t kbs) {
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
    *reinterpret_cast<uint4*>(kbar + b * kbs + j * kDi + c * 8) = compress_rows(r);
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
