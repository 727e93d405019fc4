// Writes into paged caches (block table; Qwen3.8-Flash-Next blog, section
// "Attention: GDN + QSA": online serving with high prefix-cache reuse, where
// sequences share the pages of a common prefix).  Two launches append the new
// tokens of a prefill chunk: paged_rows_kernel rotates each K row into its
// page (step 0), copies the V and indexer-key rows; paged_compress_kernel then
// writes the key of every block those rows complete (step 1), reading the
// block's 4 indexer-key rows back from their page, exactly as
// compress_kernel does on a contiguous cache.
#include "compress_common.h"
#include "rope_common.h"

namespace qsa {

struct PagedRowsArgs {
    const uint16_t* k_new;      // [B][T][2][256] unrotated (nullable)
    const uint16_t* v_new;      // [B][T][2][256] (nullable)
    int64_t kvns;               // sequence stride of k_new / v_new
    const uint16_t* k_idx_new;  // [B][T][128] (nullable)
    int64_t kins;
    uint16_t* k;                // pools
    uint16_t* v;
    uint16_t* k_idx;
};

// One wave per new token row (4 rows per workgroup).
__global__ __launch_bounds__(256) void paged_rows_kernel(PagedRowsArgs a, PageMap pm, Positions pos0, int n_tokens,
                                                         int64_t rows, InvFreq inv) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                            // whole wave
    const int lane = threadIdx.x & 63;
    const int b = static_cast<int>(row / n_tokens);
    const int i = static_cast<int>(row % n_tokens);
    const int x = pos0.p[b] + i;
    const int64_t dst = phys_token(pm, b, x);
    if (a.k_new != nullptr)
        rope_row_wave(a.k_new + b * a.kvns + static_cast<int64_t>(i) * (kHkv * kD), a.k + dst * (kHkv * kD), kHkv,
                      static_cast<double>(x), inv, false);
    if (a.v_new != nullptr)                             // 2 x 256 values: 16 B per lane
        *reinterpret_cast<uint4*>(a.v + dst * (kHkv * kD) + 8 * lane) =
            *reinterpret_cast<const uint4*>(a.v_new + b * a.kvns + static_cast<int64_t>(i) * (kHkv * kD) + 8 * lane);
    if (a.k_idx_new != nullptr && lane < kDi / 8)
        *reinterpret_cast<uint4*>(a.k_idx + dst * kDi + 8 * lane) =
            *reinterpret_cast<const uint4*>(a.k_idx_new + b * a.kins + static_cast<int64_t>(i) * kDi + 8 * lane);
}

// One 16-lane group per (sequence, block) of blocks [j0[b], j0[b] + n[b]):
// lane c handles dims 8c .. 8c + 7.
__global__ __launch_bounds__(256) void paged_compress_kernel(const uint16_t* __restrict__ k_idx,
                                                             uint16_t* __restrict__ kbar, PageMap pm,
                                                             Positions j0, Positions nblk, int max_blocks,
                                                             int64_t items) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
    if (item >= items) return;
    const int b = static_cast<int>(item / max_blocks);
    const int jj = static_cast<int>(item % max_blocks);
    if (jj >= nblk.p[b]) return;
    const int c = threadIdx.x & 15;
    const int j = j0.p[b] + jj;
    uint4 r[kBlock];
#pragma unroll
    for (int t = 0; t < kBlock; ++t)
        r[t] = *reinterpret_cast<const uint4*>(k_idx + phys_token(pm, b, static_cast<int64_t>(kBlock) * j + t) * kDi +
                                               8 * c);
    *reinterpret_cast<uint4*>(kbar + phys_block(pm, b, j) * kDi + 8 * c) = compress_rows(r);
}

hipError_t launch_paged_append(const PageMap& pm, uint16_t* k, uint16_t* v, uint16_t* k_idx, uint16_t* kbar,
                               const uint16_t* k_new, const uint16_t* v_new, int64_t kvns,
                               const uint16_t* k_idx_new, int64_t kins, const Positions& pos0, int batch,
                               int n_tokens, const qsa_rope_t& rope, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * n_tokens;
    if (rows == 0) return hipSuccess;
    PagedRowsArgs a{k_new, v_new, kvns, k_idx_new, kins, k, v, k_idx};
    if (k_new != nullptr || v_new != nullptr || k_idx_new != nullptr) {
        hipLaunchKernelGGL(paged_rows_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, a,
                           pm, pos0, n_tokens, rows, make_inv_freq(rope));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (kbar == nullptr) return hipSuccess;
    // blocks j with 4j + 3 in [pos0, pos0 + n_tokens)
    Positions j0{}, nb{};
    int max_blocks = 0;
    for (int b = 0; b < batch; ++b) {
        j0.p[b] = pos0.p[b] / kBlock;
        nb.p[b] = (pos0.p[b] + n_tokens) / kBlock - j0.p[b];
        max_blocks = max(max_blocks, nb.p[b]);
    }
    if (max_blocks == 0) return hipSuccess;
    const int64_t items = static_cast<int64_t>(batch) * max_blocks;
    hipLaunchKernelGGL(paged_compress_kernel, dim3(static_cast<unsigned>((items + 15) / 16)), dim3(256), 0, stream,
                       k_idx, kbar, pm, j0, nb, max_blocks, items);
    return hipGetLastError();
}

}  // namespace qsa
