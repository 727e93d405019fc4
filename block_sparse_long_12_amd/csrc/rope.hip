// Step 0: rotary embedding of Q / K rows, one wave per token row
// (rope_common.h holds the row rotation and its sources).  HBM-bound single
// pass: 512 bytes read and written per head row.
#include "rope_common.h"

namespace qsa {

__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* x, int64_t xs, int64_t xt,
                                                   uint16_t* y, int64_t ys, int64_t yt, int batch,
                                                   int n_tokens, int n_heads, Positions pos0,
                                                   InvFreq inv, bool in_place) {
    const int wave = threadIdx.x >> 6;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= static_cast<int64_t>(batch) * n_tokens) return;   // wave-uniform
    const int b = static_cast<int>(row / n_tokens);
    const int i = static_cast<int>(row % n_tokens);
    rope_row_wave(x + b * xs + i * xt, y + b * ys + i * yt, n_heads,
                  static_cast<double>(pos0.p[b] + i), inv, in_place);
}

hipError_t launch_rope(const uint16_t* x, int64_t xs, int64_t xt, uint16_t* y, int64_t ys,
                       int64_t yt, int batch, int n_tokens, int n_heads, const Positions& pos0,
                       const qsa_rope_t& rope, bool in_place, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * n_tokens;
    if (rows == 0) return hipSuccess;
    const InvFreq inv = make_inv_freq(rope);
    const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
    hipLaunchKernelGGL(rope_kernel, dim3(grid), dim3(256), 0, stream, x, xs, xt, y, ys, yt, batch,
                       n_tokens, n_heads, pos0, inv, in_place);
    return hipGetLastError();
}

}  // namespace qsa
