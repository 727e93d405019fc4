// Step 3: per-token block selection -- one workgroup per query row running
// the exact radix select of select_common.h on the row's float32 scores.
#include "select_common.h"

namespace qsa {

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ scores, int64_t ld,
                                                    int64_t ss, Positions pos0, int tq, int budget,
                                                    int32_t* __restrict__ sel, int64_t sels) {
    __shared__ SelectSmem sm;
    const int b = blockIdx.x / tq;
    const int i = blockIdx.x % tq;
    const int p = pos0.p[b] + i;
    const int o = p / kBlock;
    const int keep = min(budget - 1, o);
    select_row<NT>(scores + b * ss + static_cast<int64_t>(i) * ld, o, keep, budget,
                   sel + b * sels + static_cast<int64_t>(i) * budget, sm);
}

hipError_t launch_select(const float* scores, int64_t ld, int64_t ss, const Positions& pos0,
                         int batch, int tq, int budget, int32_t* sel, int64_t sels,
                         hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * tq;
    if (rows == 0) return hipSuccess;
    if (rows < 1024) {
        hipLaunchKernelGGL(select_kernel<1024>, dim3(static_cast<unsigned>(rows)), dim3(1024), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels);
    } else {
        hipLaunchKernelGGL(select_kernel<256>, dim3(static_cast<unsigned>(rows)), dim3(256), 0,
                           stream, scores, ld, ss, pos0, tq, budget, sel, sels);
    }
    return hipGetLastError();
}

}  // namespace qsa
