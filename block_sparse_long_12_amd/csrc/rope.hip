// Step 0: rotary embedding of Q / K rows (Qwen3.8-Flash-Next model card,
// "Processing Ultra-Long Texts", rope_parameters: rope_theta 1e7,
// partial_rotary_factor 0.25 -> 64 of 256 dims; for text the interleaved
// mRoPE sections [11, 11, 10] all carry the same position, which is plain
// 1-D rotary over 32 frequencies).
//
// HBM-bound single pass.  One wave per token row: lanes 0..31 evaluate the
// 32 angles and their sines/cosines in float64 once per row, every lane then
// owns 4 consecutive dims (8 bytes) of each head, so a head row of 512 bytes
// is one coalesced wave access.  Pair (d, d+32) lives in lanes (d/4, d/4+8);
// partners are exchanged with a lane xor of 8.
#include "qsa_internal.h"

namespace qsa {

struct InvFreq {
    double f[kRot / 2];
};

__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* x, int64_t xs,
                                                   int64_t xt, uint16_t* y, int64_t ys, int64_t yt,
                                                   int batch, int n_tokens, int n_heads,
                                                   Positions pos0, InvFreq inv, bool in_place) {
#pragma clang fp contract(off)
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= static_cast<int64_t>(batch) * n_tokens) return;   // wave-uniform
    const int b = static_cast<int>(row / n_tokens);
    const int i = static_cast<int>(row % n_tokens);
    const double p = static_cast<double>(pos0.p[b] + i);

    double sn = 0.0, cs = 1.0;
    if (lane < kRot / 2) sincos(p * inv.f[lane], &sn, &cs);
    // lane L (< 16) rotates the pairs d = 4 * (L & 7) + e, e < 4
    double c4[4], s4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int src = 4 * (lane & 7) + e;
        c4[e] = __shfl(cs, src);
        s4[e] = __shfl(sn, src);
    }

    const uint16_t* xr = x + b * xs + i * xt;
    uint16_t* yr = y + b * ys + i * yt;
    for (int h = 0; h < n_heads; ++h) {
        const uint2 v = *reinterpret_cast<const uint2*>(xr + h * kD + lane * 4);
        const uint32_t px = __shfl_xor(v.x, 8);
        const uint32_t py = __shfl_xor(v.y, 8);
        uint2 o = v;
        if (lane < 16) {
            const uint32_t own[2] = {v.x, v.y};
            const uint32_t oth[2] = {px, py};
            uint32_t res[2];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                uint32_t packed = 0;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int e = 2 * w + half;
                    const double mine = bf16_to_f32(static_cast<uint16_t>(own[w] >> (16 * half)));
                    const double other = bf16_to_f32(static_cast<uint16_t>(oth[w] >> (16 * half)));
                    double r;
                    if (lane < 8) {          // first half of the pair: a cos - c sin
                        const double t1 = mine * c4[e];
                        const double t2 = other * s4[e];
                        r = t1 - t2;
                    } else {                 // second half: c cos + a sin
                        const double t1 = mine * c4[e];
                        const double t2 = other * s4[e];
                        r = t1 + t2;
                    }
                    packed |= static_cast<uint32_t>(f64_to_bf16(r)) << (16 * half);
                }
                res[w] = packed;
            }
            o.x = res[0];
            o.y = res[1];
        }
        if (!in_place || lane < 16) *reinterpret_cast<uint2*>(yr + h * kD + lane * 4) = o;
    }
}

hipError_t launch_rope(const uint16_t* x, int64_t xs, int64_t xt, uint16_t* y, int64_t ys,
                       int64_t yt, int batch, int n_tokens, int n_heads, const Positions& pos0,
                       double theta, bool in_place, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * n_tokens;
    if (rows == 0) return hipSuccess;
    InvFreq inv;
    for (int d = 0; d < kRot / 2; ++d) inv.f[d] = pow(theta, -static_cast<double>(d) / (kRot / 2));
    const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
    hipLaunchKernelGGL(rope_kernel, dim3(grid), dim3(256), 0, stream, x, xs, xt, y, ys, yt, batch,
                       n_tokens, n_heads, pos0, inv, in_place);
    return hipGetLastError();
}

}  // namespace qsa
