// Rotary embedding of one token row (Qwen3.8-Flash-Next model card,
// "Processing Ultra-Long Texts": rope_theta 1e7, partial_rotary_factor 0.25;
// text positions make the interleaved mRoPE plain 1-D rotary): pair
// (d, d+32), d < 32, of each head is turned by p * theta^(-d/32), or by the
// static-YaRN rates with cos and sin scaled (make_inv_freq).  Shared by
// the rotary kernel and the kernels that rotate rows on the fly, so every
// path produces the same bits: angles, sines and the rotation in float64,
// one rounding to bf16.
#pragma once

#include "qsa_internal.h"

namespace qsa {

struct InvFreq {
    double f[kRot / 2];      // per-pair angle rate, computed on the host with libm
    double m;                // factor on cos and sin (1 for plain rotary)
};

// Plain rotary: f[d] = theta^(-d/32), m = 1.  Static YaRN (yarn_factor s > 1;
// YaRN paper, Peng et al. 2023: NTK-by-parts interpolation and the attention
// temperature; one table for every length): pair d turns
// L * theta^(-d/32) / (2 pi) times over the original context L; the pair index
// where that count is rho is 32 ln(L / (2 pi rho)) / ln theta.  Pairs up to
// floor of that index at rho = 32 keep their rate, pairs from its ceiling at
// rho = 1 (at most 63) run s times slower, pairs between blend linearly in d;
// cos and sin are scaled by 1 + 0.1 ln s.
inline InvFreq make_inv_freq(const qsa_rope_t& r) {
    InvFreq inv;
    inv.m = 1.0;
    for (int d = 0; d < kRot / 2; ++d) inv.f[d] = pow(r.theta, -static_cast<double>(d) / (kRot / 2));
    if (r.yarn_factor > 1.0) {
        const double s = r.yarn_factor;
        const double L = static_cast<double>(r.yarn_original_max);
        const double two_pi = 6.283185307179586;
        auto pair_at = [&](double rho) { return (kRot / 2) * log(L / (two_pi * rho)) / log(r.theta); };
        const double lo = fmax(floor(pair_at(32.0)), 0.0);
        double hi = fmin(ceil(pair_at(1.0)), kRot - 1.0);
        if (lo == hi) hi += 0.001;
        for (int d = 0; d < kRot / 2; ++d) {
            const double g = fmin(fmax((d - lo) / (hi - lo), 0.0), 1.0);
            inv.f[d] = (inv.f[d] / s) * g + inv.f[d] * (1.0 - g);
        }
        inv.m = 0.1 * log(s) + 1.0;
    }
    return inv;
}

// (a, c) -> (a cos - c sin, c cos + a sin) for the first half of a pair
// (first = true, mine = a, other = c) or the second half (mine = c, other = a).
__device__ __forceinline__ uint16_t rotate_half_elem(double mine, double other, double cs, double sn,
                                                     bool first) {
#pragma clang fp contract(off)
    const double t1 = mine * cs;
    const double t2 = other * sn;
    return f64_to_bf16(first ? (t1 - t2) : (t1 + t2));
}

// One wave rotates one token row of n_heads heads: lane L owns dims 4L..4L+3
// of every head (one 512-byte access per head); lanes 0..31 evaluate the 32
// angles.  Every lane of the wave must call it.
__device__ __forceinline__ void rope_row_wave(const uint16_t* xr, uint16_t* yr, int n_heads, double p,
                                              const InvFreq& inv, bool in_place) {
    const int lane = threadIdx.x & 63;
    double sn = 0.0, cs = 1.0;
    if (lane < kRot / 2) {
        sincos(p * inv.f[lane], &sn, &cs);
        sn *= inv.m;
        cs *= inv.m;
    }
    double c4[4], s4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int src = 4 * (lane & 7) + e;
        c4[e] = __shfl(cs, src);
        s4[e] = __shfl(sn, src);
    }
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
                    packed |= static_cast<uint32_t>(rotate_half_elem(mine, other, c4[e], s4[e], lane < 8))
                              << (16 * half);
                }
                res[w] = packed;
            }
            o.x = res[0];
            o.y = res[1];
        }
        if (!in_place || lane < 16) *reinterpret_cast<uint2*>(yr + h * kD + lane * 4) = o;
    }
}

}  // namespace qsa
