// Step 4: grouped-query attention over the selected micro-blocks
// (Qwen3.8-Flash-Next model card, "Model Overview": 24 query heads, 2 KV
// heads, head dim 256; blog "Attention: GDN + QSA": attention runs over the
// selected regions; "QSA's Attention Kernel" covers prefill and decode).
//
// For query position p, KV head g and each of its 12 query heads h:
//   out[h] = sum_n softmax_n(scale * q[h] . k[n][g]) v[n][g]
// over the tokens n = 4j + e of the selected blocks j, with n <= p.
//
// One wave per (query, KV head).  The wave walks the selected blocks 4 at a
// time (16 tokens):
//   - each lane gathers one token row of K and of V (lane & 15 = token slot,
//     lane >> 4 = which 16-byte slice), 8 KiB + 8 KiB per step per wave, as
//     whole 512-byte rows of the token-major cache; the next step's rows are
//     requested before the current step is computed.  Slots that hold no
//     token (padding, or past the query in its own block) read the query's
//     own row instead and are masked out of the softmax, so no load is ever
//     predicated or zero-filled;
//   - S^T (16 tokens x 16 head slots, 12 real) = K Q^T on
//     v_mfma_f32_16x16x32_bf16 with Q^T held in registers;
//   - online softmax in float32 (exp2, scale folded into log2 e).  Each lane
//     owns one head for all its accumulators.  The reference maximum of a head
//     is only raised when a logit exceeds it by more than 8 in exp2 units, so
//     the accumulators are rescaled once or twice per query instead of every
//     step; the weights stay below 2^8 and the result is the same softmax;
//   - O^T (256 dims x 16 heads) += V^T P^T on v_mfma_f32_16x16x16bf16_1k.
//     The S^T accumulator layout (lane: tokens 4*(l/16)+r of head l%16) is
//     exactly the B-operand layout the PV product needs, so P never moves
//     between lanes; V is transposed through a wave-private LDS tile.
// The gather is the bound (12 flop per gathered byte), not the matrix cores.
#include <math.h>

#include "rope_common.h"

namespace qsa {

constexpr int kVtStride = 20;                 // bf16 per dim row of the V^T tile (16 tokens + pad)
constexpr int kVtElems = kD * kVtStride;      // one wave's tile
constexpr float kRescaleSlack = 8.0f;         // exp2 units a logit may exceed the reference max

struct WaveState {
    float m;            // reference max of raw logits q.k for this lane's head
    float l;            // softmax denominator relative to m
    f32x4_t acc[16];    // O^T rows 16*nt + 4*(lane/16) + r, head lane%16
};

struct Chunk {
    bf16x8_t ka[8];
    bf16x8_t vv[8];
    uint64_t vmask;     // token slots holding a real token
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Paged caches: the sequence's block-table row, the page size and the
// page of the query position (the row that stands in for empty slots).
struct KvPages {
    const int32_t* tbl;
    int shift;
    int n_pages;
    int pp;
};

template <bool kPaged>
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                                           const int32_t* __restrict__ selrow, int cb, int blk_end, int p,
                                           const KvPages& kp, Chunk& ch) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    // the chunk's 4 selection entries through wave-uniform (scalar) loads, so
    // waiting for them never waits on the K/V gathers still in flight
    const int cbu = __builtin_amdgcn_readfirstlane(cb);
    const int endu = __builtin_amdgcn_readfirstlane(blk_end);
    const int s0 = selrow[min(cbu + 0, endu - 1)];
    const int s1 = selrow[min(cbu + 1, endu - 1)];
    const int s2 = selrow[min(cbu + 2, endu - 1)];
    const int s3 = selrow[min(cbu + 3, endu - 1)];
    const int q4 = c16 >> 2;
    const int slot_blk = cb + q4;
    const int jl = (q4 == 0) ? s0 : (q4 == 1) ? s1 : (q4 == 2) ? s2 : s3;
    const int j = (slot_blk < blk_end) ? jl : -1;
    const int n = kBlock * j + (c16 & 3);
    const bool valid = (j >= 0) && (j <= p / kBlock) && (n <= p);
    int64_t row = valid ? n : p;
    if constexpr (kPaged) {
        // page of each of the 4 blocks (wave-uniform: scalar loads); a slot
        // that holds no legal block reads the query's own row, in page pp
        auto page = [&](int sb) {
            const int tok = (sb >= 0 && sb <= p / kBlock) ? kBlock * sb : p;
            return min(max(kp.tbl[tok >> kp.shift], 0), kp.n_pages - 1);
        };
        const int g0 = page(s0), g1 = page(s1), g2 = page(s2), g3 = page(s3);
        const int gl = (q4 == 0) ? g0 : (q4 == 1) ? g1 : (q4 == 2) ? g2 : g3;
        row = (static_cast<int64_t>(valid ? gl : kp.pp) << kp.shift) | (row & ((int64_t{1} << kp.shift) - 1));
    }
    const uint16_t* kr = kg + row * (kHkv * kD);
    const uint16_t* vr = vg + row * (kHkv * kD);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        ch.ka[s] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * s + 8 * G);
        ch.vv[s] = *reinterpret_cast<const bf16x8_t*>(vr + 8 * (4 * s + G));
    }
    ch.vmask = __ballot(valid);
}

// A row's selection resolved once into LDS (resolve_selection): for slot i
// the cache row of the block's first token (physical with paged caches) and
// how many of its 4 tokens are attended (0: no legal block; fewer than 4: the
// own block, cut at the query).  Per chunk a lane then needs one LDS read
// instead of a chain of dependent memory loads.
template <bool kPaged>
__device__ __forceinline__ void resolve_selection(const int32_t* __restrict__ selrow, int n, int p,
                                                  const KvPages& kp, int32_t* row, int32_t* nv) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int s = selrow[i];
        const bool legal = s >= 0 && s <= p / kBlock;
        const int tok = legal ? kBlock * s : p;
        int r = tok;
        if constexpr (kPaged) {
            const int pg = min(max(kp.tbl[tok >> kp.shift], 0), kp.n_pages - 1);
            r = (pg << kp.shift) | (tok & ((1 << kp.shift) - 1));
        }
        row[i] = r;
        nv[i] = legal ? min(kBlock, p - kBlock * s + 1) : 0;
    }
}

// The chunk of slots cb .. cb+3 from the resolved selection; row_p is the
// query's own row, read by lanes with nothing to attend.
__device__ __forceinline__ void load_chunk_lds(const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                                               const int32_t* row, const int32_t* nv, int cb, int blk_end,
                                               int row_p, Chunk& ch) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int slot = cb + (c16 >> 2);
    const bool in = slot < blk_end;
    const int rb = row[in ? slot : cb];
    const int cnt = in ? nv[slot] : 0;
    const bool valid = (c16 & 3) < cnt;
    const int64_t r = valid ? rb + (c16 & 3) : row_p;
    const uint16_t* kr = kg + r * (kHkv * kD);
    const uint16_t* vr = vg + r * (kHkv * kD);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        ch.ka[s] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * s + 8 * G);
        ch.vv[s] = *reinterpret_cast<const bf16x8_t*>(vr + 8 * (4 * s + G));
    }
    ch.vmask = __ballot(valid);
}

__device__ __forceinline__ void attend_chunk(const Chunk& ch, const bf16x8_t (&qf)[8], float c,
                                             WaveState& st, uint16_t* vt) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;

    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.ka[ks], qf[ks], s, 0, 0, 0);

    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = (ch.vmask >> (4 * G + r)) & 1ull;
        sv[r] = ok ? s[r] : -INFINITY;
        mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // raise the reference max only when the new logits would exceed it by the slack
    const bool raise = (mx - st.m) * c > kRescaleSlack;     // always true while st.m = -inf
    if (__ballot(raise) != 0ull) {                          // wave-uniform
        const float m_new = raise ? mx : st.m;
        const float alpha = exp2f((st.m - m_new) * c);      // 1 for heads not raised, 0 from -inf
        st.l *= alpha;
        st.m = m_new;
#pragma unroll
        for (int t = 0; t < 16; ++t) st.acc[t] *= alpha;
    }
    s16x4_t pb;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float pr = exp2f((sv[r] - st.m) * c);         // 0 for masked slots
        const uint16_t pbits = f32_to_bf16(pr);
        pb[r] = static_cast<short>(pbits);
        ps += bf16_to_f32(pbits);          // the denominator uses the weights the product sees
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    st.l += ps;

    // V^T tile: vt[dim * kVtStride + token slot]
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&ch.vv[s2]);
        const int d0 = 8 * (4 * s2 + G);
#pragma unroll
        for (int q = 0; q < 8; ++q) vt[(d0 + q) * kVtStride + c16] = e[q];
    }
    wave_lds_sync();
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
        const s16x4_t va = *reinterpret_cast<const s16x4_t*>(vt + (16 * nt + c16) * kVtStride + 4 * G);
        st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.acc[nt], 0, 0, 0);
    }
    wave_lds_sync();
}

// Attend over the slots blk_begin .. blk_end of the selection for the query
// at position p; load(cb, chunk) issues the loads of slots cb .. cb + 3.
// `cur` must hold the loads of the first chunk (issued by the caller, so they
// can overlap the query set-up).  Chunks are processed in statically unrolled
// groups of kUnroll with two named buffers: inside a group the code is
// straight-line, so each wait covers only the chunk about to be used and the
// next chunk's rows stay in flight (a loop-carried pipeline makes the
// compiler drain all loads at every loop head).  Steps past the end re-read
// the last chunk's rows (cache hits) and are skipped.
template <int kUnroll, typename Load>
__device__ __forceinline__ void attend_blocks(Load&& load, int blk_begin, int blk_end, const bf16x8_t (&qf)[8],
                                              float c, WaveState& st, uint16_t* vt, Chunk& cur) {
    const int last = blk_begin + (blk_end - 1 - blk_begin) / 4 * 4;      // first block of the last chunk
    Chunk other;
    for (int cb = blk_begin; cb < blk_end; cb += 4 * kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; u += 2) {
            const int c0 = cb + 4 * u;
            const int c1 = c0 + 4;
            const int c2 = c1 + 4;
            load(min(c1, last), other);
            if (c0 < blk_end && cur.vmask != 0ull) attend_chunk(cur, qf, c, st, vt);
            load(min(c2, last), cur);
            if (c1 < blk_end && other.vmask != 0ull) attend_chunk(other, qf, c, st, vt);
        }
    }
}

// Q^T fragments of this lane's head (lane & 15 < 12), k slices 32*ks + 8*(lane/16).
__device__ __forceinline__ void issue_q_frags(const uint16_t* qh, bool ok, bf16x8_t (&qf)[8]) {
    const int G = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qf[ks] = ok ? *reinterpret_cast<const bf16x8_t*>(qh + 32 * ks + 8 * G) : bf16x8_t{};
}

// Rotary angles of position p: each lane evaluates one of the 32 angles (the
// same call as rope_row_wave); needs no loaded data, so it can run while loads
// are in flight.
struct RopeAngle {
    double sn, cs;
};
__device__ __forceinline__ RopeAngle rope_angle(int p, const InvFreq& inv) {
    RopeAngle a;
    sincos(static_cast<double>(p) * inv.f[threadIdx.x & 31], &a.sn, &a.cs);
    a.sn *= inv.m;
    a.cs *= inv.m;
    return a;
}

// Rotates the loaded fragments: the rotary pairs (d, d + 32), d = 8*(lane/16)
// + e, sit in fragments 0 and 1 of the same lane; each takes the 8 angles its
// k slice needs from its peers, exactly as the rotary kernel rotates, so an
// unrotated q gives the same bits as a pre-rotated one.
__device__ __forceinline__ void rotate_q_frags(const RopeAngle& a, bf16x8_t (&qf)[8]) {
    const int G = (threadIdx.x & 63) >> 4;
    uint16_t* lo = reinterpret_cast<uint16_t*>(&qf[0]);
    uint16_t* hi = reinterpret_cast<uint16_t*>(&qf[1]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double cs = __shfl(a.cs, 8 * G + e);
        const double sn = __shfl(a.sn, 8 * G + e);
        const double x = bf16_to_f32(lo[e]);
        const double y = bf16_to_f32(hi[e]);
        lo[e] = rotate_half_elem(x, y, cs, sn, true);
        hi[e] = rotate_half_elem(y, x, cs, sn, false);
    }
}

// Output gate (blog, "Training stability": the attention output gating
// mechanism is retained): the factor 1 / (1 + exp(-g)) of a bf16 gate logit.
__device__ __forceinline__ float gate_factor(uint16_t g) { return 1.f / (1.f + expf(-bf16_to_f32(g))); }

// The 4 gated output values of one lane (4 consecutive dims), packed as bf16.
__device__ __forceinline__ uint2 pack_out4(float o0, float o1, float o2, float o3, const uint2* g) {
    if (g != nullptr) {
        o0 *= gate_factor(static_cast<uint16_t>(g->x));
        o1 *= gate_factor(static_cast<uint16_t>(g->x >> 16));
        o2 *= gate_factor(static_cast<uint16_t>(g->y));
        o3 *= gate_factor(static_cast<uint16_t>(g->y >> 16));
    }
    uint2 w;
    w.x = f32_to_bf16(o0) | (static_cast<uint32_t>(f32_to_bf16(o1)) << 16);
    w.y = f32_to_bf16(o2) | (static_cast<uint32_t>(f32_to_bf16(o3)) << 16);
    return w;
}

__device__ __forceinline__ void init_state(WaveState& st) {
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------- prefill

// K / V of the sequence, or of the page pool: KV head g's base and the
// sequence's pages
template <bool kPaged>
__device__ __forceinline__ void kv_bases(const uint16_t* k, const uint16_t* v, int64_t kvs, const PageMap& pm,
                                         int b, int g, int p, const uint16_t*& kg, const uint16_t*& vg,
                                         KvPages& kp) {
    if constexpr (kPaged) {
        kg = k + g * kD;
        vg = v + g * kD;
        kp.tbl = pm.table + b * pm.ts;
        kp.shift = pm.shift;
        kp.n_pages = pm.n_pages;
        kp.pp = min(max(kp.tbl[p >> pm.shift], 0), pm.n_pages - 1);
    } else {
        kg = k + b * kvs + g * kD;
        vg = v + b * kvs + g * kD;
        kp = KvPages{};
    }
}

template <bool kPaged>
__global__ __launch_bounds__(128) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs, const int32_t* __restrict__ sel, int64_t sels,
    Positions pos0, int tq, int budget, float scale, float c, uint16_t* __restrict__ out,
    int64_t os, float* __restrict__ lse, int64_t lss, const uint16_t* __restrict__ gate, int64_t gs,
    InvFreq inv, int rope_q, PageMap pm) {
    __shared__ uint16_t vt_all[2 * kVtElems];
    __shared__ int32_t s_row[QSA_MAX_BUDGET];
    __shared__ int32_t s_nv[QSA_MAX_BUDGET];
    const int g = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int b = blockIdx.x / tq;
    const int i = blockIdx.x % tq;
    const int p = pos0.p[b] + i;
    const int head = g * kGroup + c16;
    const bool head_ok = c16 < kGroup;

    const uint16_t *kg, *vg;
    KvPages kp;
    kv_bases<kPaged>(k, v, kvs, pm, b, g, p, kg, vg, kp);
    const int32_t* selrow = sel + b * sels + static_cast<int64_t>(i) * budget;
    bf16x8_t qf[8];
    const uint16_t* qrow = q + b * qs + static_cast<int64_t>(i) * (kHq * kD);
    issue_q_frags(qrow + (head_ok ? head : 0) * kD, head_ok, qf);
    resolve_selection<kPaged>(selrow, budget, p, kp, s_row, s_nv);
    __syncthreads();
    const int row_p = kPaged ? (kp.pp << kp.shift) | (p & ((1 << kp.shift) - 1)) : p;
    auto load = [&](int cb, Chunk& ch) { load_chunk_lds(kg, vg, s_row, s_nv, cb, budget, row_p, ch); };
    Chunk first;
    load(0, first);
    if (rope_q) rotate_q_frags(rope_angle(p, inv), qf);
    WaveState st;
    init_state(st);
    attend_blocks<8>(load, 0, budget, qf, c, st, vt_all + g * kVtElems, first);

    if (head_ok) {
        const float inv_l = 1.f / st.l;
        const int64_t off = static_cast<int64_t>(i) * (kHq * kD) + head * kD + 4 * G;
        uint16_t* orow = out + b * os + off;
        uint2 gv[16];
        if (gate != nullptr) {
#pragma unroll
            for (int nt = 0; nt < 16; ++nt) gv[nt] = *reinterpret_cast<const uint2*>(gate + b * gs + off + 16 * nt);
        }
#pragma unroll
        for (int nt = 0; nt < 16; ++nt)
            *reinterpret_cast<uint2*>(orow + 16 * nt) =
                pack_out4(st.acc[nt][0] * inv_l, st.acc[nt][1] * inv_l, st.acc[nt][2] * inv_l,
                          st.acc[nt][3] * inv_l, gate != nullptr ? &gv[nt] : nullptr);
        if (lse != nullptr && G == 0)
            lse[b * lss + static_cast<int64_t>(i) * kHq + head] = st.m * scale + logf(st.l);
    }
}

hipError_t launch_attn_prefill(const uint16_t* q, int64_t qs, const uint16_t* k,
                               const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                               const Positions& pos0, int batch, int tq, int budget, float scale,
                               uint16_t* out, int64_t os, float* lse, int64_t lss, const uint16_t* gate,
                               int64_t gs, const PageMap* pm, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(batch) * tq;
    if (rows == 0) return hipSuccess;
    const float c = scale * 1.4426950408889634f;
    const InvFreq inv = make_inv_freq(qsa_rope_t{1.0e7, 1.0, 0});
    if (pm != nullptr)
        hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(128), 0, stream,
                           q, qs, k, v, kvs, sel, sels, pos0, tq, budget, scale, c, out, os, lse, lss, gate, gs,
                           inv, 0, *pm);
    else
        hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(128), 0, stream,
                           q, qs, k, v, kvs, sel, sels, pos0, tq, budget, scale, c, out, os, lse, lss, gate, gs,
                           inv, 0, PageMap{});
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode

// Decode rows: token t of sequence b (row r = b * tq + t) sits at position
// pos[b] + t; per sequence q and out are [tq][24][256] and sel [tq][budget].
// Split each row's budget over n_split workgroups; each writes the partial
// (reference max, sum, unnormalised O) of its blocks for the 24 heads.
static void decode_split(int rows, int budget, int* n_split, int* bps) {
    int s = 256 / (rows > 0 ? rows : 1);
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    const int max_s = (budget + 3) / 4;
    if (s > max_s) s = max_s;
    int per = (budget + s - 1) / s;
    per = (per + 3) & ~3;
    *bps = per;
    *n_split = (budget + per - 1) / per;
}

size_t decode_workspace_bytes(int rows, int budget) {
    int s, per;
    decode_split(rows, budget, &s, &per);
    return static_cast<size_t>(rows) * s * kHq * (2 + kD) * sizeof(float);
}

template <bool kPaged>
__global__ __launch_bounds__(128) void attn_decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs, const int32_t* __restrict__ sel, int64_t sels,
    Positions pos, int budget, int tq, int n_split, int bps, float c, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, InvFreq inv, int rope_q, PageMap pm) {
    __shared__ uint16_t vt_all[2 * kVtElems];
    const int g = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int G = lane >> 4;
    const int r = blockIdx.x / n_split;
    const int s = blockIdx.x % n_split;
    const int b = r / tq;
    const int t = r % tq;
    const int p = pos.p[b] + t;
    const int32_t* selrow = sel + b * sels + t * budget;
    const uint16_t* qrow = q + b * qs + t * (kHq * kD);
    const int head = g * kGroup + c16;
    const bool head_ok = c16 < kGroup;

    const int blk_begin = s * bps;
    const int blk_end = min(budget, blk_begin + bps);
    // query loads first, then the selection and the first chunk; the rotary
    // angles are computed while those are in flight
    bf16x8_t qf[8];
    issue_q_frags(qrow + (head_ok ? head : 0) * kD, head_ok, qf);
    const uint16_t *kg, *vg;
    KvPages kp;
    kv_bases<kPaged>(k, v, kvs, pm, b, g, p, kg, vg, kp);
    Chunk first;
    load_chunk<kPaged>(kg, vg, selrow, blk_begin, blk_end, p, kp, first);
    if (rope_q) rotate_q_frags(rope_angle(p, inv), qf);
    WaveState st;
    init_state(st);
    auto load = [&](int cb, Chunk& ch) { load_chunk<kPaged>(kg, vg, selrow, cb, blk_end, p, kp, ch); };
    attend_blocks<2>(load, blk_begin, blk_end, qf, c, st, vt_all + g * kVtElems, first);
    if (head_ok) {
        const int64_t idx = (static_cast<int64_t>(r) * n_split + s) * kHq + head;
        if (G == 0) {
            ws_ml[2 * idx] = st.m;
            ws_ml[2 * idx + 1] = st.l;
        }
        float* a = ws_acc + idx * kD + 4 * G;
#pragma unroll
        for (int nt = 0; nt < 16; ++nt)
            *reinterpret_cast<float4*>(a + 16 * nt) = make_float4(st.acc[nt][0], st.acc[nt][1], st.acc[nt][2], st.acc[nt][3]);
    }
}

// One workgroup of 256 threads per (row, head): thread t merges dims
// 4*(t%64) .. +3 over the splits s = t/64 + 4k, with all its loads issued
// before any is used; the 4 partial sums meet in LDS.
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc, int tq, int n_split, float scale,
    float c, uint16_t* __restrict__ out, int64_t os, float* __restrict__ lse, const uint16_t* __restrict__ gate,
    int64_t gs) {
    __shared__ float w_s[64];
    __shared__ float4 part[3][64];
    __shared__ float sh_M, sh_L;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int quarter = tid >> 6;
    const int r = blockIdx.x / kHq;                       // row = token t of sequence b
    const int h = blockIdx.x % kHq;
    const int b = r / tq;
    const int t = r % tq;
    const int64_t base = static_cast<int64_t>(r) * n_split * kHq + h;    // split s at base + s * kHq
    if (quarter == 0) {
        float m = -INFINITY, l = 0.f;
        if (lane < n_split) {
            m = ws_ml[2 * (base + static_cast<int64_t>(lane) * kHq)];
            l = ws_ml[2 * (base + static_cast<int64_t>(lane) * kHq) + 1];
        }
        float M = m;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float w = (m == -INFINITY) ? 0.f : exp2f((m - M) * c);
        float L = w * l;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
        w_s[lane] = w;
        if (lane == 0) {
            sh_M = M;
            sh_L = L;
        }
    }
    float4 a[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int s = quarter + 4 * k;
        a[k] = (s < n_split) ? *reinterpret_cast<const float4*>(ws_acc + (base + static_cast<int64_t>(s) * kHq) * kD + 4 * lane)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int s = quarter + 4 * k;
        const float ws = (s < n_split) ? w_s[s] : 0.f;
        acc.x += ws * a[k].x;
        acc.y += ws * a[k].y;
        acc.z += ws * a[k].z;
        acc.w += ws * a[k].w;
    }
    if (quarter > 0) part[quarter - 1][lane] = acc;
    __syncthreads();
    if (quarter == 0) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            acc.x += part[q][lane].x;
            acc.y += part[q][lane].y;
            acc.z += part[q][lane].z;
            acc.w += part[q][lane].w;
        }
        const float inv = 1.f / sh_L;
        const int64_t off = static_cast<int64_t>(t * kHq + h) * kD + 4 * lane;
        uint2 gv;
        if (gate != nullptr) gv = *reinterpret_cast<const uint2*>(gate + b * gs + off);
        *reinterpret_cast<uint2*>(out + b * os + off) =
            pack_out4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv, gate != nullptr ? &gv : nullptr);
        if (lse != nullptr && lane == 0) lse[static_cast<int64_t>(r) * kHq + h] = sh_M * scale + logf(sh_L);
    }
}

hipError_t launch_attn_decode_ex(const uint16_t* q, int64_t qs, const uint16_t* k,
                                 const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                                 const Positions& pos, int batch, int tq, int budget, float scale,
                                 uint16_t* out, int64_t os, float* lse, const uint16_t* gate, int64_t gs,
                                 void* ws, const qsa_rope_t* rope, const PageMap* pm, hipStream_t stream) {
    const int rows = batch * tq;
    if (rows == 0) return hipSuccess;
    int n_split, bps;
    decode_split(rows, budget, &n_split, &bps);
    float* ws_ml = static_cast<float*>(ws);
    float* ws_acc = ws_ml + static_cast<size_t>(rows) * n_split * kHq * 2;
    const float c = scale * 1.4426950408889634f;
    const InvFreq inv = make_inv_freq(rope != nullptr ? *rope : qsa_rope_t{1.0e7, 1.0, 0});
    if (pm != nullptr)
        hipLaunchKernelGGL(attn_decode_split_kernel<true>, dim3(static_cast<unsigned>(rows * n_split)),
                           dim3(128), 0, stream, q, qs, k, v, kvs, sel, sels, pos, budget, tq, n_split, bps,
                           c, ws_ml, ws_acc, inv, rope != nullptr ? 1 : 0, *pm);
    else
        hipLaunchKernelGGL(attn_decode_split_kernel<false>, dim3(static_cast<unsigned>(rows * n_split)),
                           dim3(128), 0, stream, q, qs, k, v, kvs, sel, sels, pos, budget, tq, n_split, bps,
                           c, ws_ml, ws_acc, inv, rope != nullptr ? 1 : 0, PageMap{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(static_cast<unsigned>(rows * kHq)), dim3(256),
                       0, stream, ws_ml, ws_acc, tq, n_split, scale, c, out, os, lse, gate, gs);
    return hipGetLastError();
}

hipError_t launch_attn_decode(const uint16_t* q, int64_t qs, const uint16_t* k,
                              const uint16_t* v, int64_t kvs, const int32_t* sel, int64_t sels,
                              const Positions& pos, int batch, int tq, int budget, float scale,
                              uint16_t* out, int64_t os, float* lse, const uint16_t* gate, int64_t gs,
                              void* ws, hipStream_t stream) {
    return launch_attn_decode_ex(q, qs, k, v, kvs, sel, sels, pos, batch, tq, budget, scale, out, os, lse,
                                 gate, gs, ws, nullptr, nullptr, stream);
}

}  // namespace qsa
