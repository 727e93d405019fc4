// Gated DeltaNet token mixer (Qwen3.8-Flash-Next blog, section "Attention:
// GDN + QSA": three of every four layers keep compressing the history into a
// fixed-size state; model card "Model Overview": 48 V heads, 16 Q/K heads,
// head dim 128).  The rule is the gated delta rule of the Gated DeltaNet
// paper: per V head, with the state S (d_k x d_v),
//     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
// alpha_t = exp(g_t); q and k L2-normalised, q scaled by 1/sqrt(128); V head
// h reads Q/K head h / 3.
//
// Prefill, chunks of 64 tokens (UT transform of the recurrence): inside a
// chunk with cumulative log decay c_i, the written rows w solve
//     (I + A) w = beta v - beta exp(c) (k S_0),  A_ij = beta_i exp(c_i - c_j) k_i.k_j  (j < i),
// so w = U - Wk S_0 with U = (I + A)^-1 beta v and Wk = (I + A)^-1 beta exp(c) k;
// then o = exp(c) (q S_0) + P w with P_ij = exp(c_i - c_j) q_i.k_j (j <= i), and
// the state leaves the chunk as exp(c_last) S_0 + k^T (exp(c_last - c) w).
//
//  gdn_prefill_kernel one launch per workspace segment of 512 chunks, with two
//                    roles: the state pass over segment s in its first
//                    workgroups and the prep of segment s + 1 in the rest (the
//                    prep depends only on the inputs, so it runs on the CUs
//                    the state pass leaves idle; two workspace halves in turn).
//   prep role        chunk-parallel, one workgroup per (sequence, chunk, Q/K
//                    head): normalises q and k (bf16, every load in flight at
//                    once) and forms k k^T and q k^T once on the matrix cores;
//                    then for each of the head's 3 V heads builds A and P from
//                    the accumulators, inverts I + A in fp32 by 16 x 16 blocks
//                    (diagonal blocks by substitution, the rest as fp32
//                    matrix-core products, in place in LDS) and forms U and Wk
//                    as bf16 matrix-core products of the column-scaled inverse
//                    (split into bf16 hi + lo) with V and k, writing U (fp32),
//                    -Wk and P (bf16) and c.
//   state role       sequential over chunks, one workgroup per (sequence, V
//                    head, 32 state columns): the state block (128 x 32 fp32)
//                    lives in matrix-core accumulators for the whole call;
//                    per chunk W = U - Wk S, o = exp(c)(q S) + P W and the
//                    state update are 28 MFMAs per wave, with the next
//                    chunk's operands in flight.
//  gdn_decode_kernel one token per sequence, one workgroup per (sequence, V
//                    head, 32 state columns): the recurrence itself in fp32.
#include "qsa_internal.h"

namespace qsa {

constexpr int kGdnHk = 16;          // Q/K heads
constexpr int kGdnHv = 48;          // V heads
constexpr int kGdnGroup = kGdnHv / kGdnHk;
constexpr int kGdnD = 128;          // head dim (keys and values)
constexpr int kGdnC = 64;           // tokens per chunk
constexpr int kGdnCols = 32;        // state columns per decode workgroup
constexpr int kStCols = 32;         // state columns per state-pass workgroup
constexpr int kStCt = kStCols / 16; // their 16-column tiles
constexpr int kGdnSegChunks = 512;  // chunks per workspace segment

// Workspace of one segment (nseg chunks), per sequence b and chunk l:
struct GdnWs {
    uint16_t* qn;    // [B][nseg][16][64][128]  normalised q / sqrt(128), token-major
    uint16_t* knt;   // [B][nseg][16][128][64]  normalised k, dim-major
    float* u;        // [B][nseg][48][16][128][4]  rows 4q .. 4q + 3 of a column together
    uint16_t* wk;    // [B][nseg][48][64][128]  -Wk
    uint16_t* p;     // [B][nseg][48][64][64]
    float* gam;      // [B][nseg][48][64]       cumulative log decay in the chunk
};

static size_t gdn_seg_bytes(int batch, int nseg) {
    const size_t per_chunk = kGdnHk * (2 * kGdnC * kGdnD * 2) +
                             kGdnHv * (kGdnC * kGdnD * 4 + kGdnC * kGdnD * 2 + kGdnC * kGdnC * 2 + kGdnC * 4);
    return static_cast<size_t>(batch) * nseg * per_chunk;
}

size_t gdn_prefill_ws_bytes(int batch, int n_tokens) {
    const int chunks = (n_tokens + kGdnC - 1) / kGdnC;
    // two segments' operands when there are several: one is read while the next is written
    return gdn_seg_bytes(batch, chunks < kGdnSegChunks ? chunks : kGdnSegChunks) * (chunks > kGdnSegChunks ? 2 : 1);
}

static GdnWs gdn_carve(void* ws, int batch, int nseg) {
    char* p = static_cast<char*>(ws);
    const size_t n = static_cast<size_t>(batch) * nseg;
    GdnWs w;
    w.qn = reinterpret_cast<uint16_t*>(p);
    p += n * kGdnHk * kGdnC * kGdnD * 2;
    w.knt = reinterpret_cast<uint16_t*>(p);
    p += n * kGdnHk * kGdnC * kGdnD * 2;
    w.u = reinterpret_cast<float*>(p);
    p += n * kGdnHv * kGdnC * kGdnD * 4;
    w.wk = reinterpret_cast<uint16_t*>(p);
    p += n * kGdnHv * kGdnC * kGdnD * 2;
    w.p = reinterpret_cast<uint16_t*>(p);
    p += n * kGdnHv * kGdnC * kGdnC * 2;
    w.gam = reinterpret_cast<float*>(p);
    return w;
}

// ---------------------------------------------------------------- prep

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats to packed bf16, round to nearest even (one hardware conversion)
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// LDS of the prep kernel.  The normalised rows (first phase) and, per V head,
// V^T with the triangular matrix (A, then (I + A)^-1 in place) share one region.
struct alignas(16) PrepSmem {
    union {
        struct {
            uint16_t qn[kGdnC][kGdnD + 8];     // +8: rows 16 B apart in bank phase
            uint16_t kn[kGdnC][kGdnD + 8];
        } p1;
        struct {
            uint16_t vt[kGdnD][kGdnC + 8];     // V^T: [dim][token]
            float t[kGdnC * kGdnC];            // element (i, j) at tix(i, j)
        } p2;
    };
    uint16_t kt[kGdnD][kGdnC + 8];             // k^T: [dim][token]
    float gam[kGdnC];                          // cumulative log decay
    float beta[kGdnC];
    float bexp[kGdnC];                         // beta exp(c)
};

// Row i of the 64 x 64 matrix holds its 16-byte chunk q (columns 4q .. 4q + 3)
// at position q ^ (i % 16): the 16 rows of a block read the same chunk from 16
// different bank groups.
__device__ __forceinline__ int tix(int i, int j) { return i * kGdnC + ((((j >> 2) ^ i) & 15) << 2) + (j & 3); }

// acc + X Y for the 16 x 16 blocks X = (xr, xc) and Y = (yr, yc) of t, fp32 on
// the matrix cores (A operand: row l % 16, column 4q + l / 16; B operand: row
// 4q + l / 16, column l % 16; result rows 4(l / 16) + r, column l % 16)
__device__ __forceinline__ f32x4_t blk_mma(const float* t, int lane, int xr, int xc, int yr, int yc, f32x4_t acc) {
    const int c16 = lane & 15, G = lane >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(t[tix(16 * xr + c16, 16 * xc + 4 * q + G)],
                                                   t[tix(16 * yr + 4 * q + G, 16 * yc + c16)], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ void blk_store(float* t, int lane, int br, int bc, const f32x4_t& v, float sign) {
    const int c16 = lane & 15, G = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[tix(16 * br + 4 * G + r, 16 * bc + c16)] = sign * v[r];
}

// Tokens 2p, 2p + 1 (8 bf16 each, dims 8d .. 8d + 7) into dst[dim][token] as
// packed token pairs.
__device__ __forceinline__ void put_pair_t(uint16_t (*dst)[kGdnC + 8], int p, int d, const uint4& a, const uint4& c) {
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        *reinterpret_cast<uint32_t*>(&dst[8 * d + 2 * k][2 * p]) = (av[k] & 0xffffu) | (cv[k] << 16);
        *reinterpret_cast<uint32_t*>(&dst[8 * d + 2 * k + 1][2 * p]) = (av[k] >> 16) | (cv[k] & 0xffff0000u);
    }
}

__device__ __forceinline__ void gdn_prep_body(const GdnIn& in, const GdnWs& w, int seg_c0, int nseg, int T, int bid,
                                              PrepSmem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    const int hk = bid % kGdnHk;
    const int rest = bid / kGdnHk;
    const int cl = rest % nseg;
    const int b = rest / nseg;
    const int t0 = (seg_c0 + cl) * kGdnC;
    const int n = min(kGdnC, T - t0);
    const int64_t slot = static_cast<int64_t>(b) * nseg + cl;

    // the gates of the 3 V heads (thread 64e + i: head e, token i), in flight with the rows
    float g_in = 0.f, b_in = 0.f;
    if (tid < kGdnGroup * kGdnC && tid % kGdnC < n) {
        const int64_t gi = b * in.gs + static_cast<int64_t>(t0 + tid % kGdnC) * kGdnHv + hk * kGdnGroup + tid / kGdnC;
        g_in = in.g[gi];
        b_in = in.beta[gi];
    }
    // V rows of one head for the transposed write: item m covers tokens 2p, 2p + 1
    // (p = tid / 16 + 16m, rows past the chunk end read its last row) at dims 8d .. 8d + 7 (d = tid % 16)
    uint4 vraw[2][2];
    auto load_v = [&](int h) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int tok = min(2 * ((tid >> 4) + 16 * m) + x, n - 1);
                vraw[m][x] = *reinterpret_cast<const uint4*>(
                    in.v + b * in.vs + (static_cast<int64_t>(t0 + tok) * kGdnHv + h) * kGdnD + 8 * (tid & 15));
            }
    };
    load_v(hk * kGdnGroup);
    // normalised q / sqrt(128) and k, rounded to bf16: wave w takes rows 16w .. 16w+15,
    // lane L dims 2L, 2L+1; all 32 loads of a lane are issued before any is used
    uint32_t qraw[16], kraw[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int i = 16 * wave + rr;
        const int64_t off = static_cast<int64_t>(t0 + min(i, n - 1)) * (kGdnHk * kGdnD) + hk * kGdnD + 2 * lane;
        qraw[rr] = *reinterpret_cast<const uint32_t*>(in.q + b * in.qks + off);
        kraw[rr] = *reinterpret_cast<const uint32_t*>(in.k + b * in.qks + off);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int i = 16 * wave + rr;
        const bool ok = i < n;
        const float q0 = ok ? bf16_to_f32(static_cast<uint16_t>(qraw[rr])) : 0.f;
        const float q1 = ok ? bf16_to_f32(static_cast<uint16_t>(qraw[rr] >> 16)) : 0.f;
        const float k0 = ok ? bf16_to_f32(static_cast<uint16_t>(kraw[rr])) : 0.f;
        const float k1 = ok ? bf16_to_f32(static_cast<uint16_t>(kraw[rr] >> 16)) : 0.f;
        float sq = q0 * q0 + q1 * q1, sk = k0 * k0 + k1 * k1;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sq += __shfl_xor(sq, off);
            sk += __shfl_xor(sk, off);
        }
        const float iq = sq > 0.f ? 1.f / (sqrtf(sq) * sqrtf(static_cast<float>(kGdnD))) : 0.f;
        const float ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
        const uint32_t qb = f32_to_bf16(q0 * iq) | (static_cast<uint32_t>(f32_to_bf16(q1 * iq)) << 16);
        const uint32_t kb = f32_to_bf16(k0 * ik) | (static_cast<uint32_t>(f32_to_bf16(k1 * ik)) << 16);
        *reinterpret_cast<uint32_t*>(&sm.p1.qn[i][2 * lane]) = qb;
        *reinterpret_cast<uint32_t*>(&sm.p1.kn[i][2 * lane]) = kb;
    }
    lds_barrier();
    // normalised q to the workspace (token-major); k^T into LDS
    {
        uint16_t* qdst = w.qn + (slot * kGdnHk + hk) * (kGdnC * kGdnD);
        for (int e = tid; e < kGdnC * kGdnD / 8; e += 256) {
            const int i = e / (kGdnD / 8), d8 = e % (kGdnD / 8);
            *reinterpret_cast<uint4*>(qdst + i * kGdnD + 8 * d8) = *reinterpret_cast<const uint4*>(&sm.p1.qn[i][8 * d8]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int p = (tid >> 4) + 16 * m, d = tid & 15;
            put_pair_t(sm.kt, p, d, *reinterpret_cast<const uint4*>(&sm.p1.kn[2 * p][8 * d]),
                       *reinterpret_cast<const uint4*>(&sm.p1.kn[2 * p + 1][8 * d]));
        }
    }
    // k k^T and q k^T of the chunk (shared by the 3 V heads): wave w takes rows 16w .. 16w + 15
    f32x4_t kk[4], qk[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
        kk[tj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        qk[tj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8_t bk = lds_frag(&sm.p1.kn[16 * tj + c16][32 * s + 8 * G]);
            kk[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(&sm.p1.kn[16 * wave + c16][32 * s + 8 * G]), bk,
                                                             kk[tj], 0, 0, 0);
            qk[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(&sm.p1.qn[16 * wave + c16][32 * s + 8 * G]), bk,
                                                             qk[tj], 0, 0, 0);
        }
    }
    lds_barrier();
    // k^T to the workspace (dim-major)
    {
        uint16_t* kdst = w.knt + (slot * kGdnHk + hk) * (kGdnD * kGdnC);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 256 * m, d = e >> 3, i8 = e & 7;
            *reinterpret_cast<uint4*>(kdst + d * kGdnC + 8 * i8) = *reinterpret_cast<const uint4*>(&sm.kt[d][8 * i8]);
        }
    }
    float* t = sm.p2.t;
#pragma unroll 1
    for (int e = 0; e < kGdnGroup; ++e) {
        const int h = hk * kGdnGroup + e;
        const int64_t hs = slot * kGdnHv + h;
        // the lane index, opaque to the compiler in each pass: the per-lane
        // addresses below are recomputed per head instead of being hoisted out
        // of the loop and held (spilled) across it
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int c16 = lane & 15, G = lane >> 4;
        // gates; rows past the chunk end write nothing (beta 0) and keep the decay.
        // The cumulative log decay is an inclusive scan over the wave that holds the head.
        if (wave == e) {
            float c = g_in;
#pragma unroll
            for (int off = 1; off < kGdnC; off <<= 1) {
                const float up = __shfl_up(c, off);
                if (lane >= off) c += up;
            }
            sm.gam[lane] = c;
            sm.beta[lane] = b_in;
            sm.bexp[lane] = b_in * expf(c);
            w.gam[hs * kGdnC + lane] = c;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) put_pair_t(sm.p2.vt, (tid >> 4) + 16 * m, tid & 15, vraw[m][0], vraw[m][1]);
        lds_barrier();
        if (e + 1 < kGdnGroup) load_v(h + 1);               // the next head's rows, in flight from here
        // A (strictly lower) into t, P (lower incl. the diagonal, bf16) to the workspace
        {
            uint16_t* pdst = w.p + hs * (kGdnC * kGdnC);
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const int j = 16 * tj + c16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * wave + 4 * G + r;
                    const float dec = j <= i ? expf(sm.gam[i] - sm.gam[j]) : 0.f;
                    t[tix(i, j)] = j < i ? sm.beta[i] * dec * kk[tj][r] : 0.f;
                    pdst[i * kGdnC + j] = f32_to_bf16(dec * qk[tj][r]);
                }
            }
        }
        lds_barrier();
        // (I + A)^-1 in place, by 16 x 16 blocks.  The diagonal blocks: wave d
        // inverts block d by substitution, column l % 16 per lane.
        {
            const int d = wave, c = c16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float* row = t + (16 * d + r) * kGdnC;
                float acc = r == c ? 1.f : 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (4 * q >= r) break;
                    const float4 a = *reinterpret_cast<const float4*>(row + ((((4 * d + q) ^ r) & 15) << 2));
                    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (4 * q + u < r) acc -= av[u] * x[4 * q + u];
                }
                x[r] = acc;
                __builtin_amdgcn_sched_barrier(0);        // one row's loads at a time (registers)
            }
            if (lane < 16) {
#pragma unroll
                for (int r = 0; r < 16; ++r) t[tix(16 * d + r, 16 * d + c)] = x[r];
            }
        }
        lds_barrier();
        // the 32 x 32 diagonal halves: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22
        if (wave & 1) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t X = blk_mma(t, lane, wave, wave - 1, wave - 1, wave - 1, z);
            blk_store(t, lane, wave, wave - 1, X, 1.f);
            const f32x4_t Y = blk_mma(t, lane, wave, wave, wave, wave - 1, z);
            blk_store(t, lane, wave, wave - 1, Y, -1.f);
        }
        lds_barrier();
        // the lower-left 32 x 32 half: -T_hi A_lowleft T_lo, one 16 x 16 block (a, bc) per wave
        {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const int a = 2 + (wave >> 1), bc = wave & 1;
            f32x4_t Z;
            if (bc == 0)
                Z = blk_mma(t, lane, a, 1, 1, 0, blk_mma(t, lane, a, 0, 0, 0, z));
            else
                Z = blk_mma(t, lane, a, 1, 1, 1, z);
            lds_barrier();
            blk_store(t, lane, a, bc, Z, 1.f);
            lds_barrier();
            f32x4_t Y = blk_mma(t, lane, a, 2, 2, bc, z);
            if (a == 3) Y = blk_mma(t, lane, 3, 3, 3, bc, Y);
            lds_barrier();
            blk_store(t, lane, a, bc, Y, -1.f);
        }
        lds_barrier();
        // U = T diag(beta) V and Wk = T diag(beta exp(c)) k on the matrix cores, each
        // scaled T split into bf16 hi + lo; wave w takes column tiles 2w, 2w + 1
        {
            bf16x8_t vb[2][2], kb[2][2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    vb[cc][s] = lds_frag(&sm.p2.vt[16 * (2 * wave + cc) + c16][32 * s + 8 * G]);
                    kb[cc][s] = lds_frag(&sm.kt[16 * (2 * wave + cc) + c16][32 * s + 8 * G]);
                }
            float* udst = w.u + hs * (kGdnC * kGdnD);
            uint16_t* wdst = w.wk + hs * (kGdnC * kGdnD);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4_t U[2], W[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    U[cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    W[cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                const int i = 16 * rt + c16;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s == 1 && rt < 2) break;                  // T rows below 32 end before column 32
                    float tr[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const float4 v = *reinterpret_cast<const float4*>(t + i * kGdnC +
                                                                          ((((8 * s + 2 * G + hh) ^ i) & 15) << 2));
                        tr[4 * hh] = v.x;
                        tr[4 * hh + 1] = v.y;
                        tr[4 * hh + 2] = v.z;
                        tr[4 * hh + 3] = v.w;
                    }
                    uint32_t uh[4], ul[4], wh[4], wl[4];
#pragma unroll
                    for (int x = 0; x < 8; x += 2) {
                        const int j = 32 * s + 8 * G + x;
                        const float a0 = tr[x] * sm.beta[j], a1 = tr[x + 1] * sm.beta[j + 1];
                        const float e0 = tr[x] * sm.bexp[j], e1 = tr[x + 1] * sm.bexp[j + 1];
                        const uint32_t ha = cvt_bf16x2(a0, a1), he = cvt_bf16x2(e0, e1);
                        uh[x / 2] = ha;
                        wh[x / 2] = he;
                        ul[x / 2] = cvt_bf16x2(a0 - __uint_as_float(ha << 16), a1 - __uint_as_float(ha & 0xffff0000u));
                        wl[x / 2] = cvt_bf16x2(e0 - __uint_as_float(he << 16), e1 - __uint_as_float(he & 0xffff0000u));
                    }
                    const bf16x8_t fuh = __builtin_bit_cast(bf16x8_t, uh), ful = __builtin_bit_cast(bf16x8_t, ul);
                    const bf16x8_t fwh = __builtin_bit_cast(bf16x8_t, wh), fwl = __builtin_bit_cast(bf16x8_t, wl);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        U[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fuh, vb[cc][s], U[cc], 0, 0, 0);
                        U[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ful, vb[cc][s], U[cc], 0, 0, 0);
                        W[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fwh, kb[cc][s], W[cc], 0, 0, 0);
                        W[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fwl, kb[cc][s], W[cc], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int col = 16 * (2 * wave + cc) + c16;
                    const uint32_t w01 = cvt_bf16x2(-W[cc][0], -W[cc][1]), w23 = cvt_bf16x2(-W[cc][2], -W[cc][3]);
                    *reinterpret_cast<f32x4_t*>(udst + ((4 * rt + G) * kGdnD + col) * 4) = U[cc];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * rt + 4 * G + r;
                        wdst[row * kGdnD + col] = static_cast<uint16_t>((r < 2 ? w01 : w23) >> (16 * (r & 1)));
                    }
                }
            }
        }
        lds_barrier();                                      // t, V^T and the gates are rewritten by the next head
    }
}

// ---------------------------------------------------------------- state pass

// One chunk's operands of one wave (row tile w of the chunk, tile rows 2w, 2w+1
// of the state block), loaded one chunk ahead.
struct GdnOps {
    bf16x8_t wk[4];      // -Wk rows 16w + l%16, dims 32s + 8(l/16) ..
    bf16x8_t qn[4];      // q rows, same layout
    bf16x8_t p[2];       // P rows 16w + l%16, tokens 32s + 8(l/16) ..
    bf16x8_t kt[2][2];   // k^T rows (dims) 32w + 16rt + l%16, tokens 32s + 8(l/16) ..
    float u[kStCt][4];   // U rows 16w + 4(l/16) + r, column 16ct + l%16 of the block
    float gr[4];         // c of rows 16w + 4(l/16) + r
    float glast;         // c of the chunk's last token
};

// Per-lane byte offsets of a wave's operands from their per-chunk bases, fixed
// for the whole call: each load is a scalar base plus a 32-bit lane offset.
struct GdnOff {
    uint32_t a;     // -Wk and q rows 16w + l%16, dims 8(l/16) ..
    uint32_t p;     // P rows 16w + l%16, tokens 8(l/16) ..
    uint32_t kt;    // k^T rows 32w + l%16, tokens 8(l/16) ..
    uint32_t u;     // U rows 16w + 4(l/16) .. + 3, column l%16 of the block (one float4)
    uint32_t g;     // c of rows 16w + 4(l/16) ..
};

__device__ __forceinline__ GdnOff gdn_offsets(int cb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    GdnOff f;
    f.a = static_cast<uint32_t>(((16 * wave + c16) * kGdnD + 8 * G) * 2);
    f.p = static_cast<uint32_t>(((16 * wave + c16) * kGdnC + 8 * G) * 2);
    f.kt = static_cast<uint32_t>(((32 * wave + c16) * kGdnC + 8 * G) * 2);
    f.u = static_cast<uint32_t>(((4 * wave + G) * kGdnD + kStCols * cb + c16) * 16);
    f.g = static_cast<uint32_t>((16 * wave + 4 * G) * 4);
    return f;
}

template <typename T>
__device__ __forceinline__ T ld_off(const void* base, uint32_t off) {
    return *reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

__device__ __forceinline__ void gdn_load_ops(const GdnWs& w, int64_t slot, int hk, int h, const GdnOff& f, GdnOps& o) {
    const int64_t hs = slot * kGdnHv + h;
    const uint16_t* wk = w.wk + hs * (kGdnC * kGdnD);
    const uint16_t* qn = w.qn + (slot * kGdnHk + hk) * (kGdnC * kGdnD);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.wk[s] = ld_off<bf16x8_t>(wk, f.a + 64 * s);
        o.qn[s] = ld_off<bf16x8_t>(qn, f.a + 64 * s);
    }
    const uint16_t* pp = w.p + hs * (kGdnC * kGdnC);
    o.p[0] = ld_off<bf16x8_t>(pp, f.p);
    o.p[1] = ld_off<bf16x8_t>(pp, f.p + 64);
    const uint16_t* kt = w.knt + (slot * kGdnHk + hk) * (kGdnD * kGdnC);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        o.kt[rt][0] = ld_off<bf16x8_t>(kt, f.kt + 16 * rt * kGdnC * 2);
        o.kt[rt][1] = ld_off<bf16x8_t>(kt, f.kt + 16 * rt * kGdnC * 2 + 64);
    }
    const float* u = w.u + hs * (kGdnC * kGdnD);
#pragma unroll
    for (int ct = 0; ct < kStCt; ++ct) {
        const f32x4_t u4 = ld_off<f32x4_t>(u, f.u + 16 * ct * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) o.u[ct][r] = u4[r];
    }
    const float* gm = w.gam + hs * kGdnC;
    const float4 g4 = ld_off<float4>(gm, f.g);
    o.gr[0] = g4.x;
    o.gr[1] = g4.y;
    o.gr[2] = g4.z;
    o.gr[3] = g4.w;
    o.glast = gm[kGdnC - 1];
}

struct StateBuf {
    alignas(16) uint16_t st[kStCols][kGdnD + 8];    // bf16 S^T of the block: [column][dim]
    alignas(16) uint16_t wt[kStCols][kGdnC + 8];    // bf16 W^T: [column][token]
    alignas(16) uint16_t dwt[kStCols][kGdnC + 8];   // bf16 (exp(c_last - c) W)^T
};


// One chunk.  Consecutive chunks use the two buffers in turn, so the buffer a
// chunk writes was last read two chunks earlier, before the first barrier of
// the chunk in between: two barriers per chunk.
__device__ __forceinline__ void gdn_chunk(const GdnOps& o, f32x4_t (&S)[2][kStCt], StateBuf& sm, const GdnIn& in,
                                          int b, int h, int cb, int t0, int n) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    // the state block as a bf16 B operand: S^T rows (columns of S) in LDS
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kStCt; ++ct) {
            uint2 pk;
            pk.x = cvt_bf16x2(S[rt][ct][0], S[rt][ct][1]);
            pk.y = cvt_bf16x2(S[rt][ct][2], S[rt][ct][3]);
            *reinterpret_cast<uint2*>(&sm.st[16 * ct + c16][32 * wave + 16 * rt + 4 * G]) = pk;
        }
    // decay factors of this lane's 4 rows (computed while the stores drain)
    float eg[4], ed[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        eg[r] = __expf(o.gr[r]);
        ed[r] = __expf(o.glast - o.gr[r]);
    }
    const float el = __expf(o.glast);
    // the chunk's output rows as a buffer of exactly its n valid tokens: the
    // stores of rows past the sequence end fall outside it and the hardware
    // drops them, so every store is issued unconditionally and the wait
    // counts for the prefetched operands stay exact
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        in.out + b * in.os + static_cast<int64_t>(t0) * (kGdnHv * kGdnD), 0, n * (kGdnHv * kGdnD * 2), 0x00020000);
    lds_barrier();
    // W = U - Wk S for tokens 16w .. 16w + 15 (U added after the products, so
    // the prefetched U stays where it landed until here)
    f32x4_t W[kStCt];
#pragma unroll
    for (int ct = 0; ct < kStCt; ++ct) {
        W[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            W[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.wk[s], lds_frag(&sm.st[16 * ct + c16][32 * s + 8 * G]),
                                                           W[ct], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) W[ct][r] += o.u[ct][r];
    }
    // W^T and (exp(c_last - c) W)^T in bf16 for the next two products
#pragma unroll
    for (int ct = 0; ct < kStCt; ++ct) {
        uint2 pw, pd;
        pw.x = cvt_bf16x2(W[ct][0], W[ct][1]);
        pw.y = cvt_bf16x2(W[ct][2], W[ct][3]);
        pd.x = cvt_bf16x2(ed[0] * W[ct][0], ed[1] * W[ct][1]);
        pd.y = cvt_bf16x2(ed[2] * W[ct][2], ed[3] * W[ct][3]);
        *reinterpret_cast<uint2*>(&sm.wt[16 * ct + c16][16 * wave + 4 * G]) = pw;
        *reinterpret_cast<uint2*>(&sm.dwt[16 * ct + c16][16 * wave + 4 * G]) = pd;
    }
    lds_barrier();
    // o = exp(c) (q S) + P W for tokens 16w .. 16w + 15
#pragma unroll
    for (int ct = 0; ct < kStCt; ++ct) {
        f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            O = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.qn[s], lds_frag(&sm.st[16 * ct + c16][32 * s + 8 * G]), O,
                                                        0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[r] *= eg[r];
#pragma unroll
        for (int s = 0; s < 2; ++s)
            O = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.p[s], lds_frag(&sm.wt[16 * ct + c16][32 * s + 8 * G]), O, 0,
                                                        0, 0);
        const uint32_t o01 = cvt_bf16x2(O[0], O[1]), o23 = cvt_bf16x2(O[2], O[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * G + r;
            const uint32_t pr = r < 2 ? o01 : o23;
            const uint32_t off = static_cast<uint32_t>(((i * kGdnHv + h) * kGdnD + kStCols * cb + 16 * ct + c16) * 2);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pr >> (16 * (r & 1))), orsrc, off, 0, 0);
        }
    }
    // S = exp(c_last) S + k^T (exp(c_last - c) W)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kStCt; ++ct) {
            S[rt][ct] *= el;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                S[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    o.kt[rt][s], lds_frag(&sm.dwt[16 * ct + c16][32 * s + 8 * G]), S[rt][ct], 0, 0, 0);
        }
}

__device__ __forceinline__ void gdn_state_body(const GdnIn& in, const GdnWs& w, int seg_c0, int nseg, int T, int bid,
                                               int nwg, StateBuf (&sm)[2]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    // workgroups are dealt to the 8 XCDs round-robin; renumber them so the
    // column blocks of one head run on one XCD and share its L2 copy of the
    // head's chunk operands (their count, batch x 48 x blocks, is a multiple of 8)
    const int wg = (bid % 8) * (nwg / 8) + bid / 8;
    const int cb = wg % (kGdnD / kStCols);
    const int rest = wg / (kGdnD / kStCols);
    const int h = rest % kGdnHv;
    const int b = rest / kGdnHv;
    const int hk = h / kGdnGroup;
    // the state block: rows 32w + 16rt + 4(l/16) + r, column 32cb + 16ct + l%16
    float* sg = in.state + (static_cast<int64_t>(b) * kGdnHv + h) * (kGdnD * kGdnD) + kStCols * cb + c16;
    f32x4_t S[2][kStCt];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kStCt; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[rt][ct][r] = sg[(32 * wave + 16 * rt + 4 * G + r) * kGdnD + 16 * ct];
    GdnOps A, B;
    const int64_t slot0 = static_cast<int64_t>(b) * nseg;
    const GdnOff off = gdn_offsets(cb);
    gdn_load_ops(w, slot0, hk, h, off, A);
    // two named operand buffers: chunk l + 1 loads while chunk l computes
    auto run = [&](const GdnOps& o, int l) {
        const int t0 = (seg_c0 + l) * kGdnC;
        gdn_chunk(o, S, sm[l & 1], in, b, h, cb, t0, min(kGdnC, T - t0));
    };
    // (the next chunk's loads are issued unconditionally, past the end clamped to
    // the last chunk, so the wait counts stay exact: a skipped load would make the
    // compiler drain every load in flight)
    for (int l = 0; l < nseg; l += 2) {
        gdn_load_ops(w, slot0 + min(l + 1, nseg - 1), hk, h, off, B);
        run(A, l);
        if (l + 1 >= nseg) break;
        gdn_load_ops(w, slot0 + min(l + 2, nseg - 1), hk, h, off, A);
        run(B, l + 1);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kStCt; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) sg[(32 * wave + 16 * rt + 4 * G + r) * kGdnD + 16 * ct] = S[rt][ct][r];
}

// One launch per workspace segment: its first nwg_state workgroups run the
// state pass over segment s while the rest run the prep of segment s + 1 (which
// depends only on the inputs), so the prep fills the CUs the chunk-sequential
// state pass leaves idle.  Consecutive segments use the two halves of the
// workspace in turn; each half is written by one launch and read by the next.
union GdnSmem {
    PrepSmem p;
    StateBuf s[2];
};

__global__ __launch_bounds__(256, 2) void gdn_prefill_kernel(GdnIn in, GdnWs ws_state, int c0_state, int nseg_state,
                                                            int nwg_state, GdnWs ws_prep, int c0_prep, int nseg_prep,
                                                            int T) {
    __shared__ GdnSmem sm;
    const int bid = static_cast<int>(blockIdx.x);
    if (bid < nwg_state)
        gdn_state_body(in, ws_state, c0_state, nseg_state, T, bid, nwg_state, sm.s);
    else
        gdn_prep_body(in, ws_prep, c0_prep, nseg_prep, T, bid - nwg_state, sm.p);
}

hipError_t launch_gdn_prefill(const GdnIn& in, int batch, int n_tokens, void* ws, hipStream_t stream) {
    const int chunks = (n_tokens + kGdnC - 1) / kGdnC;
    const int nsegs = (chunks + kGdnSegChunks - 1) / kGdnSegChunks;
    const size_t half = gdn_seg_bytes(batch, min(chunks, kGdnSegChunks));
    auto seg_len = [&](int s) { return min(kGdnSegChunks, chunks - s * kGdnSegChunks); };
    auto seg_ws = [&](int s) { return gdn_carve(static_cast<char*>(ws) + (s & 1) * half, batch, seg_len(s)); };
    const int nwg_state = batch * kGdnHv * (kGdnD / kStCols);
    for (int s = -1; s < nsegs; ++s) {
        const bool st = s >= 0, pr = s + 1 < nsegs;
        const int n_st = st ? nwg_state : 0;
        const int n_pr = pr ? batch * seg_len(s + 1) * kGdnHk : 0;
        const GdnWs w_st = st ? seg_ws(s) : GdnWs{};
        const GdnWs w_pr = pr ? seg_ws(s + 1) : GdnWs{};
        hipLaunchKernelGGL(gdn_prefill_kernel, dim3(static_cast<unsigned>(n_st + n_pr)), dim3(256), 0, stream, in, w_st,
                           st ? s * kGdnSegChunks : 0, st ? seg_len(s) : 0, n_st, w_pr,
                           pr ? (s + 1) * kGdnSegChunks : 0, pr ? seg_len(s + 1) : 0, n_tokens);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- decode

// Thread t holds state rows 16 (t / 32) .. + 15 of column 32cb + t % 32.
// Only LDS data crosses threads (each thread reads and rewrites its own
// state rows), so the barriers are LDS-only: the output's reduction does not
// wait for the state rows still being written back.
__global__ __launch_bounds__(256) void gdn_decode_kernel(GdnIn in) {
    __shared__ float s_q[kGdnD], s_k[kGdnD];
    __shared__ float red[2][8][kGdnCols];
    __shared__ float s_norm[2][4];
    const int tid = threadIdx.x;
    const int cb = blockIdx.x % (kGdnD / kGdnCols);
    const int rest = blockIdx.x / (kGdnD / kGdnCols);
    const int h = rest % kGdnHv;
    const int b = rest / kGdnHv;
    const int hk = h / kGdnGroup;
    const int j = tid % kGdnCols;
    const int d0 = 16 * (tid / kGdnCols);
    float* sg = in.state + (static_cast<int64_t>(b) * kGdnHv + h) * (kGdnD * kGdnD) + kGdnCols * cb + j;
    float s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = sg[(d0 + r) * kGdnD];
    // normalised q / sqrt(128) and k
    float qv = 0.f, kv = 0.f;
    if (tid < kGdnD) {
        qv = bf16_to_f32(in.q[b * in.qks + hk * kGdnD + tid]);
        kv = bf16_to_f32(in.k[b * in.qks + hk * kGdnD + tid]);
    }
    float sq = qv * qv, sk = kv * kv;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off);
        sk += __shfl_xor(sk, off);
    }
    if ((tid & 63) == 0 && tid < kGdnD) {
        s_norm[0][tid >> 6] = sq;
        s_norm[1][tid >> 6] = sk;
    }
    lds_barrier();
    const float nq = s_norm[0][0] + s_norm[0][1], nk = s_norm[1][0] + s_norm[1][1];
    if (tid < kGdnD) {
        s_q[tid] = nq > 0.f ? qv / (sqrtf(nq) * sqrtf(static_cast<float>(kGdnD))) : 0.f;
        s_k[tid] = nk > 0.f ? kv / sqrtf(nk) : 0.f;
    }
    lds_barrier();
    const float alpha = expf(in.g[b * in.gs + h]);
    const float beta = in.beta[b * in.gs + h];
    // k^T S for this column
    float ks = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ks += s_k[d0 + r] * s[r];
    red[0][tid / kGdnCols][j] = ks;
    lds_barrier();
    float kst = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) kst += red[0][x][j];
    const float vj = bf16_to_f32(in.v[b * in.vs + h * kGdnD + kGdnCols * cb + j]);
    const float u = beta * (vj - alpha * kst);
    float os = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[r] = alpha * s[r] + s_k[d0 + r] * u;
        os += s_q[d0 + r] * s[r];
        sg[(d0 + r) * kGdnD] = s[r];
    }
    red[1][tid / kGdnCols][j] = os;
    lds_barrier();
    if (tid < kGdnCols) {
        float o = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) o += red[1][x][tid];
        in.out[b * in.os + h * kGdnD + kGdnCols * cb + tid] = f32_to_bf16(o);
    }
}

hipError_t launch_gdn_decode(const GdnIn& in, int batch, hipStream_t stream) {
    hipLaunchKernelGGL(gdn_decode_kernel, dim3(static_cast<unsigned>(batch * kGdnHv * (kGdnD / kGdnCols))), dim3(256),
                       0, stream, in);
    return hipGetLastError();
}

}  // namespace qsa
