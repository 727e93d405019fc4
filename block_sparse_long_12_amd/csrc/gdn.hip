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
//  gdn_prep_kernel   chunk-parallel, one workgroup per (sequence, chunk, Q/K
//                    head): normalises q and k (bf16, every load in flight at
//                    once), and for each of the head's 3 V heads forms k k^T
//                    and q k^T on the matrix cores, builds A and P from the
//                    accumulators, and solves the unit lower-triangular system
//                    by forward substitution in fp32 (one thread per
//                    right-hand column, its 64 unknowns in registers),
//                    writing U (fp32), -Wk and P (bf16) and c.  Sized for 3
//                    workgroups per CU, so one's loads overlap another's solve.
//  gdn_state_kernel  sequential over chunks, one workgroup per (sequence, V
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
constexpr int kGdnCols = 32;        // state columns per state-pass workgroup
constexpr int kGdnSegChunks = 512;  // chunks per workspace segment

// Workspace of one segment (nseg chunks), per sequence b and chunk l:
struct GdnWs {
    uint16_t* qn;    // [B][nseg][16][64][128]  normalised q / sqrt(128), token-major
    uint16_t* knt;   // [B][nseg][16][128][64]  normalised k, dim-major
    float* u;        // [B][nseg][48][64][128]
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
    return gdn_seg_bytes(batch, chunks < kGdnSegChunks ? chunks : kGdnSegChunks);
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

struct PrepSmem {
    alignas(16) uint16_t qn[kGdnC][kGdnD + 8];     // +8: rows 16 B apart in bank phase
    alignas(16) uint16_t kn[kGdnC][kGdnD + 8];
    alignas(16) float a[kGdnC][kGdnC];              // strictly lower part used
    float gam[kGdnC];
    float beta[kGdnC];
};

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }


__global__ __launch_bounds__(256, 3) void gdn_prep_kernel(GdnIn in, GdnWs w, int seg_c0, int nseg, int T) {
    __shared__ PrepSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hk = blockIdx.x % kGdnHk;
    const int rest = blockIdx.x / kGdnHk;
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
        *reinterpret_cast<uint32_t*>(&sm.qn[i][2 * lane]) = qb;
        *reinterpret_cast<uint32_t*>(&sm.kn[i][2 * lane]) = kb;
    }
    lds_barrier();
    // normalised rows to the workspace: q token-major, k dim-major
    {
        uint16_t* qdst = w.qn + (slot * kGdnHk + hk) * (kGdnC * kGdnD);
        for (int e = tid; e < kGdnC * kGdnD / 8; e += 256) {
            const int i = e / (kGdnD / 8), d8 = e % (kGdnD / 8);
            *reinterpret_cast<uint4*>(qdst + i * kGdnD + 8 * d8) = *reinterpret_cast<const uint4*>(&sm.qn[i][8 * d8]);
        }
        uint16_t* kdst = w.knt + (slot * kGdnHk + hk) * (kGdnD * kGdnC);
        for (int e = tid; e < kGdnD * kGdnC / 8; e += 256) {      // 8 tokens of one dim per store
            const int d = e / (kGdnC / 8), i8 = e % (kGdnC / 8);
            uint16_t v8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) v8[x] = sm.kn[8 * i8 + x][d];
            *reinterpret_cast<uint4*>(kdst + d * kGdnC + 8 * i8) = *reinterpret_cast<const uint4*>(v8);
        }
    }
    for (int e = 0; e < kGdnGroup; ++e) {
        const int h = hk * kGdnGroup + e;
        const int64_t hs = slot * kGdnHv + h;
        // this head's V rows for the substitution, in flight during the work below
        float x[kGdnC];
        const int col = tid & (kGdnD - 1);
        if (tid < kGdnD) {
#pragma unroll
            for (int i = 0; i < kGdnC; ++i)
                x[i] = bf16_to_f32(in.v[b * in.vs + (static_cast<int64_t>(t0 + min(i, n - 1)) * kGdnHv + h) * kGdnD + col]);
        }
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
            w.gam[hs * kGdnC + lane] = c;
        }
        lds_barrier();
        // A (strictly lower) and P (lower incl. the diagonal, bf16 to the workspace)
        // straight from k k^T and q k^T on the matrix cores: wave w takes rows 16w .. 16w + 15
        {
            const int c16 = lane & 15, G = lane >> 4;
            uint16_t* pdst = w.p + hs * (kGdnC * kGdnC);
            for (int tj = 0; tj < 4; ++tj) {
                f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8_t bk = lds_frag(&sm.kn[16 * tj + c16][32 * s + 8 * G]);
                    ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(&sm.kn[16 * wave + c16][32 * s + 8 * G]),
                                                                 bk, ag, 0, 0, 0);
                    aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(&sm.qn[16 * wave + c16][32 * s + 8 * G]),
                                                                 bk, aq, 0, 0, 0);
                }
                const int j = 16 * tj + c16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * wave + 4 * G + r;
                    const float dec = j <= i ? expf(sm.gam[i] - sm.gam[j]) : 0.f;
                    sm.a[i][j] = j < i ? sm.beta[i] * dec * ag[r] : 0.f;
                    pdst[i * kGdnC + j] = f32_to_bf16(dec * aq[r]);
                }
            }
        }
        lds_barrier();
        // forward substitution, one right-hand column per thread: columns 0..127 of
        // beta v, then 128..255 of beta exp(c) k (beta is 0 past the chunk end)
        if (tid < kGdnD) {
#pragma unroll
            for (int i = 0; i < kGdnC; ++i) x[i] *= sm.beta[i];
        } else {
#pragma unroll
            for (int i = 0; i < kGdnC; ++i) x[i] = sm.beta[i] * expf(sm.gam[i]) * bf16_to_f32(sm.kn[i][col]);
        }
#pragma unroll
        for (int i = 1; i < kGdnC; ++i) {
            float acc = x[i];
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= sm.a[i][j] * x[j];
            x[i] = acc;
        }
        if (tid < kGdnD) {
            float* udst = w.u + hs * (kGdnC * kGdnD) + col;
#pragma unroll
            for (int i = 0; i < kGdnC; ++i) udst[i * kGdnD] = x[i];
        } else {
            uint16_t* wdst = w.wk + hs * (kGdnC * kGdnD) + col;
#pragma unroll
            for (int i = 0; i < kGdnC; ++i) wdst[i * kGdnD] = f32_to_bf16(-x[i]);
        }
        lds_barrier();
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
    float u[2][4];       // U rows 16w + 4(l/16) + r, column 16ct + l%16 of the block
    float gr[4];         // c of rows 16w + 4(l/16) + r
    float glast;         // c of the chunk's last token
};

__device__ __forceinline__ void gdn_load_ops(const GdnWs& w, int64_t slot, int hk, int h, int cb, GdnOps& o) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    const int64_t hs = slot * kGdnHv + h;
    const uint16_t* wk = w.wk + hs * (kGdnC * kGdnD) + (16 * wave + c16) * kGdnD + 8 * G;
    const uint16_t* qn = w.qn + (slot * kGdnHk + hk) * (kGdnC * kGdnD) + (16 * wave + c16) * kGdnD + 8 * G;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.wk[s] = *reinterpret_cast<const bf16x8_t*>(wk + 32 * s);
        o.qn[s] = *reinterpret_cast<const bf16x8_t*>(qn + 32 * s);
    }
    const uint16_t* pp = w.p + hs * (kGdnC * kGdnC) + (16 * wave + c16) * kGdnC + 8 * G;
    o.p[0] = *reinterpret_cast<const bf16x8_t*>(pp);
    o.p[1] = *reinterpret_cast<const bf16x8_t*>(pp + 32);
    const uint16_t* kt = w.knt + (slot * kGdnHk + hk) * (kGdnD * kGdnC) + (32 * wave + c16) * kGdnC + 8 * G;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        o.kt[rt][0] = *reinterpret_cast<const bf16x8_t*>(kt + 16 * rt * kGdnC);
        o.kt[rt][1] = *reinterpret_cast<const bf16x8_t*>(kt + 16 * rt * kGdnC + 32);
    }
    const float* u = w.u + hs * (kGdnC * kGdnD) + (16 * wave + 4 * G) * kGdnD + kGdnCols * cb + c16;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) o.u[ct][r] = u[r * kGdnD + 16 * ct];
    const float* gm = w.gam + hs * kGdnC;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.gr[r] = gm[16 * wave + 4 * G + r];
    o.glast = gm[kGdnC - 1];
}

struct StateBuf {
    alignas(16) uint16_t st[kGdnCols][kGdnD + 8];    // bf16 S^T of the block: [column][dim]
    alignas(16) uint16_t wt[kGdnCols][kGdnC + 8];    // bf16 W^T: [column][token]
    alignas(16) uint16_t dwt[kGdnCols][kGdnC + 8];   // bf16 (exp(c_last - c) W)^T
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats to packed bf16, round to nearest even (one hardware conversion)
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// One chunk.  Consecutive chunks use the two buffers in turn, so the buffer a
// chunk writes was last read two chunks earlier, before the first barrier of
// the chunk in between: two barriers per chunk.
__device__ __forceinline__ void gdn_chunk(const GdnOps& o, f32x4_t (&S)[2][2], StateBuf& sm, const GdnIn& in,
                                          int b, int h, int cb, int t0, int n) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    // the state block as a bf16 B operand: S^T rows (columns of S) in LDS
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
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
    lds_barrier();
    // W = U - Wk S for tokens 16w .. 16w + 15 (U added after the products, so
    // the prefetched U stays where it landed until here)
    f32x4_t W[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
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
    for (int ct = 0; ct < 2; ++ct) {
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
    for (int ct = 0; ct < 2; ++ct) {
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
            if (i < n)
                in.out[b * in.os + (static_cast<int64_t>(t0 + i) * kGdnHv + h) * kGdnD + kGdnCols * cb + 16 * ct + c16] =
                    static_cast<uint16_t>(pr >> (16 * (r & 1)));
        }
    }
    // S = exp(c_last) S + k^T (exp(c_last - c) W)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            S[rt][ct] *= el;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                S[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    o.kt[rt][s], lds_frag(&sm.dwt[16 * ct + c16][32 * s + 8 * G]), S[rt][ct], 0, 0, 0);
        }
}

__global__ __launch_bounds__(256) void gdn_state_kernel(GdnIn in, GdnWs w, int seg_c0, int nseg, int T) {
    __shared__ StateBuf sm[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, G = lane >> 4;
    const int cb = blockIdx.x % (kGdnD / kGdnCols);
    const int rest = blockIdx.x / (kGdnD / kGdnCols);
    const int h = rest % kGdnHv;
    const int b = rest / kGdnHv;
    const int hk = h / kGdnGroup;
    // the state block: rows 32w + 16rt + 4(l/16) + r, column 32cb + 16ct + l%16
    float* sg = in.state + (static_cast<int64_t>(b) * kGdnHv + h) * (kGdnD * kGdnD) + kGdnCols * cb + c16;
    f32x4_t S[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[rt][ct][r] = sg[(32 * wave + 16 * rt + 4 * G + r) * kGdnD + 16 * ct];
    GdnOps A, B;
    const int64_t slot0 = static_cast<int64_t>(b) * nseg;
    gdn_load_ops(w, slot0, hk, h, cb, A);
    // two named operand buffers: chunk l + 1 loads while chunk l computes
    auto run = [&](const GdnOps& o, int l) {
        const int t0 = (seg_c0 + l) * kGdnC;
        gdn_chunk(o, S, sm[l & 1], in, b, h, cb, t0, min(kGdnC, T - t0));
    };
    // (the next chunk's loads are issued unconditionally, past the end clamped to
    // the last chunk, so the wait counts stay exact: a skipped load would make the
    // compiler drain every load in flight)
    for (int l = 0; l < nseg; l += 2) {
        gdn_load_ops(w, slot0 + min(l + 1, nseg - 1), hk, h, cb, B);
        run(A, l);
        if (l + 1 >= nseg) break;
        gdn_load_ops(w, slot0 + min(l + 2, nseg - 1), hk, h, cb, A);
        run(B, l + 1);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) sg[(32 * wave + 16 * rt + 4 * G + r) * kGdnD + 16 * ct] = S[rt][ct][r];
}

hipError_t launch_gdn_prefill(const GdnIn& in, int batch, int n_tokens, void* ws, hipStream_t stream) {
    const int chunks = (n_tokens + kGdnC - 1) / kGdnC;
    for (int c0 = 0; c0 < chunks; c0 += kGdnSegChunks) {
        const int nseg = min(kGdnSegChunks, chunks - c0);
        const GdnWs w = gdn_carve(ws, batch, nseg);
        hipLaunchKernelGGL(gdn_prep_kernel, dim3(static_cast<unsigned>(batch * nseg * kGdnHk)), dim3(256), 0, stream,
                           in, w, c0, nseg, n_tokens);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(gdn_state_kernel, dim3(static_cast<unsigned>(batch * kGdnHv * (kGdnD / kGdnCols))),
                           dim3(256), 0, stream, in, w, c0, nseg, n_tokens);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- decode

// Thread t holds state rows 16 (t / 32) .. + 15 of column 32cb + t % 32.
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
    __syncthreads();
    const float nq = s_norm[0][0] + s_norm[0][1], nk = s_norm[1][0] + s_norm[1][1];
    if (tid < kGdnD) {
        s_q[tid] = nq > 0.f ? qv / (sqrtf(nq) * sqrtf(static_cast<float>(kGdnD))) : 0.f;
        s_k[tid] = nk > 0.f ? kv / sqrtf(nk) : 0.f;
    }
    __syncthreads();
    const float alpha = expf(in.g[b * in.gs + h]);
    const float beta = in.beta[b * in.gs + h];
    // k^T S for this column
    float ks = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ks += s_k[d0 + r] * s[r];
    red[0][tid / kGdnCols][j] = ks;
    __syncthreads();
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
    __syncthreads();
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
