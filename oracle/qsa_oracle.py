"""CPU oracle for one layer of Qwen Sparse Attention (QSA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import or run this module; the product path (the HIP
library and its Python binding) never does, and shares no code with it.

What the layer computes, from the pages:
  * Qwen3.8-Flash-Next blog, section "Attention: GDN + QSA": a lightweight
    indexer first aggregates the sequence into micro-blocks, estimates context
    importance at block level, then selects the most relevant regions, and
    attention runs over those regions only.
  * Qwen3.8-Flash-Next model card (GGUF mirror), "Model Overview", entry
    "Qwen Sparse Attention": 24 query heads and 2 KV heads, head dimension 256,
    rotary dimension 64, indexer = MQA with 4 query heads and 1 shared key
    head of dimension 128, budget 512 blocks or 2048 tokens (so 4 tokens per
    micro-block).
  * model card, "Processing Ultra-Long Texts" (rope_parameters): rope_theta
    1e7, partial_rotary_factor 0.25 (64 of 256 dims), mRoPE sections
    [11, 11, 10] interleaved -- for text all three position ids are equal, so
    it is ordinary 1-D rotary embedding over 32 frequencies.

Readings taken where the pages are silent (each restated at its function):
  block key   = mean of the block's 4 indexer keys, summed in float32 in token
                order, times 0.25, rounded to bf16 (nearest, ties to even);
  block score = sum over the 4 indexer heads of q_h . kbar, no weights, no
                scale, no activation; computed in float64 (each bf16 x bf16
                product exact, the 512-term sum within 2^-44 of sum |q k|,
                far below the float32 rounding) and rounded once to float32;
  candidates  = complete blocks strictly before the query's own block
                o(t) = floor(t / 4); the own block is always selected and
                counts toward the budget;
  selection   = top (budget - 1) candidates by (score descending, block index
                ascending); -0.0 ties +0.0; NaN ranks below every number;
                emitted ascending, padded with -1;
  attention   = per query token, shared by all heads; query head h reads KV
                head floor(h / 12); softmax scale 1/sqrt(256); tokens of the
                own block are attended only up to the query itself;
  rotary      = rotate-half pairing (i, i + 32) inside the first 64 dims,
                angle = position * theta**(-i / 32), applied to Q and K only;
  static YaRN = (optional; model card, "Processing Ultra-Long Texts": rope_type
                yarn, factor 4, original_max_position_embeddings 262144, for
                contexts past 262144) the YaRN paper's NTK-by-parts blend of
                the frequencies with the frameworks' integer ramp ends and
                beta_fast 32 / beta_slow 1, cos and sin scaled by 0.1 ln s + 1
                (the pages name the method and its parameters only);
  output gate = (optional) out * sigmoid(g) per head dim, g an input of the
                output's shape (blog, "Training stability": the attention
                output gating mechanism is retained; its definition is not
                given).

Arithmetic is float64 except where a stored precision is part of the
definition (bf16 block keys, float32 scores).  Functions take generic head
counts and dimensions so brute-force pins can run on tiny shapes.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 4
ROPE_THETA = 1.0e7


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16)."""
    u32 = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 in ONE round-to-nearest-even step.

    bf16 keeps 8 significant bits.  Write x = m * 2**e with 0.5 <= |m| < 1,
    round m * 2**8 to the nearest integer (ties to even) and scale back.  The
    result is exactly representable in float32, whose upper 16 bits are the
    bf16 pattern.  Inputs must be finite, and zero or of magnitude at least
    2**-126 (bf16's smallest normal number).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    if not np.all(np.isfinite(x)) or np.any((ax != 0) & (ax < 2.0 ** -126)) or np.any(ax >= 2.0 ** 128):
        raise ValueError("f64_to_bf16: value outside bf16's normal range")
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# step 0: rotary embedding of the attention Q and K
# --------------------------------------------------------------------------

def rope_inv_freq(rot_dim: int = 64, theta: float = ROPE_THETA) -> np.ndarray:
    """theta**(-2i/rot_dim) for i < rot_dim/2 (model card rope_parameters)."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / rot_dim)


@dataclass(frozen=True)
class Yarn:
    """Static YaRN rotary scaling (model card, "Processing Ultra-Long Texts":
    rope_type yarn, factor 4.0, original_max_position_embeddings 262144; a
    context of about 512K is better served by factor 2).  beta_fast and
    beta_slow are the YaRN paper's alpha / beta bounds on rotation counts."""
    factor: float = 4.0
    original_max: int = 262144
    beta_fast: float = 32.0
    beta_slow: float = 1.0


def yarn_inv_freq(yarn: Yarn, rot_dim: int = 64, theta: float = ROPE_THETA) -> tuple[np.ndarray, float]:
    """Frequencies and cos/sin factor of static YaRN (Peng et al., 2023,
    "YaRN: Efficient Context Window Extension of Large Language Models":
    NTK-by-parts interpolation plus the attention temperature), static, i.e.
    one table for every length, as the model card says the frameworks do.

    Pair i turns L * w_i / (2 pi) times over the original context L, where
    w_i = theta**(-2i/rot_dim).  Solving that count = rho for i gives
    i(rho) = (rot_dim / 2) * ln(L / (2 pi rho)) / ln(theta).  The ramp runs
    from lo = floor(i(beta_fast)) to hi = ceil(i(beta_slow)) (lo at least 0,
    hi at most rot_dim - 1, hi nudged by 0.001 if they meet): pairs at or
    below lo keep w_i (many turns: extrapolated), pairs at or above hi take
    w_i / s (interpolated), and in between the two blend linearly in i.
    cos and sin are multiplied by 0.1 * ln(s) + 1 (the paper's sqrt(1/t)).
    s = 1 returns the plain frequencies and factor 1.
    """
    w = rope_inv_freq(rot_dim, theta)
    s = float(yarn.factor)
    if s <= 1.0:
        return w, 1.0
    L = float(yarn.original_max)

    def pair_at(rho: float) -> float:
        return (rot_dim / 2) * np.log(L / (2.0 * np.pi * rho)) / np.log(theta)

    lo = max(np.floor(pair_at(yarn.beta_fast)), 0.0)
    hi = min(np.ceil(pair_at(yarn.beta_slow)), rot_dim - 1.0)
    if lo == hi:
        hi += 0.001
    i = np.arange(rot_dim // 2, dtype=np.float64)
    ramp = np.clip((i - lo) / (hi - lo), 0.0, 1.0)      # 0: keep w_i, 1: w_i / s
    inv = (w / s) * ramp + w * (1.0 - ramp)
    return inv, 0.1 * np.log(s) + 1.0


def rope_rotate_f64(x: np.ndarray, positions: np.ndarray, rot_dim: int = 64,
                    theta: float = ROPE_THETA, yarn: Yarn | None = None) -> np.ndarray:
    """Unrounded rotary embedding.  x: float64 [..., T, H, D]; positions: [T].

    Pair (i, i + rot_dim/2) of the rotary slice is turned by the angle
    position * inv_freq[i]:  (a, b) -> (a cos - b sin, b cos + a sin).
    Dimensions from rot_dim on pass through unchanged.  With yarn, inv_freq
    and the factor on cos and sin come from yarn_inv_freq.
    """
    half = rot_dim // 2
    if yarn is None:
        inv, m = rope_inv_freq(rot_dim, theta), 1.0
    else:
        inv, m = yarn_inv_freq(yarn, rot_dim, theta)
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]
    c = (np.cos(ang) * m)[:, None, :]
    s = (np.sin(ang) * m)[:, None, :]
    a = x[..., :half]
    b = x[..., half:rot_dim]
    out = np.array(x, dtype=np.float64, copy=True)
    out[..., :half] = a * c - b * s
    out[..., half:rot_dim] = b * c + a * s
    return out


def rope_rotate(x_bits: np.ndarray, positions: np.ndarray, rot_dim: int = 64,
                theta: float = ROPE_THETA, yarn: Yarn | None = None) -> np.ndarray:
    """Rotary embedding of bf16 tensors [..., T, H, D]; result rounded once to bf16."""
    return f64_to_bf16(rope_rotate_f64(bf16_to_f64(x_bits), positions, rot_dim, theta, yarn))


# --------------------------------------------------------------------------
# step 1: micro-block key compression
# --------------------------------------------------------------------------

def compress_block_keys(k_idx_bits: np.ndarray, block_begin: int, block_end: int) -> np.ndarray:
    """Block keys of blocks [block_begin, block_end) of one sequence.

    k_idx_bits: bf16 [L, Di] indexer keys (one shared key head) with
    L >= 4 * block_end.  The block key is the mean of the block's 4 keys
    (blog, "Attention: GDN + QSA": the indexer aggregates the sequence into
    micro-blocks): the 4 keys are added in float32 in token order, the sum is
    multiplied by 0.25 and the result is rounded to bf16.
    """
    n = block_end - block_begin
    di = k_idx_bits.shape[-1]
    if n <= 0:
        return np.zeros((0, di), np.uint16)
    k = bf16_to_f64(k_idx_bits[BLOCK * block_begin: BLOCK * block_end]).astype(np.float32)
    k = k.reshape(n, BLOCK, di)
    total = k[:, 0, :] + k[:, 1, :]
    total = total + k[:, 2, :]
    total = total + k[:, 3, :]
    mean = total * np.float32(0.25)
    return f64_to_bf16(mean.astype(np.float64))


# --------------------------------------------------------------------------
# step 2: block scores of the MQA indexer
# --------------------------------------------------------------------------

def index_scores(q_idx_bits: np.ndarray, kbar_f64: np.ndarray) -> np.ndarray:
    """Scores of query rows against blocks, float32 [R, n].

    q_idx_bits: bf16 [R, Hi, Di] indexer queries; kbar_f64: [n, Di] block keys
    as float64.  score[r, j] = sum_h sum_d q[r, h, d] * kbar[j, d] (model card:
    MQA indexer, 4 query heads sharing 1 key head), evaluated in float64 and
    rounded once to float32.  Causality (which j a row may see) is applied by
    the selection step.
    """
    q = bf16_to_f64(q_idx_bits)                       # [R, Hi, Di]
    r, hi, di = q.shape
    per_head = kbar_f64 @ q.reshape(r * hi, di).T     # [n, R*Hi]
    s = per_head.reshape(-1, r, hi).sum(axis=2)       # [n, R]
    return s.T.astype(np.float32)


# --------------------------------------------------------------------------
# step 3: top-k block selection
# --------------------------------------------------------------------------

def own_block(t: int) -> int:
    return t // BLOCK


def select_blocks(scores_row: np.ndarray, t: int, budget: int) -> np.ndarray:
    """Selected blocks of the query at position t, int32 [budget].

    Candidates are the complete blocks before the own block, j < o = t // 4
    (scores_row[j] for j < o).  The budget (model card: 512 blocks) counts the
    own block, which is always kept; the other budget - 1 slots go to the
    highest scores, ties to the lower block index, -0.0 equal to +0.0 and NaN
    below every number.  The set is returned in ascending order, padded with -1.
    """
    o = own_block(t)
    keep = min(budget - 1, o)
    s = np.asarray(scores_row[:o], np.float64)
    isnan = np.isnan(s)
    s = np.where(isnan, 0.0, s) + 0.0                 # + 0.0 turns -0.0 into +0.0
    order = np.lexsort((np.arange(o), -s, isnan))     # primary: isnan, then -s, then j
    chosen = np.sort(np.append(order[:keep], o)).astype(np.int32)
    out = np.full(budget, -1, np.int32)
    out[:chosen.size] = chosen
    return out


def expand_tokens(sel: np.ndarray, t: int) -> np.ndarray:
    """Token positions attended by the query at t: the 4 tokens of every
    selected block, cut at t (only the own block reaches past t)."""
    blocks = np.asarray(sel)[np.asarray(sel) >= 0].astype(np.int64)
    tok = (BLOCK * blocks[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
    return tok[tok <= t]


# --------------------------------------------------------------------------
# step 4: attention over the gathered tokens
# --------------------------------------------------------------------------

def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Grouped-query softmax attention of one query token.

    q: float64 [Hq, D]; k, v: float64 [n, Hkv, D] (already gathered).
    Query head h reads KV head h // (Hq // Hkv).  Returns (out [Hq, D],
    lse [Hq]) with a max-subtracted float64 softmax.
    """
    hq = q.shape[0]
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    lse = np.zeros(hq)
    for h in range(hq):
        g = h // group
        logits = (k[:, g, :] @ q[h]) * scale          # [n]
        m = logits.max()
        p = np.exp(logits - m)
        l = p.sum()
        out[h] = (p @ v[:, g, :]) / l
        lse[h] = m + np.log(l)
    return out, lse


# --------------------------------------------------------------------------
# optional epilogue of step 4: the attention output gate
# --------------------------------------------------------------------------

def output_gate(out: np.ndarray, gate_bits: np.ndarray) -> np.ndarray:
    """Gated attention output (blog, "Training stability": the attention
    output gating mechanism is retained; the pages do not define it).
    Reading: every head's output is scaled elementwise by the logistic
    function of a gate logit, out * 1 / (1 + exp(-g)), with the logits g
    (bf16, the output's shape) an input of the layer like Q, K and V.
    float64; the log-sum-exp of the softmax is not gated."""
    g = bf16_to_f64(gate_bits)
    return out / (1.0 + np.exp(-g))


# --------------------------------------------------------------------------
# the layer, row by row
# --------------------------------------------------------------------------

@dataclass
class RowResult:
    scores: np.ndarray      # float32 [o(t)]
    sel: np.ndarray         # int32 [budget]
    out: np.ndarray         # float64 [Hq, D]
    lse: np.ndarray         # float64 [Hq]


class OracleLayer:
    """The whole layer for chosen query rows of one batch of sequences.

    Inputs are raw bf16 bit arrays (uint16): q [B, tq, Hq, D],
    q_idx [B, tq, Hi, Di], k and v [B, L, Hkv, D], k_idx [B, L, Di];
    q_pos0[b] is the position of the first query row of sequence b.  Q and K
    are rotated here (K rows stand in the cache rotated), block keys are
    compressed here from k_idx, then every row is scored, selected and
    attended independently.  gate (optional, bf16 bits [B, tq, Hq, D]) gates
    the outputs (output_gate).  yarn (optional) selects static YaRN rotary.
    """

    def __init__(self, q, q_idx, k, v, k_idx, q_pos0, budget: int,
                 rot_dim: int = 64, theta: float = ROPE_THETA, scale: float | None = None, gate=None,
                 yarn: Yarn | None = None):
        self.q, self.q_idx, self.k, self.v, self.k_idx = q, q_idx, k, v, k_idx
        self.gate = gate
        self.yarn = yarn
        self.q_pos0 = np.asarray(q_pos0, np.int64)
        self.budget = budget
        self.rot_dim, self.theta = rot_dim, theta
        self.scale = (1.0 / np.sqrt(q.shape[-1])) if scale is None else scale
        self._kbar: dict[int, np.ndarray] = {}

    def kbar_bits(self, b: int) -> np.ndarray:
        """Block keys of every complete block of sequence b (bf16 bits)."""
        if b not in self._kbar:
            n = self.k_idx.shape[1] // BLOCK
            self._kbar[b] = compress_block_keys(self.k_idx[b], 0, n)
        return self._kbar[b]

    def rows(self, rows, sel_override: dict | None = None) -> list[RowResult]:
        """Run the layer for query rows [(b, t), ...] (t absolute positions).

        sel_override maps (b, t) to a selection to attend with instead of
        the oracle's own (used to replay another implementation's choice)."""
        results = []
        by_seq: dict[int, list[int]] = {}
        for b, t in rows:
            by_seq.setdefault(b, []).append(t)
        cache: dict[tuple[int, int], RowResult] = {}
        for b, ts in by_seq.items():
            kbar = bf16_to_f64(self.kbar_bits(b))
            r_idx = np.array([t - self.q_pos0[b] for t in ts])
            max_o = max(own_block(t) for t in ts)
            sc = index_scores(self.q_idx[b, r_idx], kbar[:max_o])    # [R, max_o]
            for i, t in enumerate(ts):
                o = own_block(t)
                scores = sc[i, :o]
                sel = select_blocks(scores, t, self.budget)
                if sel_override is not None and (b, t) in sel_override:
                    sel = np.asarray(sel_override[(b, t)], np.int32)
                tok = expand_tokens(sel, t)
                qr = rope_rotate(self.q[b, r_idx[i]][None], np.array([t]), self.rot_dim, self.theta,
                                 self.yarn)[0]
                kr = rope_rotate(self.k[b, tok], tok, self.rot_dim, self.theta, self.yarn)
                out, lse = attend(bf16_to_f64(qr), bf16_to_f64(kr), bf16_to_f64(self.v[b, tok]),
                                  self.scale)
                if self.gate is not None:
                    out = output_gate(out, self.gate[b, r_idx[i]])
                cache[(b, t)] = RowResult(scores, sel, out, lse)
        for b, t in rows:
            results.append(cache[(b, t)])
        return results


def bits(t) -> np.ndarray:
    """uint16 bit view of a CPU torch bf16 tensor (or pass a uint16 array through)."""
    if isinstance(t, np.ndarray):
        return t
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
