"""CPU oracle for the Gated DeltaNet (GDN) token mixer of the hybrid layers.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import or run this module; the product path never
does, and shares no code with it.

What the pages fix:
  * Qwen3.8-Flash-Next blog, section "Attention: GDN + QSA": three of every
    four layers are Gated DeltaNet layers (reference [1] there), which keep
    compressing the history into a state of fixed size.
  * model card, "Model Overview", entry "Gated DeltaNet": 48 linear-attention
    heads for V and 16 for Q/K, head dimension 128.

The rule itself is the gated delta rule of the Gated DeltaNet paper (Yang,
Kautz and Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
Rule"), restated here from its definition.  Per V head, with the state S a
d_k x d_v matrix (S^T maps keys to values):

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

alpha_t = exp(g_t) in (0, 1] is the gate (decay), beta_t in [0, 1] the
writing strength.

Readings taken where the pages are silent (each restated where used):
  heads      = V head h reads Q/K head h // 3 (48 / 16 = 3 V heads per Q/K
               head, grouped as in grouped-query attention);
  gates      = g and beta are per V head and token (g <= 0 as the log of the
               decay, beta in [0, 1]), given as float32 inputs;
  q, k       = L2-normalised per head (the paper normalises queries and keys),
               then q scaled by 1 / sqrt(128);
  state      = float32 in and out, [d_k][d_v] per V head; the layer starts
               from the projected q / k / v / g / beta (the projections, the
               short convolution and the output norm are not part of it);
  output     = bf16; arithmetic here is float64.
"""

from __future__ import annotations

import numpy as np

HK = 16        # query / key heads
HV = 48        # value heads
DK = 128       # key head dim
DV = 128       # value head dim


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16)."""
    u32 = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """x / ||x|| over the last axis (float64); a zero row stays zero."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def prepare_qk(q: np.ndarray, k: np.ndarray, normalize: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """The rule's q and k: L2-normalised per head, q scaled by 1/sqrt(d_k)."""
    d = q.shape[-1]
    if normalize:
        q, k = l2_normalize(q), l2_normalize(k)
    return q / np.sqrt(d), k


def gated_delta_rule(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
                     s0: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """One V head, token by token: q, k [T, d_k], v [T, d_v], g, beta [T],
    s0 [d_k, d_v] (all float64, q and k already prepared).  Returns the
    outputs [T, d_v] and the final state [d_k, d_v]."""
    s = np.array(s0, dtype=np.float64, copy=True)
    out = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        a = np.exp(g[t])
        kt = k[t]
        # alpha (I - beta k k^T) S + beta k v^T, written out
        s = a * (s - beta[t] * np.outer(kt, kt @ s)) + beta[t] * np.outer(kt, v[t])
        out[t] = s.T @ q[t]
    return out, s


def gdn_layer(q_bits, k_bits, v_bits, g, beta, s0, normalize: bool = True):
    """The whole token mixer for a batch: q, k bf16 bits [B, T, 16, 128], v
    bf16 bits [B, T, 48, 128], g and beta float32 [B, T, 48], s0 float32
    [B, 48, 128, 128].  Returns float64 outputs [B, T, 48, 128] and final
    states [B, 48, 128, 128]."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, hk, _ = q.shape
    hv = v.shape[2]
    group = hv // hk
    out = np.zeros(v.shape)
    s_fin = np.zeros(np.asarray(s0).shape)
    for b in range(B):
        qp, kp = prepare_qk(q[b], k[b], normalize)
        for h in range(hv):
            o, s = gated_delta_rule(qp[:, h // group], kp[:, h // group], v[b, :, h], g[b, :, h], beta[b, :, h],
                                    np.asarray(s0[b, h], np.float64))
            out[b, :, h] = o
            s_fin[b, h] = s
    return out, s_fin
