"""A model of the rounding in the chunk-parallel Gated DeltaNet prefill, used
to derive the tolerance of its GPU test.

TEST INFRASTRUCTURE.  It restates, in float64 numpy, the chunked form of the
gated delta rule (the UT transform of the recurrence over chunks of 64
tokens) and rounds to bf16 at every point where the GPU kernel stores or
feeds a matrix-core product with a bf16 value; everything else is float64
(the kernel accumulates in float32, about 2^-24 relative, far below the bf16
steps of 2^-9 that dominate).  It imports nothing from the HIP path.

Chunk of n tokens with in-chunk cumulative log decay c (c_i = g_1 + .. + g_i):
  qn = bf16(q / (|q| sqrt(128))),  kn = bf16(k / |k|)            (normalised rows)
  A_ij = beta_i exp(c_i - c_j) kn_i.kn_j   (j < i)
  P_ij = bf16(exp(c_i - c_j) qn_i.kn_j)    (j <= i)
  T = (I + A)^-1
  U  = split(T diag(beta)) V               split(X) = bf16(X) + bf16(X - bf16(X))
  Wk = bf16(split(T diag(beta exp(c))) kn)
  per chunk with the state S (d_k x d_v):
  Sb = bf16(S),  W = U - Wk Sb,  Wb = bf16(W),  Db = bf16(exp(c_n - c) W)
  o  = bf16(exp(c) (qn Sb) + P Wb)
  S  = exp(c_n) S + kn^T Db
The exact recurrence (oracle/gdn_oracle.py) is the same algebra without the
roundings: the pins of that oracle include the chunked form solved exactly.
"""

from __future__ import annotations

import numpy as np
import torch

CHUNK = 64


ROUND = True          # False: no rounding anywhere (the exact chunked algebra)


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 the way the kernel does: the float32 value, then
    round-to-nearest-even to bf16 (torch's cast), returned as float64."""
    if not ROUND:
        return np.asarray(x, dtype=np.float64)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def split(x: np.ndarray) -> np.ndarray:
    hi = bf16(x)
    return hi + bf16(x - hi)


def normalise(q: np.ndarray, k: np.ndarray):
    """Rows of one Q/K head [T, 128] (float64 values of bf16 inputs)."""
    nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    nk = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    qn = bf16(np.where(nq > 0, q / np.where(nq > 0, nq, 1.0) / np.sqrt(q.shape[-1]), 0.0))
    kn = bf16(np.where(nk > 0, k / np.where(nk > 0, nk, 1.0), 0.0))
    return qn, kn


def chunked_head(qn, kn, v, g, beta, s0):
    """One V head over T tokens: qn, kn [T, 128] (already normalised and
    rounded), v [T, 128], g, beta [T], s0 [128, 128].  Returns the outputs
    (bf16 values) [T, 128] and the final state (float64) [128, 128]."""
    T = qn.shape[0]
    S = np.array(s0, dtype=np.float64, copy=True)
    out = np.zeros((T, v.shape[1]))
    for t0 in range(0, T, CHUNK):
        n = min(CHUNK, T - t0)
        sl = slice(t0, t0 + n)
        q_c, k_c, v_c, b_c = qn[sl], kn[sl], v[sl], beta[sl]
        c = np.cumsum(g[sl])
        dec = np.exp(c[:, None] - c[None, :])
        low = np.tril(np.ones((n, n)), -1)
        A = b_c[:, None] * dec * (k_c @ k_c.T) * low
        P = bf16(dec * (q_c @ k_c.T) * np.tril(np.ones((n, n))))
        Tm = np.linalg.inv(np.eye(n) + A)
        U = split(Tm * b_c[None, :]) @ v_c
        Wk = bf16(split(Tm * (b_c * np.exp(c))[None, :]) @ k_c)
        Sb = bf16(S)
        W = U - Wk @ Sb
        Wb = bf16(W)
        Db = bf16(np.exp(c[-1] - c)[:, None] * W)
        out[sl] = bf16(np.exp(c)[:, None] * (q_c @ Sb) + P @ Wb)
        S = np.exp(c[-1]) * S + k_c.T @ Db
    return out, S


def emulate(q, k, v, g, beta, s0, heads=None):
    """The prefill of one sequence: q, k [T, 16, 128] and v [T, 48, 128] as
    float64 values of bf16 inputs, g and beta [T, 48], s0 [48, 128, 128].
    heads: the V heads to run (default all).  Returns {h: (out [T, 128],
    state [128, 128])}."""
    res = {}
    prep = {}
    for h in (range(v.shape[1]) if heads is None else heads):
        hk = h // (v.shape[1] // q.shape[1])
        if hk not in prep:
            prep[hk] = normalise(q[:, hk], k[:, hk])
        qn, kn = prep[hk]
        res[h] = chunked_head(qn, kn, v[:, h], np.asarray(g[:, h], np.float64), np.asarray(beta[:, h], np.float64),
                              s0[h])
    return res
