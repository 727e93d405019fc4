"""Seeded synthetic inputs for one Qwen Sparse Attention (QSA) layer.

This module only draws random numbers and decides where the planted "needle"
blocks go.  It holds none of the layer's arithmetic (no rotary embedding, no
block compression, no scoring, no selection, no attention), so the CPU oracle
and the HIP path can both consume its tensors without sharing any of the
method's code.

Shapes follow the QSA entry of the Qwen3.8-Flash-Next model card (GGUF mirror,
section "Model Overview"): 24 query heads and 2 KV heads of dimension 256, an
MQA indexer with 4 query heads and 1 shared key head of dimension 128, and a
budget of 512 blocks or 2048 tokens (so a micro-block holds 4 tokens).

Distributions: attention Q/K/V are N(0, 1); indexer q/k are N(0, 1/128).  Every
tensor is drawn as float32 from numpy's PCG64, scaled in float32, then rounded
to bfloat16 (round-to-nearest-even, done by torch's CPU cast).  Each tensor has
its own SeedSequence(seed, spawn_key=(tensor_id,)) and is filled in fixed
chunks, each from its own child stream, so the bits do not depend on the
number of worker threads.

K and Q are returned *unrotated*: the rotary pre-pass is part of the layer.

Needles ("keys aligned to random queries"): for a needle (b, t, j) the 4 indexer
keys of block j are all set to bf16(4 * u), u being the unit vector along the
sum of the 4 indexer query heads of token t.  Such a block outscores every
random block by a wide margin for query t (about 8 against a spread of about
0.09), so any correct selection must keep it.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 4          # tokens per micro-block (512 blocks == 2048 tokens)
HQ = 24            # attention query heads
HKV = 2            # attention key/value heads
D = 256            # attention head dimension
ROT = 64           # rotary slice
HI = 4             # indexer query heads
DI = 128           # indexer head dimension
ROPE_THETA = 1.0e7

_CHUNK = 1 << 22   # elements per independently seeded chunk

# tensor ids inside a workload's seed tree
_T_Q, _T_K, _T_V, _T_QI, _T_KI, _T_NEEDLE = range(6)


@dataclass(frozen=True)
class Workload:
    """One synthetic QSA workload.

    kind     'prefill' (tq new query tokens at positions q_pos0 .. q_pos0+tq-1,
             attending to everything before them) or 'decode' (one new token
             at position ctx, after ctx cached tokens).
    ctx      tokens already in the cache before the new ones (prefill: q_pos0).
    chunk    query tokens per indexer/select launch in prefill (None = all).
    """
    name: str
    kind: str
    batch: int
    ctx: int
    tq: int
    budget: int
    n_needles: int
    seed: int
    chunk: int | None = None
    description: str = ""

    @property
    def length(self) -> int:
        """Rows held per sequence in the caches (cached + new)."""
        return self.ctx + self.tq

    @property
    def n_blocks(self) -> int:
        """Complete micro-blocks in the caches after the new tokens."""
        return self.length // BLOCK


WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("prefill_T2048_budget64", "prefill", batch=1, ctx=0, tq=2048,
             budget=64, n_needles=8, seed=1000,
             description="one-layer prefill, B=1, T=2048 (512 blocks), budget 64 blocks, 8 needles"),
    Workload("decode_B32_ctx32K", "decode", batch=32, ctx=32768, tq=1,
             budget=512, n_needles=8, seed=1001,
             description="decode, B=32, one new token after 32768 cached tokens (8192 blocks), budget 512"),
    Workload("prefill_T131072", "prefill", batch=1, ctx=0, tq=131072,
             budget=512, n_needles=64, seed=1002, chunk=8192,
             description="prefill, B=1, T=131072 (32768 blocks), budget 512, 8192-query chunks, 64 needles"),
    Workload("decode_B4_ctx1M", "decode", batch=4, ctx=1048576, tq=1,
             budget=512, n_needles=8, seed=1003,
             description="decode, B=4, one new token after 1048576 cached tokens (262144 blocks), budget 512"),
    Workload("prefill_prefix943718_chunk104858", "prefill", batch=1, ctx=943718,
             tq=104858, budget=512, n_needles=64, seed=1004, chunk=8192,
             description="chunked prefill with a 90% prefix-cache hit: 104858 new tokens after "
                         "943718 cached ones (1M context), budget 512, 8192-query chunks, "
                         "64 needles in the cached prefix"),
]}


def custom_workload(kind: str, batch: int, ctx: int, tq: int, budget: int,
                    n_needles: int = 0, seed: int = 7, chunk: int | None = None) -> Workload:
    """A workload of any size with the same distributions."""
    name = f"{kind}_B{batch}_ctx{ctx}_T{tq}_budget{budget}_seed{seed}"
    return Workload(name, kind, batch, ctx, tq, budget, n_needles, seed, chunk)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_normal(out: torch.Tensor, entropy: int, tensor_id: int, sigma: float,
                 threads: int | None = None) -> None:
    """Fill a contiguous CPU bf16 tensor with bf16(float32(N(0,1)) * sigma)."""
    assert out.dtype == torch.bfloat16 and out.is_contiguous() and out.device.type == "cpu"
    flat = out.view(-1)
    n = flat.numel()
    if n == 0:
        return
    nchunks = (n + _CHUNK - 1) // _CHUNK
    children = np.random.SeedSequence(entropy, spawn_key=(tensor_id,)).spawn(nchunks)
    s32 = np.float32(sigma)

    def work(i: int) -> None:
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            np.multiply(x, s32, out=x)
        flat[lo:hi] = torch.from_numpy(x).to(torch.bfloat16)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(work, range(nchunks)))


@dataclass
class Inputs:
    """Raw (unrotated) layer inputs of a workload, as CPU bf16 tensors.

    q       [B, tq, 24, 256]   attention queries of the new tokens
    q_idx   [B, tq, 4, 128]    indexer queries of the new tokens
    k, v    [B, L, 2, 256]     attention keys/values of all L = ctx + tq rows
    k_idx   [B, L, 128]        indexer keys of all rows (needles planted)
    q_pos0  [B] int32          position of the first new token per sequence
    needles [n, 3] int64       (b, t, j): block j planted for the query at position t
    """
    workload: Workload
    q: torch.Tensor
    q_idx: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    k_idx: torch.Tensor
    q_pos0: np.ndarray
    needles: np.ndarray = field(default_factory=lambda: np.zeros((0, 3), np.int64))


def _plant_needles(wl: Workload, q_idx: torch.Tensor, k_idx: torch.Tensor,
                   q_pos0: np.ndarray) -> np.ndarray:
    if wl.n_needles == 0:
        return np.zeros((0, 3), np.int64)
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(wl.seed, spawn_key=(_T_NEEDLE,))))
    # decode: n_needles per sequence, all aligned to its one new token;
    # prefill: n_needles in total, spread round-robin over the sequences
    total = wl.n_needles * (wl.batch if wl.kind == "decode" else 1)
    used: set[tuple[int, int]] = set()
    out = []
    for i in range(total):
        b = i % wl.batch
        for _attempt in range(1000):
            if wl.kind == "decode":
                t = wl.ctx
            else:
                lo_t = max(wl.ctx, BLOCK)   # a query with a complete block before its own
                if lo_t >= wl.ctx + wl.tq:
                    break
                t = int(rng.integers(lo_t, wl.ctx + wl.tq))
            own = t // BLOCK
            # with a cached prefix, prefill needles sit in blocks complete before the chunk
            hi_j = own if (wl.kind == "decode" or wl.ctx == 0) else min(own, wl.ctx // BLOCK)
            if hi_j <= 0:
                continue
            j = int(rng.integers(0, hi_j))
            if (b, j) in used:
                continue
            used.add((b, j))
            out.append((b, t, j))
            break
    needles = np.array(out, dtype=np.int64).reshape(-1, 3)
    plant_needles(q_idx, k_idx, q_pos0, needles)
    return needles


def plant_needles(q_idx: torch.Tensor, k_idx: torch.Tensor, q_pos0, needles) -> None:
    """Plant needles (b, t, j) in place: the 4 indexer keys of block j of
    sequence b become bf16(4 * u), u the unit vector along the sum of the 4
    indexer query heads of the token at position t (row t - q_pos0[b] of
    q_idx).  q_idx [B, tq, 4, 128] and k_idx [B, L, 128] are CPU bf16."""
    for b, t, j in np.asarray(needles, dtype=np.int64).reshape(-1, 3):
        row = q_idx[b, t - int(q_pos0[b])].to(torch.float64).sum(dim=0)
        u = row / row.norm()
        key = (4.0 * u).to(torch.bfloat16)
        k_idx[b, BLOCK * j: BLOCK * j + BLOCK, :] = key


def make_inputs(wl: Workload | str, threads: int | None = None) -> Inputs:
    """Draw the raw inputs of a workload (deterministic in wl.seed)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B, L, T = wl.batch, wl.length, wl.tq
    bf = torch.bfloat16
    q = torch.empty((B, T, HQ, D), dtype=bf)
    q_idx = torch.empty((B, T, HI, DI), dtype=bf)
    k = torch.empty((B, L, HKV, D), dtype=bf)
    v = torch.empty((B, L, HKV, D), dtype=bf)
    k_idx = torch.empty((B, L, DI), dtype=bf)
    sig_i = 1.0 / math.sqrt(DI)
    _fill_normal(q, wl.seed, _T_Q, 1.0, threads)
    _fill_normal(k, wl.seed, _T_K, 1.0, threads)
    _fill_normal(v, wl.seed, _T_V, 1.0, threads)
    _fill_normal(q_idx, wl.seed, _T_QI, sig_i, threads)
    _fill_normal(k_idx, wl.seed, _T_KI, sig_i, threads)
    q_pos0 = np.full((B,), wl.ctx, dtype=np.int32)
    needles = _plant_needles(wl, q_idx, k_idx, q_pos0)
    return Inputs(wl, q, q_idx, k, v, k_idx, q_pos0, needles)


def sample_rows(wl: Workload, n: int, seed: int = 99) -> list[tuple[int, int]]:
    """A seeded sample of (b, t) query rows of a workload, t absolute."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(wl.seed,))))
    rows = set()
    total = wl.batch * wl.tq
    n = min(n, total)
    while len(rows) < n:
        r = int(rng.integers(0, total))
        rows.add((r // wl.tq, wl.ctx + r % wl.tq))
    return sorted(rows)


# ---------------------------------------------------------------- Gated DeltaNet

GDN_HK, GDN_HV, GDN_D = 16, 48, 128   # model card "Model Overview": 16 Q/K heads, 48 V heads, dim 128
_T_GQ, _T_GK, _T_GV, _T_GG, _T_GB, _T_GS = range(10, 16)


@dataclass
class GdnInputs:
    """q, k [B, T, 16, 128] and v [B, T, 48, 128] bf16; g, beta [B, T, 48]
    float32; s0 [B, 48, 128, 128] float32 (all CPU tensors)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    s0: torch.Tensor


def make_gdn_inputs(batch: int, n_tokens: int, seed: int = 11, state_sigma: float = 0.1,
                    threads: int | None = None) -> GdnInputs:
    """Seeded synthetic inputs of the Gated DeltaNet token mixer: q, k, v
    N(0, 1) in bf16; g = -softplus(z - 3) and beta = sigmoid(z') with z, z'
    N(0, 1) (a decay exp(g) mostly between 0.9 and 1, writing strengths
    spread over (0, 1)), drawn in float32; an initial state N(0, state_sigma^2)."""
    B, T = batch, n_tokens
    bf = torch.bfloat16
    q = torch.empty((B, T, GDN_HK, GDN_D), dtype=bf)
    k = torch.empty_like(q)
    v = torch.empty((B, T, GDN_HV, GDN_D), dtype=bf)
    _fill_normal(q, seed, _T_GQ, 1.0, threads)
    _fill_normal(k, seed, _T_GK, 1.0, threads)
    _fill_normal(v, seed, _T_GV, 1.0, threads)
    zg = torch.empty((B, T, GDN_HV), dtype=torch.float32)
    zb = torch.empty_like(zg)
    s0 = torch.empty((B, GDN_HV, GDN_D, GDN_D), dtype=torch.float32)
    for t, tid, sig in ((zg, _T_GG, 1.0), (zb, _T_GB, 1.0), (s0, _T_GS, state_sigma)):
        flat = t.view(-1)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid,))))
        x = g.standard_normal(flat.numel(), dtype=np.float32)
        flat.copy_(torch.from_numpy(x * np.float32(sig)))
    g_log = -torch.nn.functional.softplus(zg - 3.0)
    beta = torch.sigmoid(zb)
    return GdnInputs(q, k, v, g_log, beta, s0)
