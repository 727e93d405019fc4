"""Shared helpers of the GPU parity tests: device set-up of a workload through
the HIP path, and the comparisons against the CPU oracle."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from block_sparse_long_12_amd import inputs as I
from block_sparse_long_12_amd import qsa
from oracle import qsa_oracle as O

# tolerances of the attention output (bf16 in, float32 accumulate)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return O.bits(t.detach().cpu())


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 units in the last place (sign-magnitude patterns)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def score_bound(q_idx_bits: np.ndarray, kbar_bits: np.ndarray) -> np.ndarray:
    """Worst-case float32 accumulation error of sum_{h,d} q[h,d] k[j,d] for
    512 exact products: 2^-15 * sum |q k| (n * 2^-24 with n = 512)."""
    q = np.abs(O.bf16_to_f64(q_idx_bits))           # [Hi, Di]
    k = np.abs(O.bf16_to_f64(kbar_bits))            # [n, Di]
    return (k @ q.sum(axis=0)) * 2.0 ** -15 + 1e-30


class DevicePrefill:
    """A prefill workload on the device, run through the HIP path."""

    def __init__(self, x: I.Inputs, rope=None):
        wl = x.workload
        self.x, self.wl, self.rope = x, wl, rope
        B, L, ctx, T = wl.batch, wl.length, wl.ctx, wl.tq
        dev = "cuda"
        self.q_raw = x.q.to(dev)
        self.k_new = x.k[:, ctx:].contiguous().to(dev)
        self.q_idx = x.q_idx.to(dev)
        self.k_idx = x.k_idx.to(dev)
        self.v_cache = x.v.to(dev)
        self.k_cache = x.k.to(dev)
        if ctx > 0:     # the cached prefix is stored rotated
            qsa.rope_apply(self.k_cache[:, :ctx], [0] * B, rope=rope)
        self.kbar = torch.zeros((B, max(1, L // 4), 128), dtype=torch.bfloat16, device=dev)
        if ctx // 4 > 0:
            qsa.compress_block_keys(self.k_idx, 0, ctx // 4, self.kbar)
        self.bufs = qsa.PrefillBuffers(B, T, ctx, wl.budget, wl.chunk)
        self.out = torch.empty((B, T, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, T, 24), dtype=torch.float32, device=dev)
        self.q_rot = torch.empty_like(self.q_raw)

    def run(self, gate=None):
        qsa.prefill_layer(self.q_raw, self.k_new, self.q_idx, self.k_idx, self.k_cache, self.v_cache,
                          self.kbar, self.wl.ctx, self.wl.budget, self.out, self.lse, self.bufs, self.q_rot,
                          gate=gate, rope=self.rope)
        torch.cuda.synchronize()


class DeviceDecode:
    """A decode workload on the device: caches prefilled, one new token."""

    def __init__(self, x: I.Inputs):
        wl = x.workload
        self.x, self.wl = x, wl
        B, ctx = wl.batch, wl.ctx
        dev = "cuda"
        self.pos = ctx
        self.k_cache = x.k.to(dev)
        qsa.rope_apply(self.k_cache[:, :ctx], [0] * B)
        self.v_cache = x.v.to(dev)
        self.k_idx = x.k_idx.to(dev)
        self.kbar = torch.zeros((B, max(1, (ctx + 1) // 4), 128), dtype=torch.bfloat16, device=dev)
        if ctx // 4 > 0:
            qsa.compress_block_keys(self.k_idx, 0, ctx // 4, self.kbar)
        self.q_raw = x.q.to(dev)                     # [B, 1, 24, 256]
        self.k_new = x.k[:, ctx:ctx + 1].contiguous().to(dev)
        self.q_idx = x.q_idx.to(dev)                 # [B, 1, 4, 128]
        ld = max(4, (ctx // 4 + 3) // 4 * 4)
        self.scores = torch.empty((B, 1, ld), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, 1, wl.budget), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
        self.ws = qsa.decode_step_workspace(B, wl.budget)

    def run(self):
        qsa.decode_step(self.q_raw, self.k_new, self.q_idx, self.k_idx, self.k_cache, self.v_cache, self.kbar,
                        self.pos, self.wl.budget, self.out, self.lse, self.scores, self.sel, self.ws)
        torch.cuda.synchronize()


def oracle_layer(x: I.Inputs, yarn: O.Yarn | None = None) -> O.OracleLayer:
    B = O.bits
    return O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, x.workload.budget,
                         yarn=yarn)


def compare_rows(layer: O.OracleLayer, x: I.Inputs, rows, gpu_scores, gpu_sel, gpu_out, gpu_lse):
    """The end-to-end protocol on query rows [(b, t)]:
      (i)   GPU scores within the float32 accumulation bound of the oracle's;
      (ii)  where GPU scores are given, the GPU selection is exactly the
            oracle's selection over those scores (select_blocks on the GPU's
            own float32 row); where the selected sets differ from the
            oracle's own, every swapped pair is a near tie (oracle scores
            within the two bounds);
      (iii) the GPU output equals the oracle's attention recomputed with the
            GPU's own selection (max-abs / mean-abs tolerances);
      (iv)  every planted needle of the row is selected.
    gpu_scores(b, t) -> float32 [o], gpu_sel(b, t) -> int32 [budget],
    gpu_out(b, t) -> float [24, 256], gpu_lse(b, t) -> float [24]."""
    ref = layer.rows(rows)
    needles = {}
    for b, t, j in x.needles:
        needles.setdefault((int(b), int(t)), []).append(int(j))
    swaps = 0
    override = {}
    worst_score = 0.0
    for (b, t), r in zip(rows, ref):
        o = t // 4
        sg = gpu_scores(b, t) if gpu_scores is not None else None
        kb = layer.kbar_bits(b)[:o]
        qb = layer.q_idx[b, t - layer.q_pos0[b]]
        bound = score_bound(qb, kb) if o > 0 else np.zeros(0)
        if sg is not None and o > 0:
            err = np.abs(sg.astype(np.float64) - r.scores.astype(np.float64))
            assert np.all(err <= bound), (b, t, float(err.max()), float(bound[np.argmax(err - bound)]))
            worst_score = max(worst_score, float((err / bound).max()))
        sgpu = gpu_sel(b, t)
        if sg is not None:
            exact = O.select_blocks(np.asarray(sg[:o], np.float32), t, layer.budget)
            assert np.array_equal(np.asarray(sgpu, np.int32), exact), (b, t, "selection of the GPU's own scores")
        A = set(int(v) for v in sgpu if v >= 0)
        Bs = set(int(v) for v in r.sel if v >= 0)
        assert len(A) == len(Bs) and o in A, (b, t)
        assert sorted(A) == [int(v) for v in sgpu[:len(A)]] and np.all(sgpu[len(A):] == -1), (b, t)
        if A != Bs:
            swaps += 1
            for a in A - Bs:
                for c in Bs - A:
                    gap = abs(float(r.scores[a]) - float(r.scores[c]))
                    assert gap <= bound[a] + bound[c], (b, t, a, c, gap)
        for j in needles.get((b, t), []):
            assert j in A, (b, t, j)
        override[(b, t)] = sgpu
    again = layer.rows(rows, sel_override=override)
    max_abs = 0.0
    sum_abs = 0.0
    n = 0
    lse_abs = 0.0
    for (b, t), r in zip(rows, again):
        go = gpu_out(b, t).astype(np.float64)
        d = np.abs(go - r.out)
        max_abs = max(max_abs, float(d.max()))
        sum_abs += float(d.sum())
        n += d.size
        lse_abs = max(lse_abs, float(np.abs(gpu_lse(b, t).astype(np.float64) - r.lse).max()))
    mean_abs = sum_abs / max(1, n)
    say(f"  rows={len(rows)} near-tie rows={swaps} worst score err/bound={worst_score:.3g} "
        f"max_abs={max_abs:.3g} mean_abs={mean_abs:.3g} lse_abs={lse_abs:.3g}")
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS and lse_abs <= LSE_ABS
    return swaps


def ragged_decode_inputs(pos, tq: int, seed: int, needles_per_seq: int = 3, share: int = 0) -> I.Inputs:
    """Seeded inputs of a decode step whose sequences sit at different
    positions: sequence b holds pos[b] cached rows and its tq new tokens at
    pos[b] .. pos[b] + tq - 1 (rows pos[b] + t of k, v, k_idx and row t of q,
    q_idx).  The first `share` rows of every sequence are sequence 0's (one
    shared prefix).  Needles: needles_per_seq blocks per sequence, each
    aligned to one of its new tokens, in blocks complete before that token."""
    B = len(pos)
    wl = I.custom_workload("prefill", batch=B, ctx=max(pos), tq=tq, budget=512, n_needles=0, seed=seed)
    x = I.make_inputs(wl)
    x.q_pos0 = np.asarray(pos, np.int32)
    rng = np.random.default_rng(seed)
    items = []
    for b in range(B):
        used = set()
        for i in range(needles_per_seq):
            t = int(pos[b]) + i % tq
            j = int(rng.integers(0, t // 4))
            if j in used or 4 * j + 4 <= share and b > 0:
                continue            # one needle per block; shared blocks belong to sequence 0
            used.add(j)
            items.append((b, t, j))
    x.needles = np.asarray(items, np.int64).reshape(-1, 3)
    I.plant_needles(x.q_idx, x.k_idx, x.q_pos0, x.needles)
    for b in range(1, B):       # after planting: the shared rows carry sequence 0's needles too
        x.k[b, :share], x.v[b, :share], x.k_idx[b, :share] = x.k[0, :share], x.v[0, :share], x.k_idx[0, :share]
    return x


class DeviceRaggedDecode:
    """Device caches of ragged_decode_inputs: sequence b's first pos[b] rows
    in place (K rotated, block keys of its complete blocks), every row from
    pos[b] on (those the step writes) and every later block key filled with
    garbage; new-token tensors [B, tq, ...]."""

    def __init__(self, x: I.Inputs, tq: int, rope=None):
        pos = [int(p) for p in x.q_pos0]
        B = len(pos)
        dev = "cuda"
        L = x.k.shape[1]
        self.pos, self.tq = pos, tq
        g = torch.Generator().manual_seed(12345)
        junk = lambda shape: (torch.randn(shape, generator=g) * 7).to(torch.bfloat16)
        k = junk(x.k.shape)
        v = junk(x.v.shape)
        ki = junk(x.k_idx.shape)
        for b in range(B):
            k[b, :pos[b]], v[b, :pos[b]], ki[b, :pos[b]] = x.k[b, :pos[b]], x.v[b, :pos[b]], x.k_idx[b, :pos[b]]
        self.k_cache, self.v_cache, self.k_idx = k.to(dev), v.to(dev), ki.to(dev)
        self.kbar = junk((B, L // 4 + 1, 128)).to(dev)
        for b in range(B):
            qsa.rope_apply(self.k_cache[b:b + 1, :pos[b]], [0], rope=rope)
            qsa.compress_block_keys(self.k_idx[b:b + 1], 0, pos[b] // 4, self.kbar[b:b + 1])
        sl = lambda t: torch.stack([t[b, pos[b]:pos[b] + tq] for b in range(B)]).contiguous().to(dev)
        self.k_new, self.v_new, self.k_idx_new = sl(x.k), sl(x.v), sl(x.k_idx)
        self.q_raw = x.q[:, :tq].contiguous().to(dev)
        self.q_idx = x.q_idx[:, :tq].contiguous().to(dev)
        self.ld = max(4, (max(p + tq - 1 for p in pos) // 4 + 3) // 4 * 4)
        self.scores = torch.full((B, tq, self.ld), float("nan"), device=dev)
        self.sel = torch.empty((B, tq, 512), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, tq, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)

    def results(self):
        """{(b, t): (scores [o], sel, out, lse)} of the step's rows."""
        sc, se = self.scores.cpu().numpy(), self.sel.cpu().numpy()
        ou, ls = self.out.float().cpu().numpy(), self.lse.cpu().numpy()
        res = {}
        for b, p in enumerate(self.pos):
            for t in range(self.tq):
                res[(b, p + t)] = (sc[b, t, :(p + t) // 4], se[b, t], ou[b, t], ls[b, t])
        return res


def compare_result_rows(layer: O.OracleLayer, x: I.Inputs, res: dict):
    """compare_rows over a {(b, t): (scores, sel, out, lse)} map."""
    rows = sorted(res)
    return compare_rows(layer, x, rows, lambda b, t: res[(b, t)][0], lambda b, t: res[(b, t)][1],
                        lambda b, t: res[(b, t)][2], lambda b, t: res[(b, t)][3])
