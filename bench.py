#!/usr/bin/env python
"""Benchmark of one Qwen Sparse Attention layer on one MI355X.

Prints ONE JSON line.  `value` is prefill throughput (new tokens/s) of the
1M-context chunked prefill (104858 new tokens after a 943718-token cached
prefix, the pages' 90% prefix-cache-hit setting), one step = every step of the
layer (rotary of the new Q/K rows, compression of the blocks they complete,
index scores, block selection and sparse attention for all 8192-query chunks).
The same line carries the 1M-context serving decode step (B=4, one new token
each: its K/V/indexer-key rows appended, scores, selection, attention) under
"decode", and the same step with 4 new tokens per sequence (the shape of
multi-token prediction or speculative verification) under
"decode_multi_token", and one sequence at the same context under
"decode_single_sequence".  Inputs are seeded synthetic tensors already resident
in HBM.  Rotary uses the model card's static YaRN table (factor 4 over 262144
positions), as contexts past 262144 call for; --rope plain selects the plain
table (the same work).

Timing: W untimed warm-up steps, then K steps between two device
synchronisations; per-kernel durations come from HIP events recorded on the
launch stream around every launch inside the timed steps.  Decode steps are
timed one by one after reading a 1 GiB buffer (outside the events), which
leaves the 256 MB last-level cache full of clean, unrelated lines, so the
k-bar scan reads HBM and pays no write-back of dirty lines.

Rooflines (MI355X published peaks): HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s.
`roofline` is the dominant prefill kernel (the sparse-attention gather);
`decode.roofline` the dominant decode kernel (the block-key scan).  Achieved
figures are algorithmic bytes (or flops) per launch over the measured average
launch time.  `cpu_baseline` is the CPU oracle timed on a sample of rows.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA prefill tokens/s + decode step µs at 1M ctx; % of MFMA / HBM roofline"
HBM_PEAK = 8.0e12
BF16_PEAK = 2.5e15


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="prefill_prefix943718_chunk104858")
    ap.add_argument("--decode-workload", default="decode_B4_ctx1M")
    ap.add_argument("--decode-steps", type=int, default=30)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-tq", type=int, default=4,
                    help="also time a decode step of this many new tokens per sequence (1 = skip)")
    ap.add_argument("--cpu-rows", type=int, default=512, help="oracle rows timed for cpu_baseline (0 = skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (2048-token prefill, 32K decode of 32 sequences, "
                         "131072-token prefill)")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet measurements")
    ap.add_argument("--serial", action="store_true",
                    help="prefill on one stream (index-select, then attention, per query chunk)")
    ap.add_argument("--gdn-tokens", type=int, default=104858, help="tokens of the Gated DeltaNet prefill")
    ap.add_argument("--page-tokens", type=int, default=256,
                    help="page size of the paged-cache measurements (0 = skip them)")
    ap.add_argument("--rope", choices=("yarn", "plain"), default="yarn",
                    help="rotary table: the model card's static YaRN (factor 4 over 262144, for contexts past "
                         "262144) or plain rotary")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill measurements (for counter runs of the decode kernels)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the calibration kernels of known traffic for the HBM byte counters: a 1 GiB "
                         "device copy and a gather of 2^21 random 512-byte rows from a 2 GiB buffer")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def calibrate(torch):
    """Kernels of known traffic for checking the memory-traffic counters
    (TCC_EA0_RDREQ_DRAM_32B / TCC_EA0_WRREQ_WRITE_DRAM_32B, and the derived
    FETCH_SIZE / WRITE_SIZE): a 1 GiB copy (reads and writes 2^30 bytes) and a gather of
    2^21 distinct random rows of 512 bytes out of a 2 GiB bf16 buffer (reads
    2^30 bytes of rows plus 2^24 bytes of int64 indices, writes 2^30 bytes;
    the shape of the attention's K/V row gathers)."""
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    buf = torch.ones((1 << 22, 256), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(3)
    idx = torch.randperm(1 << 22, generator=g, device="cuda")[: 1 << 21].contiguous()
    out = torch.empty((1 << 21, 256), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
        torch.index_select(buf, 0, idx, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": {
        "copy": {"read_bytes": 1 << 30, "write_bytes": 1 << 30, "kernel": "__amd_rocclr_copyBuffer"},
        "gather": {"read_bytes": (1 << 30) + (1 << 24), "write_bytes": 1 << 30,
                   "rows": 1 << 21, "row_bytes": 512, "source_bytes": 1 << 31,
                   "kernel": "torch index_select (index_elementwise_kernel)"}}}))


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload geometry

def attended_tokens(pos: int, budget: int) -> int:
    o = pos // 4
    return 4 * min(budget - 1, o) + (pos % 4) + 1


def prefill_geometry(wl, c0: int, c1: int):
    """Algorithmic bytes / flops of query rows [c0, c1) of a prefill chunk."""
    n_tok = 0
    cand = 0
    for i in range(c0, c1):
        p = wl.ctx + i
        n_tok += attended_tokens(p, wl.budget)
        cand += p // 4
    rows = (c1 - c0) * wl.batch
    n_tok *= wl.batch
    cand *= wl.batch
    return dict(
        rows=rows,
        gathered_tokens=n_tok,
        # K and V rows of both KV heads (2 x 2 x 256 bf16 = 2 KiB per token), Q read, O written
        attn_bytes=n_tok * 2 * 2 * 256 * 2 + rows * 24 * 256 * 2 * 2,
        attn_flops=n_tok * 24 * 256 * 2 * 2,
        candidates=cand,
        # folded minimum: 2 * 128 flop per (query, candidate); kbar read once, scores written
        index_flops=cand * 2 * 128,
        index_bytes_min=cand * 4,
    )


# ------------------------------------------------------------------ device set-up

class Prefill:
    def __init__(self, wl, x, torch, qsa, rope=None):
        B, L, ctx, T = wl.batch, wl.length, wl.ctx, wl.tq
        dev = "cuda"
        self.wl, self.qsa, self.torch, self.rope = wl, qsa, torch, rope
        self.q_raw = x.q.to(dev)
        self.k_new = x.k[:, ctx:].contiguous().to(dev)
        self.q_idx = x.q_idx.to(dev)
        self.k_idx = x.k_idx.to(dev)
        self.v_cache = x.v.to(dev)
        self.k_cache = x.k.to(dev)
        if ctx > 0:
            qsa.rope_apply(self.k_cache[:, :ctx], [0] * B, rope=rope)
        self.kbar = torch.zeros((B, max(1, L // 4), 128), dtype=torch.bfloat16, device=dev)
        if ctx // 4 > 0:
            qsa.compress_block_keys(self.k_idx, 0, ctx // 4, self.kbar)
        self.bufs = qsa.PrefillBuffers(B, T, ctx, wl.budget, wl.chunk)
        self.out = torch.empty((B, T, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, T, 24), dtype=torch.float32, device=dev)
        self.q_rot = torch.empty_like(self.q_raw)
        self.side = torch.cuda.Stream()      # default priority
        self.overlap = True
        torch.cuda.synchronize()

    def step(self, timer=None):
        """One layer step; `timer(name, stream)` returns a context that brackets launches with events.

        With `overlap` (the default) the index-selects of the query chunks run in
        order on a second stream and each chunk's attention waits only for its
        own selection, so the selection of chunk c + 1 (matrix-core bound)
        runs beside the attention of chunk c (HBM bound); the kernels and
        their results are the same as in the one-stream order."""
        wl, q, torch = self.wl, self.qsa, self.torch
        B, T, ctx = wl.batch, wl.tq, wl.ctx
        pos = [ctx] * B
        with timer("rope"):
            q.rope_apply(self.q_raw, pos, out=self.q_rot, rope=self.rope)
            q.rope_apply(self.k_new, pos, out=self.k_cache[:, ctx:ctx + T], rope=self.rope)
        with timer("compress"):
            q.compress_block_keys(self.k_idx, ctx // 4, (ctx + T) // 4, self.kbar)
        ch = self.bufs.chunk
        chunks = [(c0, min(T, c0 + ch)) for c0 in range(0, T, ch)]
        if not self.overlap:
            for c0, c1 in chunks:
                cpos = [ctx + c0] * B
                with timer("index_select"):
                    q.index_select_prefill(self.q_idx[:, c0:c1], self.kbar, cpos, wl.budget, self.bufs.scores,
                                           self.bufs.sel[:, c0:c1], self.bufs.workspace)
                with timer("sparse_attn_prefill"):
                    q.sparse_attn_prefill(self.q_rot[:, c0:c1], self.k_cache, self.v_cache,
                                          self.bufs.sel[:, c0:c1], cpos, self.out[:, c0:c1], self.lse[:, c0:c1])
            return
        main = torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record(main)
        self.side.wait_event(ready)                  # block keys compressed
        done = []
        for c0, c1 in chunks:
            with timer("index_select", self.side):
                q.index_select_prefill(self.q_idx[:, c0:c1], self.kbar, [ctx + c0] * B, wl.budget,
                                       self.bufs.scores, self.bufs.sel[:, c0:c1], self.bufs.workspace,
                                       stream=self.side)
            e = torch.cuda.Event()
            e.record(self.side)
            done.append(e)
        for (c0, c1), e in zip(chunks, done):
            main.wait_event(e)
            with timer("sparse_attn_prefill"):
                q.sparse_attn_prefill(self.q_rot[:, c0:c1], self.k_cache, self.v_cache, self.bufs.sel[:, c0:c1],
                                      [ctx + c0] * B, self.out[:, c0:c1], self.lse[:, c0:c1])
        main.wait_stream(self.side)


def random_pages(torch, B, n_log, seed):
    """A block table naming distinct pages in a random order."""
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(B * n_log, generator=g).to(torch.int32).view(B, n_log)


class PagedPrefill:
    """The prefill workload on a paged cache: the cached prefix (rotated K,
    V, indexer keys, block keys) copied into pages of P tokens in a random
    order; a step appends the chunk's rows (paged_append) and runs the fused
    index-select and attention through the block table."""

    def __init__(self, pf, P, seed=5):
        torch, qsa, wl = pf.torch, pf.qsa, pf.wl
        B, L, ctx = wl.batch, wl.length, wl.ctx
        self.pf, self.torch, self.qsa, self.wl = pf, torch, qsa, wl
        n_log = (L + P - 1) // P
        self.cache = qsa.PagedCache(B * n_log, P, B, n_log)
        self.cache.table.copy_(random_pages(torch, B, n_log, seed))
        for b in range(B):
            self.cache.write_contiguous(b, ctx, k=pf.k_cache[b], v=pf.v_cache[b], k_idx=pf.k_idx[b],
                                        kbar=pf.kbar[b])
        self.v_new = pf.v_cache[:, ctx:].contiguous()
        self.k_idx_new = pf.k_idx[:, ctx:].contiguous()
        self.bufs = qsa.PrefillBuffers(B, wl.tq, ctx, wl.budget, wl.chunk)
        torch.cuda.synchronize()

    def step(self, timer=None):
        wl, q, pf = self.wl, self.qsa, self.pf
        B, T, ctx = wl.batch, wl.tq, wl.ctx
        pos = [ctx] * B
        with timer("rope"):
            q.rope_apply(pf.q_raw, pos, out=pf.q_rot, rope=pf.rope)
        with timer("paged_append"):
            q.paged_append(self.cache, pos, k_new=pf.k_new, v_new=self.v_new, k_idx_new=self.k_idx_new,
                           rope=pf.rope)
        ch = self.bufs.chunk
        chunks = [(c0, min(T, c0 + ch)) for c0 in range(0, T, ch)]
        torch = self.torch
        side = pf.side if pf.overlap else torch.cuda.current_stream()
        main = torch.cuda.current_stream()
        if pf.overlap:                               # the same two-stream order as Prefill.step
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
        done = []
        for c0, c1 in chunks:
            with timer("index_select", side):
                q.index_select_prefill_paged(pf.q_idx[:, c0:c1], self.cache, [ctx + c0] * B, wl.budget,
                                             self.bufs.scores, self.bufs.sel[:, c0:c1], self.bufs.workspace,
                                             stream=side)
            e = torch.cuda.Event()
            e.record(side)
            done.append(e)
            if not pf.overlap:
                self._attend(timer, c0, c1)
        if pf.overlap:
            for (c0, c1), e in zip(chunks, done):
                main.wait_event(e)
                self._attend(timer, c0, c1)
            main.wait_stream(side)

    def _attend(self, timer, c0, c1):
        pf, wl = self.pf, self.wl
        with timer("sparse_attn_prefill"):
            self.qsa.sparse_attn_prefill_paged(pf.q_rot[:, c0:c1], self.cache, self.bufs.sel[:, c0:c1],
                                               [wl.ctx + c0] * wl.batch, pf.out[:, c0:c1], pf.lse[:, c0:c1])


class Decode:
    def __init__(self, wl, x, torch, qsa, rope=None):
        B, ctx = wl.batch, wl.ctx
        dev = "cuda"
        self.wl, self.qsa, self.torch, self.rope = wl, qsa, torch, rope
        self.pos = ctx
        # caches with room for up to 4 new tokens (the multi-token step)
        L = ctx + 4
        self.k_cache = torch.zeros((B, L, 2, 256), dtype=torch.bfloat16, device=dev)
        self.k_cache[:, :ctx + 1].copy_(x.k)
        qsa.rope_apply(self.k_cache[:, :ctx], [0] * B, rope=rope)
        self.v_cache = torch.zeros_like(self.k_cache)
        self.v_cache[:, :ctx + 1].copy_(x.v)
        self.k_idx = torch.zeros((B, L, 128), dtype=torch.bfloat16, device=dev)
        self.k_idx[:, :ctx + 1].copy_(x.k_idx)
        self.kbar = torch.zeros((B, L // 4 + 1, 128), dtype=torch.bfloat16, device=dev)
        qsa.compress_block_keys(self.k_idx, 0, ctx // 4, self.kbar)
        self.q_raw = x.q.to(dev)
        self.k_new = x.k[:, ctx:ctx + 1].contiguous().to(dev)
        self.v_new = x.v[:, ctx:ctx + 1].contiguous().to(dev)
        self.k_idx_new = x.k_idx[:, ctx:ctx + 1].contiguous().to(dev)
        self.q_idx = x.q_idx.to(dev)
        ld = max(4, (ctx // 4 + 3) // 4 * 4)
        self.scores = torch.empty((B, 1, ld), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, 1, wl.budget), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
        self.ws = qsa.decode_step_workspace(B, wl.budget)
        torch.cuda.synchronize()

    def multi_setup(self, tq: int, seed: int = 77):
        """Synthetic rows of tq new tokens per sequence (same distributions as
        the workload's): the shape of a multi-token prediction or speculative
        verification step."""
        torch, qsa = self.torch, self.qsa
        B, dev, bf = self.wl.batch, "cuda", torch.bfloat16
        g = torch.Generator().manual_seed(seed)
        self.m_tq = tq
        self.m_q = torch.randn((B, tq, 24, 256), generator=g).to(bf).to(dev)
        self.m_q_idx = (torch.randn((B, tq, 4, 128), generator=g) / 128 ** 0.5).to(bf).to(dev)
        self.m_k = torch.randn((B, tq, 2, 256), generator=g).to(bf).to(dev)
        self.m_v = torch.randn((B, tq, 2, 256), generator=g).to(bf).to(dev)
        self.m_k_idx = (torch.randn((B, tq, 128), generator=g) / 128 ** 0.5).to(bf).to(dev)
        ld = self.scores.shape[-1] + 4
        self.m_scores = torch.empty((B, tq, ld), dtype=torch.float32, device=dev)
        self.m_sel = torch.empty((B, tq, self.wl.budget), dtype=torch.int32, device=dev)
        self.m_out = torch.empty((B, tq, 24, 256), dtype=bf, device=dev)
        self.m_lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)
        self.m_ws = qsa.decode_step_workspace(B, self.wl.budget, tq=tq)

    def multi_step(self):
        self.qsa.decode_step(self.m_q, self.m_k, self.m_q_idx, self.k_idx, self.k_cache, self.v_cache, self.kbar,
                             self.pos, self.wl.budget, self.m_out, self.m_lse, self.m_scores, self.m_sel, self.m_ws,
                             v_new=self.m_v, k_idx_new=self.m_k_idx, rope=self.rope)

    def paged_setup(self, P, seed=9):
        """The same caches copied into pages of P tokens in a random order."""
        torch, qsa, wl = self.torch, self.qsa, self.wl
        B, L = wl.batch, self.k_cache.shape[1]
        n_log = (L + P - 1) // P
        self.cache = qsa.PagedCache(B * n_log, P, B, n_log)
        self.cache.table.copy_(random_pages(torch, B, n_log, seed))
        for b in range(B):
            self.cache.write_contiguous(b, self.pos, k=self.k_cache[b], v=self.v_cache[b], k_idx=self.k_idx[b],
                                        kbar=self.kbar[b])
        torch.cuda.synchronize()

    def paged_step(self):
        self.qsa.decode_step_paged(self.q_raw, self.k_new, self.q_idx, self.cache, self.pos, self.wl.budget,
                                   self.out, self.lse, self.scores, self.sel, self.ws, v_new=self.v_new,
                                   k_idx_new=self.k_idx_new, rope=self.rope)

    def step(self, timer):
        """One serving decode step through the single qsa_decode_step call: the
        new token's K (rotated), V and indexer-key rows appended to the caches,
        block scores, selection, attention with q rotated on load (a block
        completed by the new token would be compressed in the same call)."""
        wl, q = self.wl, self.qsa
        with timer("decode_step"):
            q.decode_step(self.q_raw, self.k_new, self.q_idx, self.k_idx, self.k_cache, self.v_cache, self.kbar,
                          self.pos, wl.budget, self.out, self.lse, self.scores, self.sel, self.ws,
                          v_new=self.v_new, k_idx_new=self.k_idx_new, rope=self.rope)


class EventTimer:
    """Records a start/end HIP event pair on the current stream around each
    bracketed group of launches; durations are read after synchronising."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []          # (name, start, end)

    def __call__(self, name, stream=None):
        timer = self

        class _Ctx:
            def __enter__(self_inner):
                self_inner.s = timer.torch.cuda.Event(enable_timing=True)
                self_inner.s.record(stream)

            def __exit__(self_inner, *exc):
                e = timer.torch.cuda.Event(enable_timing=True)
                e.record(stream)
                timer.pairs.append((name, self_inner.s, e))
                return False

        return _Ctx()

    def totals(self):
        out = {}
        for name, s, e in self.pairs:
            ms = s.elapsed_time(e)
            tot, n = out.get(name, (0.0, 0))
            out[name] = (tot + ms, n + 1)
        return out


class NullTimer:
    def __call__(self, name, stream=None):
        class _Ctx:
            def __enter__(self):
                return None

            def __exit__(self, *exc):
                return False
        return _Ctx()


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)


def source_hash(*names) -> str:
    """Hash of kernel sources with comments removed and blank space collapsed,
    so that a counter record stays attached to the code it measured."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_12_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        code = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, src: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(src):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline

def cpu_info():
    """The host the oracle runs on: logical CPUs, those this process may use,
    and the CPU model."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable": usable, "model": model}


_ORACLE = {}


def _oracle_rows(rows):
    """Worker of the oracle pool: the layer (inherited at fork) on some rows,
    one BLAS thread; returns the seconds it took."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        _ORACLE["layer"].rows(rows)
        return time.perf_counter() - t0


def cpu_baseline(wl, x, n_rows: int, args, workers: int):
    """The oracle (oracle/qsa_oracle.py, numpy float64, as it stands) on a
    seeded sample of rows of a workload: block keys of the whole context once,
    then the rows on one core and on a pool of `workers` processes (one BLAS
    thread each), each extrapolated to the whole workload."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from block_sparse_long_12_amd import inputs as I
    from oracle import qsa_oracle as O
    rows = I.sample_rows(wl, n_rows)
    B = O.bits
    with threadpool_limits(limits=1):
        layer = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget,
                              yarn=O.Yarn() if args.rope == "yarn" else None)
        t0 = time.perf_counter()
        for b in sorted({r[0] for r in rows}):
            layer.kbar_bits(b)
        t_setup = time.perf_counter() - t0
    _ORACLE["layer"] = layer
    n1 = max(1, len(rows) // 8)
    t_one = _oracle_rows(rows[:n1]) / n1                  # seconds per row on one core
    parts = [rows[i::workers] for i in range(workers)]
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_rows, parts)
        t_pool = (time.perf_counter() - t0) / len(rows)   # wall seconds per row on the pool
    _ORACLE.clear()
    total_rows = wl.batch * wl.tq
    prefill = wl.kind == "prefill"
    # a prefill step compresses its chunk's blocks; a decode step finds the
    # block keys cached (as the GPU step does), so its time is the rows' alone
    setup = t_setup if prefill else 0.0
    full_pool = setup + t_pool * total_rows
    full_one = setup + t_one * total_rows
    log(args, f"cpu oracle {wl.name}: {len(rows)} rows, {t_one * 1e3:.1f} ms/row on one core, "
              f"{t_pool * 1e3:.2f} ms/row on {workers} processes (+{t_setup:.2f}s block keys)")
    return {
        "value": total_rows / full_pool if prefill else full_pool * 1e6,
        "unit": "tokens/s" if prefill else "us/step",
        "cores": workers,
        "kind": "oracle",
        "single_core": total_rows / full_one if prefill else full_one * 1e6,
        "host": cpu_info(),
        "sample": f"{len(rows)} seeded query rows of {wl.name} on {workers} processes ({n1} of them also on one "
                  f"core), numpy float64, one BLAS thread per process; block keys of the whole context "
                  f"compressed once ({t_setup:.2f}s{'' if prefill else ', not counted: cached in a decode step'}); "
                  f"extrapolated to the {total_rows} rows of a step",
    }


def oracle_workers():
    """Processes for the oracle pool: the CPUs this process may use, at most 16."""
    return max(1, min(16, cpu_info()["usable"]))


# ------------------------------------------------------------------ main

def achievable_peaks(torch):
    """Context for the rooflines (not the kernels here): a 1 GiB device copy
    (read + write bytes over time) and a 8192^3 bf16 matrix product through
    torch's library GEMM, each the best of 5 after a warm-up."""
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    x = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    y = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(5):
            s_ev = torch.cuda.Event(enable_timing=True)
            e_ev = torch.cuda.Event(enable_timing=True)
            s_ev.record()
            fn()
            e_ev.record()
            torch.cuda.synchronize()
            t.append(s_ev.elapsed_time(e_ev) / 1e3)
        return min(t)

    t_copy = best(lambda: b.copy_(a))
    t_mm = best(lambda: torch.matmul(x, y))
    res = {"hbm_copy_GBs": 2 * a.numel() * 4 / t_copy / 1e9,
           "bf16_gemm_TFLOPs": 2 * 8192 ** 3 / t_mm / 1e12,
           "note": "measured context: 1 GiB device copy; 8192^3 bf16 torch.matmul"}
    del a, b, x, y
    torch.cuda.empty_cache()
    return res


def gdn_measure(args, torch, qsa, I):
    """The Gated DeltaNet token mixer of the other 3 of 4 layers: a prefill
    of --gdn-tokens tokens (one sequence, the new-token count of the QSA
    prefill) and a decode step of 4 sequences, on seeded synthetic inputs."""
    T, Bd = args.gdn_tokens, 4
    x = I.make_gdn_inputs(1, T, seed=3)
    q, k, v, g, beta = (t.cuda() for t in (x.q, x.k, x.v, x.g, x.beta))
    state = x.s0.cuda()
    out = torch.empty_like(v)
    ws = qsa.gdn_prefill_workspace(1, T)
    for _ in range(args.warmup):
        qsa.gdn_prefill(q, k, v, g, beta, state, out, ws)
    torch.cuda.synchronize()
    t_ms = []
    for _ in range(max(1, args.steps)):
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        s_ev.record()
        qsa.gdn_prefill(q, k, v, g, beta, state, out, ws)
        e_ev.record()
        torch.cuda.synchronize()
        t_ms.append(s_ev.elapsed_time(e_ev))
    t_ms.sort()
    pre_ms = t_ms[len(t_ms) // 2]
    # algorithmic bytes: q, k, v, g, beta read and o written once, the state read and written once
    io = T * (2 * 16 * 128 * 2 + 48 * 128 * 2 * 2 + 48 * 4 * 2) + 2 * 48 * 128 * 128 * 4
    del x, q, k, v, g, beta, out, ws, state
    torch.cuda.empty_cache()
    xd = I.make_gdn_inputs(Bd, 1, seed=4)
    dq, dk, dv, dg, db = (t[:, 0].contiguous().cuda() for t in (xd.q, xd.k, xd.v, xd.g, xd.beta))
    dstate = xd.s0.cuda()
    dout = torch.empty_like(dv)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(3):
        qsa.gdn_decode(dq, dk, dv, dg, db, dstate, dout)
    d_ms = []
    for _ in range(args.decode_steps):
        flush.sum()
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        s_ev.record()
        qsa.gdn_decode(dq, dk, dv, dg, db, dstate, dout)
        e_ev.record()
        torch.cuda.synchronize()
        d_ms.append(s_ev.elapsed_time(e_ev))
    d_ms.sort()
    dec_us = d_ms[len(d_ms) // 2] * 1e3
    dec_bytes = Bd * (2 * 48 * 128 * 128 * 4 + 2 * 16 * 128 * 2 + 2 * 48 * 128 * 2 + 2 * 48 * 4)
    del flush
    torch.cuda.empty_cache()
    res = {
        "prefill": {"workload": f"gdn_prefill_B1_T{T}", "ms": pre_ms, "tokens_per_s": T / (pre_ms / 1e3),
                    "algorithmic_bytes": io, "hbm_frac": io / (pre_ms / 1e3) / HBM_PEAK,
                    "bound": "latency of the chunk-sequential state pass (192 workgroups)"},
        "decode": {"workload": f"gdn_decode_B{Bd}", "step_us_median": dec_us, "step_us_min": d_ms[0] * 1e3,
                   "algorithmic_bytes": dec_bytes, "hbm_frac": dec_bytes / (dec_us / 1e6) / HBM_PEAK,
                   "cache_flushed": True},
        "data": "synthetic: q, k, v N(0,1) bf16; g = -softplus(z - 3), beta = sigmoid(z'); state N(0, 0.01)",
    }
    log(args, f"gdn: prefill {pre_ms:.2f} ms ({T / pre_ms * 1e3:.0f} tok/s), decode {dec_us:.1f} us")
    return res


def time_steps(torch, fn, n, flush=None):
    """Event times (ms) of n calls of fn on the current stream, sorted; with
    flush, a read of that buffer before each call evicts the caches."""
    ts = []
    for _ in range(n):
        if flush is not None:
            flush.sum()
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        s_ev.record()
        fn()
        e_ev.record()
        torch.cuda.synchronize()
        ts.append(s_ev.elapsed_time(e_ev))
    ts.sort()
    return ts


def measure_prefill(args, torch, qsa, wl, x, rope, steps, warmup, paged=False):
    """Times `steps` whole prefill steps of a workload (after `warmup`):
    rotary, compress, then per query chunk the fused index-select and the
    attention (two streams unless --serial).  Returns the record and the
    Prefill object."""
    pf = Prefill(wl, x, torch, qsa, rope)
    pf.overlap = not args.serial
    for _ in range(warmup):
        pf.step(NullTimer())
    torch.cuda.synchronize()
    timer = EventTimer(torch)
    t_start = time.perf_counter()
    for _ in range(steps):
        pf.step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    kern = timer.totals()
    ms_per_step = wall * 1e3 / steps
    tokens = wl.batch * wl.tq
    geo = prefill_geometry(wl, 0, wl.tq)
    n_chunks = math.ceil(wl.tq / (wl.chunk or wl.tq))
    attn_ms, attn_n = kern["sparse_attn_prefill"]
    attn_avg_s = attn_ms / attn_n / 1e3
    attn_bytes_per_launch = geo["attn_bytes"] / n_chunks
    idx_ms, idx_n = kern["index_select"]
    rec = {
        "ms_per_step": ms_per_step,
        "tokens_per_s": tokens / (ms_per_step / 1e3),
        "attention": {"kernel": "sparse_attn_prefill", "ms_per_launch": attn_avg_s * 1e3,
                      "algorithmic_bytes_per_launch": attn_bytes_per_launch,
                      "gather_GBs": attn_bytes_per_launch / attn_avg_s / 1e9,
                      "hbm_frac": attn_bytes_per_launch / attn_avg_s / HBM_PEAK},
        "mfma": {
            "index_select_frac": (geo["index_flops"] / n_chunks) / (idx_ms / idx_n / 1e3) / BF16_PEAK,
            "layer_frac": (geo["index_flops"] + geo["attn_flops"]) / (ms_per_step / 1e3) / BF16_PEAK,
            "note": "folded indexer minimum (2*128 flop per query-candidate pair) plus attention flops, "
                    "over event time, against 2.5 PFLOP/s",
        },
        "kernels_ms_per_step": {k: t / steps for k, (t, n) in kern.items()},
        "launches_per_step": {k: n // steps for k, (t, n) in kern.items()},
        "gpu_ms_per_step": sum(t for t, _ in kern.values()) / steps,
        "gather_bytes_per_step": geo["gathered_tokens"] * 2 * 2 * 256 * 2,
    }
    log(args, f"prefill {wl.name}: {ms_per_step:.1f} ms/step, {rec['tokens_per_s']:.0f} tok/s; "
              f"kernels {rec['kernels_ms_per_step']}")
    if paged and args.page_tokens > 0:
        pp = PagedPrefill(pf, args.page_tokens)
        for _ in range(warmup):
            pp.step(NullTimer())
        torch.cuda.synchronize()
        ptimer = EventTimer(torch)
        t_start = time.perf_counter()
        for _ in range(steps):
            pp.step(ptimer)
        torch.cuda.synchronize()
        p_ms = (time.perf_counter() - t_start) * 1e3 / steps
        pk = ptimer.totals()
        pa_ms, pa_n = pk["sparse_attn_prefill"]
        rec["paged"] = {
            "page_tokens": args.page_tokens,
            "pages": "random page order, the cached prefix copied in before timing",
            "ms_per_step": p_ms,
            "tokens_per_s": tokens / (p_ms / 1e3),
            "kernels_ms_per_step": {k: t / steps for k, (t, n) in pk.items()},
            "sparse_attn_prefill_hbm_frac": attn_bytes_per_launch / (pa_ms / pa_n / 1e3) / HBM_PEAK,
            "note": "paged_append also copies the chunk's V and indexer-key rows into their pages",
        }
        log(args, f"prefill {wl.name}, paged: {p_ms:.1f} ms/step; kernels {rec['paged']['kernels_ms_per_step']}")
        del pp
    return rec, pf


def decode_bytes(wl, tq=1):
    """Algorithmic bytes of one decode step: the candidate block keys, the
    K/V rows of the selected blocks (both KV heads), q read and out written,
    the selection written."""
    o = wl.ctx // 4
    kbar = wl.batch * (o * 128 * 2 + 4 * 128 * 2)
    gather = wl.batch * sum(attended_tokens(wl.ctx + t, wl.budget) for t in range(tq)) * 2 * 2 * 256 * 2
    return kbar, kbar + gather + wl.batch * tq * (24 * 256 * 2 * 2 + wl.budget * 4)


def measure_decode(args, torch, qsa, I, dwl, rope, extras=True):
    """The serving decode step of a workload (one qsa_decode_step call per
    step, caches evicted between steps by reading 1 GiB), its fused
    index-select alone, and (extras) the 4-token step and the paged step."""
    t0 = time.time()
    dx = I.make_inputs(dwl)
    log(args, f"inputs {dwl.name}: {time.time() - t0:.1f}s")
    dd = Decode(dwl, dx, torch, qsa, rope)
    del dx
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(3):
        dd.step(NullTimer())
    torch.cuda.synchronize()
    steps_ms = time_steps(torch, lambda: dd.step(NullTimer()), args.decode_steps, flush)
    med = steps_ms[len(steps_ms) // 2]
    # the dominant kernels alone: the fused index-select (block-key scan and
    # the selection), same launch configuration as inside the step
    sel_ws = qsa.index_select_workspace(dwl.batch)
    # rows that leave the candidate lists for the exact path (diagnostic hook)
    exact_rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    qsa.set_decode_fallback_counter(exact_rows)
    try:
        idx_ms = time_steps(torch, lambda: qsa.index_select_decode(dd.q_idx, dd.kbar, [dd.pos] * dwl.batch,
                                                                   dwl.budget, dd.scores, dd.sel, sel_ws),
                            args.decode_steps, flush)
    finally:
        qsa.set_decode_fallback_counter(None)
    idx_avg = sum(idx_ms) / len(idx_ms) / 1e3
    # the block-key scan alone, the dominant kernel: events the library records
    # on the call's stream right before and after the scan launch
    ev_b, ev_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_b.record()
    ev_e.record()
    torch.cuda.synchronize()
    qsa.set_scan_timing_events(ev_b, ev_e)
    scan_ms = []
    try:
        for _ in range(args.decode_steps):
            flush.sum()
            qsa.index_select_decode(dd.q_idx, dd.kbar, [dd.pos] * dwl.batch, dwl.budget, dd.scores, dd.sel, sel_ws)
            torch.cuda.synchronize()
            scan_ms.append(ev_b.elapsed_time(ev_e))
    finally:
        qsa.set_scan_timing_events(None, None)
    scan_avg = sum(scan_ms) / len(scan_ms) / 1e3
    kbar_bytes, step_bytes = decode_bytes(dwl)
    rec = {
        "workload": dwl.name,
        "batch": dwl.batch,
        "context": dwl.ctx,
        "budget_blocks": dwl.budget,
        "step_us_median": med * 1e3,
        "step_us_min": steps_ms[0] * 1e3,
        "steps": args.decode_steps,
        "cache_flushed": True,
        "hbm_frac_step": step_bytes / (med / 1e3) / HBM_PEAK,
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_scan_kernel (the block-key scan of qsa_index_select_decode)",
            "achieved": kbar_bytes / scan_avg / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": kbar_bytes / scan_avg / HBM_PEAK,
            "launch_us": scan_avg * 1e6,
            "traffic": measured_traffic("decode_scan", "decode.hip"),
        },
        "index_select": {
            "kernels": "decode_scan_kernel + decode_finalize_kernel",
            "call_us": idx_avg * 1e6,
            "hbm_frac": kbar_bytes / idx_avg / HBM_PEAK,
            "exact_path_rows": int(exact_rows.item()),
            "rows_selected": dwl.batch * len(idx_ms),
        },
    }
    log(args, f"decode {dwl.name}: median {med * 1e3:.1f} us/step; index-select {idx_avg * 1e6:.1f} us, "
              f"its scan {scan_avg * 1e6:.1f} us")
    if extras and args.decode_tq > 1:
        # tq new tokens per sequence in one step: one pass over the block
        # keys scores all of them; each row has its own selection and attention
        mt = args.decode_tq
        dd.multi_setup(mt)
        for _ in range(3):
            dd.multi_step()
        torch.cuda.synchronize()
        m_ms = time_steps(torch, dd.multi_step, args.decode_steps, flush)
        m_med = m_ms[len(m_ms) // 2]
        _, m_bytes = decode_bytes(dwl, mt)
        rec["multi_token"] = {
            "tokens_per_sequence": mt,
            "step_us_median": m_med * 1e3,
            "step_us_min": m_ms[0] * 1e3,
            "us_per_token": m_med * 1e3 / (dwl.batch * mt),
            "single_token_us_per_token": med * 1e3 / dwl.batch,
            "hbm_frac_step": m_bytes / (m_med / 1e3) / HBM_PEAK,
            "algorithmic_bytes_per_step": m_bytes,
            "data": "synthetic new-token rows of the workload's distributions",
        }
        log(args, f"decode {dwl.name}, {mt} tokens per sequence: median {m_med * 1e3:.1f} us/step")
    if extras and args.page_tokens > 0:
        dd.paged_setup(args.page_tokens)
        for _ in range(3):
            dd.paged_step()
        torch.cuda.synchronize()
        p_ms = time_steps(torch, dd.paged_step, args.decode_steps, flush)
        p_med = p_ms[len(p_ms) // 2]
        rec["paged"] = {
            "page_tokens": args.page_tokens,
            "pages": "random page order",
            "step_us_median": p_med * 1e3,
            "step_us_min": p_ms[0] * 1e3,
            "hbm_frac_step": step_bytes / (p_med / 1e3) / HBM_PEAK,
        }
        log(args, f"decode {dwl.name}, paged: median {p_med * 1e3:.1f} us/step")
    del dd, flush
    torch.cuda.empty_cache()
    return rec


def summary_prefill(r):
    return {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
            "mfma_frac": r["mfma"]["layer_frac"], "index_select_mfma_frac": r["mfma"]["index_select_frac"],
            "gather_GBs": r["attention"]["gather_GBs"], "attention_hbm_frac": r["attention"]["hbm_frac"],
            "kernels_ms_per_step": r["kernels_ms_per_step"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus N with N > 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from block_sparse_long_12_amd import inputs as I
    from block_sparse_long_12_amd import qsa
    if not os.path.exists(qsa.LIB_PATH):
        from block_sparse_long_12_amd import build as _b
        _b.build()
    qsa.lib()
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.calibrate:
        calibrate(torch)
        return
    rope = qsa.YARN if args.rope == "yarn" else None
    wl = I.WORKLOADS[args.workload]
    rec = {
        "metric": METRIC,
        "value": None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "new_tokens": wl.tq, "cached_tokens": wl.ctx,
                   "context": wl.length, "budget_blocks": wl.budget, "block_tokens": 4,
                   "query_chunk": wl.chunk, "heads": "24q/2kv x 256, indexer 4q/1k x 128",
                   "rope": "static YaRN, factor 4 over 262144" if args.rope == "yarn" else "plain, theta 1e7"},
    }
    x = None
    if not args.no_prefill:
        t0 = time.time()
        x = I.make_inputs(wl)
        log(args, f"inputs {wl.name}: {time.time() - t0:.1f}s")
        pre, pf = measure_prefill(args, torch, qsa, wl, x, rope, args.steps, args.warmup, paged=True)
        del pf
        torch.cuda.empty_cache()
        a = pre["attention"]
        rec["value"] = pre["tokens_per_s"]
        rec["ms_per_step"] = pre["ms_per_step"]
        rec["roofline"] = {
            "bound": "hbm",
            "kernel": "sparse_attn_prefill",
            "achieved": a["gather_GBs"],
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": a["hbm_frac"],
            "traffic": measured_traffic("sparse_attn_prefill", "attention.hip"),
        }
        rec["schedule"] = ("one stream: per query chunk the index-select, then attention" if args.serial else
                           "two streams: the query chunks' index-selects in order on a second stream, each "
                           "chunk's attention after its own selection (kernel times overlap, so they sum past "
                           "ms_per_step)")
        for k in ("mfma", "kernels_ms_per_step", "launches_per_step", "gpu_ms_per_step", "gather_bytes_per_step"):
            rec[k] = pre[k]
        if "paged" in pre:
            rec["prefill_paged"] = pre["paged"]

    if not args.no_decode:
        dec = measure_decode(args, torch, qsa, I, I.WORKLOADS[args.decode_workload], rope)
        for k, dst in (("multi_token", "decode_multi_token"), ("paged", "decode_paged")):
            if k in dec:
                rec[dst] = dec.pop(k)
        rec["decode"] = dec
        # one sequence at the same context (the scan plan gives it longer
        # candidate lists instead of fewer workgroups)
        w = I.WORKLOADS[args.decode_workload]
        w1 = I.custom_workload("decode", 1, w.ctx, 1, w.budget, n_needles=w.n_needles, seed=w.seed)
        d1 = measure_decode(args, torch, qsa, I, w1, rope, extras=False)
        rec["decode_single_sequence"] = {k: d1[k] for k in ("workload", "step_us_median", "step_us_min",
                                                            "hbm_frac_step", "algorithmic_bytes_per_step")}
        rec["decode_single_sequence"]["index_select"] = d1["index_select"]
        rec["decode_single_sequence"]["scan_us"] = d1["roofline"]["launch_us"]
        torch.cuda.empty_cache()

    if not args.no_configs:
        # the other configurations: the 2048-token prefill, the 32K-context
        # decode of 32 sequences, the 131072-token prefill in 8192-query chunks
        cfg = {}
        w0 = I.WORKLOADS["prefill_T2048_budget64"]
        r0, _ = measure_prefill(args, torch, qsa, w0, I.make_inputs(w0), None, 20, 3)
        cfg[w0.name] = summary_prefill(r0)
        cfg[w0.name]["note"] = "the 4 MiB of K/V stay in the L2 and MALL: gather_GBs is mostly cache bandwidth"
        w1 = I.WORKLOADS["decode_B32_ctx32K"]
        d1 = measure_decode(args, torch, qsa, I, w1, None, extras=False)
        cfg[w1.name] = {k: d1[k] for k in ("step_us_median", "step_us_min", "hbm_frac_step",
                                           "algorithmic_bytes_per_step")}
        cfg[w1.name]["index_select_us"] = d1["index_select"]["call_us"]
        cfg[w1.name]["scan_us"] = d1["roofline"]["launch_us"]
        cfg[w1.name]["scan_hbm_frac"] = d1["roofline"]["frac"]
        w2 = I.WORKLOADS["prefill_T131072"]
        r2, _ = measure_prefill(args, torch, qsa, w2, I.make_inputs(w2), None, 2, 1)
        cfg[w2.name] = summary_prefill(r2)
        torch.cuda.empty_cache()
        rec["configs"] = cfg

    if not args.no_gdn:
        rec["gdn"] = gdn_measure(args, torch, qsa, I)
    rec["achievable_peaks"] = achievable_peaks(torch)

    if args.cpu_rows > 0 and x is not None:
        workers = oracle_workers()
        rec["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_rows, args, workers)
        del x
        dwl = I.WORKLOADS[args.decode_workload]
        rec["cpu_baseline_decode"] = cpu_baseline(dwl, I.make_inputs(dwl), dwl.batch, args, min(workers, dwl.batch))
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
