"""Paged caches (block table) against the contiguous path, bit for bit.

The caches are scattered into randomly permuted pages, with sequences that
share the pages of a common prefix; the paged prefill (append, fused
index-select, attention) and the paged decode step must give the contiguous
path's selection, output and LSE bits and leave the same rows and block keys
in the pages.  One shared-prefix prefill is also held to the oracle.
"""

import math
import types

import numpy as np
import pytest
import torch

from block_sparse_long_12_amd import qsa
from oracle import qsa_oracle as O
from tests.gpu_common import (DeviceRaggedDecode, compare_result_rows, compare_rows, oracle_layer,
                              ragged_decode_inputs, say)
from tests.test_gpu_parity import check_appended_rows

pytestmark = pytest.mark.gpu

bf = torch.bfloat16


def _table(B, n_log, n_pages, seed, share=0):
    """Distinct random pages per (sequence, logical page); sequences b >= 1
    reuse sequence 0's first `share` pages."""
    perm = np.random.default_rng(seed).permutation(n_pages)
    t = np.zeros((B, n_log), np.int32)
    k = 0
    for b in range(B):
        for i in range(n_log):
            if b > 0 and i < share:
                t[b, i] = t[0, i]
            else:
                t[b, i] = perm[k]
                k += 1
    assert k <= n_pages
    return t


def _scatter(cache, b, upto, k=None, v=None, ki=None, kb=None):
    cache.write_contiguous(b, upto, k=k, v=v, k_idx=ki, kbar=kb)


def _gather(cache, b, n_tok):
    return cache.read_contiguous(b, n_tok)


def _same(a, b, what):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


def _new_cache(B, P, max_len, share_tokens, seed, extra_pages=7):
    n_log = (max_len + P - 1) // P
    share = share_tokens // P
    n_pages = B * n_log - (B - 1) * share + extra_pages
    cache = qsa.PagedCache(n_pages, P, B, n_log + 2)
    cache.table[:, :n_log] = torch.from_numpy(_table(B, n_log, n_pages, seed, share)).cuda()
    return cache


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("ctx,tq,P,share,yarn,gated", [
    ([70001, 4099, 130000], 1, 256, 0, False, False),
    ([70003, 70001, 70002], 3, 256, 65536, False, True),       # three sequences on one 64K-token prefix
    ([9000, 6001], 4, 64, 4096, True, False),
    ([262143, 131075], 2, 1024, 131072, True, True),
])
def test_paged_decode_step_matches_contiguous(ctx, tq, P, share, yarn, gated):
    say(f"paged decode ctx={ctx} tq={tq} P={P} share={share} yarn={yarn} gate={gated}")
    B, budget, dev = len(ctx), 512, "cuda"
    L = max(ctx) + tq
    g = torch.Generator(device=dev).manual_seed(sum(ctx) + tq)
    k = torch.randn((B, L, 2, 256), generator=g, device=dev).to(bf)
    v = torch.randn((B, L, 2, 256), generator=g, device=dev).to(bf)
    ki = (torch.randn((B, L, 128), generator=g, device=dev) / math.sqrt(128)).to(bf)
    for b in range(1, B):                                   # the shared prefix is one content
        k[b, :share], v[b, :share], ki[b, :share] = k[0, :share], v[0, :share], ki[0, :share]
    rope = qsa.YARN if yarn else None
    qsa.rope_apply(k, [0] * B, rope=rope)                    # cached K is stored rotated
    kb = torch.zeros((B, L // 4 + 1, 128), dtype=bf, device=dev)
    for b in range(B):
        qsa.compress_block_keys(ki[b:b + 1], 0, ctx[b] // 4, kb[b:b + 1])
    q_raw = torch.randn((B, tq, 24, 256), generator=g, device=dev).to(bf)
    q_idx = (torch.randn((B, tq, 4, 128), generator=g, device=dev) / math.sqrt(128)).to(bf)
    k_new = torch.randn((B, tq, 2, 256), generator=g, device=dev).to(bf)
    v_new = torch.randn((B, tq, 2, 256), generator=g, device=dev).to(bf)
    k_idx_new = (torch.randn((B, tq, 128), generator=g, device=dev) / math.sqrt(128)).to(bf)
    gate = (torch.randn((B, tq, 24, 256), generator=g, device=dev) * 3).to(bf) if gated else None

    cache = _new_cache(B, P, L, share, seed=P + tq)
    for b in range(B):
        _scatter(cache, b, ctx[b], k[b], v[b], ki[b], kb[b])
    ld = max(4, ((L - 1) // 4 + 3) // 4 * 4)
    res = []
    for paged in (False, True):
        scores = torch.full((B, tq, ld), float("nan"), device=dev)
        sel = torch.empty((B, tq, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, tq, 24, 256), dtype=bf, device=dev)
        lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)
        ws = qsa.decode_step_workspace(B, budget, tq=tq)
        if paged:
            qsa.decode_step_paged(q_raw, k_new, q_idx, cache, ctx, budget, out, lse, scores, sel, ws, v_new=v_new,
                                  k_idx_new=k_idx_new, gate=gate, rope=rope)
        else:
            qsa.decode_step(q_raw, k_new, q_idx, ki, k, v, kb, ctx, budget, out, lse, scores, sel, ws, v_new=v_new,
                            k_idx_new=k_idx_new, gate=gate, rope=rope)
        torch.cuda.synchronize()
        res.append((scores, sel, out, lse))
    (sa, la, oa, ea), (sb, lb, ob, eb) = res
    _same(la, lb, "sel")
    _same(oa, ob, "out")
    _same(ea, eb, "lse")
    for b in range(B):
        for t in range(tq):
            o = (ctx[b] + t) // 4
            _same(sa[b, t, :o], sb[b, t, :o], f"scores {b} {t}")
        n = ctx[b] + tq
        gk, gv, gki, gkb = _gather(cache, b, n)
        _same(gk, k[b, :n], f"k rows {b}")
        _same(gv, v[b, :n], f"v rows {b}")
        _same(gki, ki[b, :n], f"k_idx rows {b}")
        _same(gkb, kb[b, :n // 4], f"block keys {b}")


@pytest.mark.parametrize("pos,tq,P,share,yarn", [
    ([70001, 4099, 130000], 1, 256, 0, False),
    ([70003, 70001, 66000], 4, 256, 65536, False),        # three sequences on one 64K-token prefix
    ([270001, 262142], 3, 1024, 131072, True),           # static YaRN past 262144, a 128K-token shared prefix
])
def test_paged_decode_step_matches_the_oracle_rows(pos, tq, P, share, yarn):
    """The paged decode step (random page order, sequences sharing the pages
    of one prefix, positions differing per sequence) against the oracle's
    causal rows: rows and block keys it leaves in the pages, then scores,
    selection, output and LSE under the end-to-end protocol."""
    say(f"paged decode vs oracle pos={pos} tq={tq} P={P} share={share} yarn={yarn}")
    dev_rope, o_yarn = (qsa.YARN, O.Yarn()) if yarn else (None, None)
    B = len(pos)
    x = ragged_decode_inputs(pos, tq, seed=P + tq + share % 997, share=share)
    d = DeviceRaggedDecode(x, tq, rope=dev_rope)          # rotated prefixes and their block keys
    L = x.k.shape[1]
    cache = _new_cache(B, P, L, share, seed=P * 3 + tq)
    for b in range(B):
        _scatter(cache, b, pos[b], d.k_cache[b], d.v_cache[b], d.k_idx[b], d.kbar[b])
    ws = qsa.decode_step_workspace(B, 512, tq=tq)
    qsa.decode_step_paged(d.q_raw, d.k_new, d.q_idx, cache, pos, 512, d.out, d.lse, d.scores, d.sel, ws,
                          v_new=d.v_new, k_idx_new=d.k_idx_new, rope=dev_rope)
    torch.cuda.synchronize()
    rows = [_gather(cache, b, pos[b] + tq) for b in range(B)]
    check_appended_rows(x, pos, tq, lambda b: rows[b][0][pos[b]:].cpu(), lambda b: rows[b][1][pos[b]:].cpu(),
                        lambda b: rows[b][2][pos[b]:].cpu(), lambda b, j: rows[b][3][j].cpu(), yarn=o_yarn)
    compare_result_rows(oracle_layer(x, o_yarn), x, d.results())


# ---------------------------------------------------------------- prefill

def _prefill_inputs(B, ctx, T, share, seed):
    g = torch.Generator().manual_seed(seed)
    L = ctx + T
    x = types.SimpleNamespace()
    x.q = torch.randn((B, T, 24, 256), generator=g).to(bf)
    x.q_idx = (torch.randn((B, T, 4, 128), generator=g) / math.sqrt(128)).to(bf)
    x.k = torch.randn((B, L, 2, 256), generator=g).to(bf)
    x.v = torch.randn((B, L, 2, 256), generator=g).to(bf)
    x.k_idx = (torch.randn((B, L, 128), generator=g) / math.sqrt(128)).to(bf)
    for b in range(1, B):
        x.k[b, :share], x.v[b, :share], x.k_idx[b, :share] = x.k[0, :share], x.v[0, :share], x.k_idx[0, :share]
    return x


def _run_prefill(x, B, ctx, T, budget, chunk, P, share, rope, gate):
    dev = "cuda"
    L = ctx + T
    q_raw, q_idx = x.q.to(dev), x.q_idx.to(dev)
    k_full, v_full, ki_full = x.k.to(dev), x.v.to(dev), x.k_idx.to(dev)
    k_new = k_full[:, ctx:].contiguous()
    v_new = v_full[:, ctx:].contiguous()
    ki_new = ki_full[:, ctx:].contiguous()
    # contiguous path
    kc = k_full.clone()
    qsa.rope_apply(kc[:, :ctx], [0] * B, rope=rope)
    kb = torch.zeros((B, L // 4, 128), dtype=bf, device=dev)
    qsa.compress_block_keys(ki_full, 0, ctx // 4, kb)
    bufs = qsa.PrefillBuffers(B, T, ctx, budget, chunk)
    out_c = torch.empty((B, T, 24, 256), dtype=bf, device=dev)
    lse_c = torch.empty((B, T, 24), dtype=torch.float32, device=dev)
    qsa.prefill_layer(q_raw, k_new, q_idx, ki_full, kc, v_full, kb, ctx, budget, out_c, lse_c, bufs,
                      torch.empty_like(q_raw), gate=gate, rope=rope)
    torch.cuda.synchronize()
    sel_c = bufs.sel.clone()
    # paged path: the prefix (rotated K, V, indexer keys, block keys) in pages, the chunk appended
    cache = _new_cache(B, P, L, share, seed=P + T)
    k_pre = k_full[:, :ctx].clone()
    qsa.rope_apply(k_pre, [0] * B, rope=rope)
    for b in range(B):
        _scatter(cache, b, ctx, k_pre[b], v_full[b], ki_full[b], kb[b])
    bufs_p = qsa.PrefillBuffers(B, T, ctx, budget, chunk)
    out_p = torch.empty_like(out_c)
    lse_p = torch.empty_like(lse_c)
    qsa.prefill_layer_paged(q_raw, k_new, v_new, q_idx, ki_new, cache, ctx, budget, out_p, lse_p, bufs_p,
                            torch.empty_like(q_raw), gate=gate, rope=rope)
    torch.cuda.synchronize()
    _same(sel_c, bufs_p.sel, "sel")
    _same(out_c, out_p, "out")
    _same(lse_c, lse_p, "lse")
    for b in range(B):
        gk, gv, gki, gkb = _gather(cache, b, L)
        _same(gk, kc[b], f"k rows {b}")
        _same(gv, v_full[b], f"v rows {b}")
        _same(gki, ki_full[b], f"k_idx rows {b}")
        _same(gkb, kb[b, :L // 4], f"block keys {b}")
    return sel_c, out_c, lse_c


@pytest.mark.parametrize("B,ctx,T,chunk,P,share,yarn,gated", [
    (2, 70001, 300, 128, 256, 65536, False, False),     # fused index-select, a 64K-token shared prefix
    (3, 2001, 257, 64, 64, 1984, True, True),          # exact index-select (short context), ragged chunks
    (1, 131075, 130, 130, 4096, 0, False, False),      # pages of 4096 tokens, the chunk spans a page boundary
])
def test_paged_prefill_matches_contiguous(B, ctx, T, chunk, P, share, yarn, gated):
    say(f"paged prefill B={B} ctx={ctx} T={T} P={P} share={share} yarn={yarn} gate={gated}")
    x = _prefill_inputs(B, ctx, T, share, seed=ctx + T)
    gate = (torch.randn((B, T, 24, 256), generator=torch.Generator().manual_seed(5)) * 3).to(bf).cuda() \
        if gated else None
    _run_prefill(x, B, ctx, T, 512, chunk, P, share, qsa.YARN if yarn else None, gate)


def test_shared_prefix_paged_prefill_matches_the_oracle():
    """Two sequences on one shared 8192-token prefix, paged, against the
    oracle's rows under the end-to-end protocol."""
    B, ctx, T, budget, P = 2, 9001, 96, 64, 256
    say(f"shared-prefix paged prefill vs oracle B={B} ctx={ctx} T={T}")
    x = _prefill_inputs(B, ctx, T, 8192, seed=17)
    sel, out, lse = _run_prefill(x, B, ctx, T, budget, 48, P, 8192, None, None)
    sel, out, lse = sel.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    Bt = O.bits
    layer = O.OracleLayer(Bt(x.q), Bt(x.q_idx), Bt(x.k), Bt(x.v), Bt(x.k_idx), [ctx] * B, budget)
    rows = [(b, ctx + i) for b in range(B) for i in range(0, T, 5)]
    compare_rows(layer, types.SimpleNamespace(needles=[]), rows, None, lambda b, t: sel[b, t - ctx],
                 lambda b, t: out[b, t - ctx], lambda b, t: lse[b, t - ctx])


def test_paged_two_stream_prefill_matches_one_stream():
    """prefill_layer_paged with a side stream (the query chunks'
    index-selects on it, fused path: the first row sees more than 16384
    blocks) gives the one-stream selections, outputs and LSE bit for bit."""
    B, ctx, T, chunk, budget, P = 1, 70000, 1536, 512, 512, 256
    say(f"paged two-stream prefill B={B} ctx={ctx} T={T} chunk={chunk}")
    x = _prefill_inputs(B, ctx, T, 0, seed=23)
    dev = "cuda"
    res = []
    for side in (None, torch.cuda.Stream()):
        k_full = x.k.to(dev)
        k_pre = k_full[:, :ctx].clone()
        qsa.rope_apply(k_pre, [0] * B)
        ki_full = x.k_idx.to(dev)
        kb = torch.zeros((B, (ctx + T) // 4, 128), dtype=bf, device=dev)
        qsa.compress_block_keys(ki_full, 0, ctx // 4, kb)
        cache = _new_cache(B, P, ctx + T, 0, seed=29)
        v_full = x.v.to(dev)
        _scatter(cache, 0, ctx, k_pre[0], v_full[0], ki_full[0], kb[0])
        bufs = qsa.PrefillBuffers(B, T, ctx, budget, chunk)
        out = torch.empty((B, T, 24, 256), dtype=bf, device=dev)
        lse = torch.empty((B, T, 24), dtype=torch.float32, device=dev)
        q_raw = x.q.to(dev)
        qsa.prefill_layer_paged(q_raw, k_full[:, ctx:].contiguous(), v_full[:, ctx:].contiguous(), x.q_idx.to(dev),
                                ki_full[:, ctx:].contiguous(), cache, ctx, budget, out, lse, bufs,
                                torch.empty_like(q_raw), side_stream=side)
        torch.cuda.synchronize()
        res.append((bufs.sel.clone(), out, lse))
    _same(res[0][0], res[1][0], "sel")
    _same(res[0][1], res[1][1], "out")
    _same(res[0][2], res[1][2], "lse")
