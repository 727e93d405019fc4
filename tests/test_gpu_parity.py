"""HIP path against the CPU oracle, step by step and end to end.

Per-step tests feed both sides identical inputs (oracle-made where a step
consumes an earlier step's result); end-to-end tests run every step on the
GPU from the raw seeded inputs and compare with the near-tie protocol of
tests/gpu_common.compare_rows.
"""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from block_sparse_long_12_amd import qsa
from oracle import qsa_oracle as O
from tests.gpu_common import (MAX_ABS, MEAN_ABS, LSE_ABS, DeviceDecode, DevicePrefill, DeviceRaggedDecode,
                              bf16_ulp_diff, bits, compare_result_rows, compare_rows, oracle_layer,
                              ragged_decode_inputs, say, score_bound)

pytestmark = pytest.mark.gpu


def _rand_bf16(shape, seed, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(torch.bfloat16)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a device"
    qsa.lib()


# ------------------------------------------------------------------ step 0

ROPES = {
    "plain": (None, None),
    "yarn4": (qsa.YARN, O.Yarn(factor=4.0, original_max=262144)),
    "yarn2_theta5e5": (qsa.rope_params(5e5, 2.0, 32768), O.Yarn(factor=2.0, original_max=32768)),
}


@pytest.mark.parametrize("rope", list(ROPES))
@pytest.mark.parametrize("heads", [24, 2])
def test_rope_matches_oracle(heads, rope):
    say(f"rope heads={heads} {rope}")
    dev_rope, yarn = ROPES[rope]
    theta = 5e5 if rope == "yarn2_theta5e5" else O.ROPE_THETA
    x = _rand_bf16((2, 37, heads, 256), 1 + heads)
    pos0 = [0, 1048000]
    xd = x.cuda()
    yd = torch.empty_like(xd)
    qsa.rope_apply(xd, pos0, out=yd, rope=dev_rope)
    got = bits(yd)
    ref = np.stack([O.rope_rotate(bits(x[b]), np.arange(37) + pos0[b], theta=theta, yarn=yarn)
                    for b in range(2)])
    assert np.array_equal(got[..., 64:], bits(x)[..., 64:])
    ulp = bf16_ulp_diff(got, ref)
    assert ulp.max() <= 1 and np.mean(ulp == 0) >= 0.9999, (ulp.max(), np.mean(ulp == 0))
    # in place equals out of place
    qsa.rope_apply(xd, pos0, rope=dev_rope)
    assert np.array_equal(bits(xd), got)


# ------------------------------------------------------------------ step 1

def test_compress_is_bit_exact():
    say("compress")
    k = _rand_bf16((3, 4 * 701 + 2, 128), 11, sigma=1 / math.sqrt(128))
    # the hand-derived cases in the first blocks of sequence 0
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "compress_cases.json")))["cases"]
    for ci, c in enumerate(cases):
        for r, h in enumerate(c["keys"]):
            k[0, 4 * ci + r, :] = float.fromhex(h)
    kd = k.cuda()
    kbar = torch.zeros((3, 701, 128), dtype=torch.bfloat16, device="cuda")
    qsa.compress_block_keys(kd, 0, 701, kbar)
    got = bits(kbar)
    for b in range(3):
        assert np.array_equal(got[b], O.compress_block_keys(bits(k[b]), 0, 701))
    for ci, c in enumerate(cases):
        assert np.all(got[0, ci] == int(c["bits"], 16)), c
    part = torch.zeros_like(kbar)
    qsa.compress_block_keys(kd, 100, 333, part)
    pg = bits(part)
    assert np.array_equal(pg[:, 100:333], got[:, 100:333]) and not pg[:, :100].any() and not pg[:, 333:].any()


# ------------------------------------------------------------------ step 2

INDEX_CASES = [
    ("prefill ragged", 1, [0], 77),
    ("prefill batched offsets", 2, [1003, 50], 70),
    ("decode long", 3, [70001, 4096, 9999], 1),
    ("prefill one tile", 1, [4 * 64 + 1], 16),
]


def _index_case(B, pos0, tq, seed):
    q = _rand_bf16((B, tq, 4, 128), seed, sigma=1 / math.sqrt(128))
    nblk = max((p + tq - 1) // 4 for p in pos0)
    kbar = _rand_bf16((B, max(1, nblk), 128), seed + 1, sigma=1 / math.sqrt(512))
    ld = max(4, (nblk + 3) // 4 * 4)
    scores = torch.full((B, tq, ld), float("nan"), dtype=torch.float32, device="cuda")
    qsa.index_scores(q.cuda(), kbar.cuda(), pos0, scores)
    return q, kbar, scores.cpu().numpy()


@pytest.mark.parametrize("name,B,pos0,tq", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_scores_within_float32_bound(name, B, pos0, tq):
    say(f"index_scores {name}")
    q, kbar, got = _index_case(B, pos0, tq, 21 + tq)
    exact = 0
    total = 0
    for b in range(B):
        kb = bits(kbar[b])
        ref = O.index_scores(bits(q[b]), O.bf16_to_f64(kb))
        for i in range(tq):
            o = (pos0[b] + i) // 4
            if o == 0:
                continue
            bound = score_bound(bits(q[b, i]), kb[:o])
            err = np.abs(got[b, i, :o].astype(np.float64) - ref[i, :o].astype(np.float64))
            assert np.all(err <= bound), (b, i, err.max())
            exact += int(np.sum(got[b, i, :o] == ref[i, :o]))
            total += o
    say(f"  exactly rounded: {exact}/{total}")


def test_index_scores_do_not_depend_on_launch_shape():
    say("index_scores launch-shape independence")
    B, pos0, tq = 1, [2000], 64
    q, kbar, full = _index_case(B, pos0, tq, 5)
    sub = torch.full((1, 20, full.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
    qsa.index_scores(q[:, 10:30].contiguous().cuda(), kbar.cuda(), [pos0[0] + 10], sub)
    sub = sub.cpu().numpy()
    for i in range(20):
        o = (pos0[0] + 10 + i) // 4
        assert np.array_equal(sub[0, i, :o], full[0, 10 + i, :o])


# ------------------------------------------------------------------ step 3

def _select_gpu(scores_rows: np.ndarray, p0: int, budget: int) -> np.ndarray:
    """scores_rows [T, ld] float32 for rows at positions p0 .. p0+T-1."""
    T, ld = scores_rows.shape
    s = torch.from_numpy(np.ascontiguousarray(scores_rows)).reshape(1, T, ld).cuda()
    sel = torch.empty((1, T, budget), dtype=torch.int32, device="cuda")
    qsa.select_topk(s, [p0], budget, sel)
    return sel.cpu().numpy()[0]


def _rows(kind, n_cand, T, rng):
    if kind == "normal":
        return rng.standard_normal((T, n_cand)).astype(np.float32) * np.float32(0.088)
    if kind == "equal":
        return np.full((T, n_cand), 0.25, np.float32)
    if kind == "coarse":
        return (rng.integers(-4, 5, (T, n_cand)) * 0.5).astype(np.float32)
    if kind == "signed_zero":
        v = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), (T, n_cand))
        return v.astype(np.float32)
    if kind == "specials":
        v = rng.standard_normal((T, n_cand)).astype(np.float32)
        m = rng.random((T, n_cand))
        v[m < 0.05] = np.nan
        v[(m >= 0.05) & (m < 0.08)] = np.inf
        v[(m >= 0.08) & (m < 0.11)] = -np.inf
        return v
    if kind == "clustered":    # every key shares its top bits: several radix digits
        return (np.float32(1.0) + rng.integers(0, 6000, (T, n_cand)).astype(np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
    if kind == "front_loaded":   # the row's head outranks the rest: a sample there overestimates the tail
        v = rng.standard_normal((T, n_cand)).astype(np.float32)
        v[:, :256] += np.float32(10.0)
        return v
    if kind == "tie_flood":    # a few winners, then thousands of exact ties at the threshold
        v = np.full((T, n_cand), 0.5, np.float32)
        v[:, rng.choice(n_cand, 300, replace=False)] = 2.0
        v[:, rng.choice(n_cand, 200, replace=False)] = -1.0
        return v
    raise ValueError(kind)


SELECT_CASES = [
    ("normal", 70000, 512), ("normal", 2047, 512), ("normal", 5000, 64), ("normal", 600, 2048),
    ("normal", 9000, 1), ("normal", 9000, 2), ("normal", 3000, 17),
    ("equal", 10000, 512), ("coarse", 8000, 512), ("signed_zero", 6000, 300),
    ("specials", 7000, 512), ("clustered", 20000, 512), ("tie_flood", 12000, 512),
    ("tie_flood", 12000, 2048), ("front_loaded", 70000, 512), ("normal", 262144, 512),
    ("normal", 262144, 1024), ("normal", 4096, 1024), ("specials", 70000, 64),
]


@pytest.mark.parametrize("kind,n_cand,budget", SELECT_CASES,
                         ids=[f"{k}-{n}-{b}" for k, n, b in SELECT_CASES])
def test_select_is_bit_exact_on_identical_scores(kind, n_cand, budget):
    say(f"select {kind} n={n_cand} budget={budget}")
    rng = np.random.default_rng(n_cand + budget)
    T = 6
    p0 = 4 * n_cand - 2                         # rows see n_cand - 1 .. n_cand + 1 candidates
    o_max = (p0 + T - 1) // 4
    ld = (o_max + 3) // 4 * 4
    rows = np.full((T, ld), np.float32(7.0))    # poison past each row's candidates
    rows[:, :o_max] = _rows(kind, o_max, T, rng)
    got = _select_gpu(rows, p0, budget)
    for i in range(T):
        ref = O.select_blocks(rows[i], p0 + i, budget)
        assert np.array_equal(got[i], ref), (i, got[i][:8], ref[:8])


def test_select_small_rows_and_early_tokens():
    say("select early tokens")
    rng = np.random.default_rng(3)
    T = 300
    rows = rng.standard_normal((T, 76)).astype(np.float32)
    got = _select_gpu(rows, 0, 8)
    for i in range(T):
        assert np.array_equal(got[i], O.select_blocks(rows[i], i, 8)), i


# ------------------------------------------------------------------ step 4

def _oracle_inputs_for_attention(x: I.Inputs):
    """Oracle-rotated Q and K (the attention step's inputs) as device tensors."""
    wl = x.workload
    qr = np.stack([O.rope_rotate(bits(x.q[b]), wl.ctx + np.arange(wl.tq)) for b in range(wl.batch)])
    kr = np.stack([O.rope_rotate(bits(x.k[b]), np.arange(wl.length)) for b in range(wl.batch)])
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return to_dev(qr), to_dev(kr)


def _check_attention(got_out, got_lse, ref_rows):
    d = np.abs(got_out.astype(np.float64) - np.stack([r.out for r in ref_rows]))
    dl = np.abs(got_lse.astype(np.float64) - np.stack([r.lse for r in ref_rows]))
    say(f"  max_abs={d.max():.3g} mean_abs={d.mean():.3g} lse_abs={dl.max():.3g}")
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS and dl.max() <= LSE_ABS


@pytest.mark.parametrize("ctx,tq,budget", [(300, 90, 32), (0, 70, 8), (5000, 33, 512)])
def test_attention_prefill_with_oracle_selection(ctx, tq, budget):
    say(f"attention prefill ctx={ctx} tq={tq} budget={budget}")
    wl = I.custom_workload("prefill", batch=2, ctx=ctx, tq=tq, budget=budget, seed=ctx + tq)
    x = I.make_inputs(wl)
    layer = oracle_layer(x)
    rows = [(b, ctx + i) for b in range(2) for i in range(tq)]
    ref = layer.rows(rows)
    qd, kd = _oracle_inputs_for_attention(x)
    sel = torch.from_numpy(np.stack([r.sel for r in ref]).reshape(2, tq, budget)).cuda()
    out = torch.empty((2, tq, 24, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, tq, 24), dtype=torch.float32, device="cuda")
    qsa.sparse_attn_prefill(qd, kd, x.v.cuda(), sel, [ctx, ctx], out, lse)
    _check_attention(out.float().cpu().numpy().reshape(-1, 24, 256), lse.cpu().numpy().reshape(-1, 24), ref)


@pytest.mark.parametrize("ctx,budget", [(8000, 512), (8000, 64), (100, 512), (1, 4)])
def test_attention_decode_with_oracle_selection(ctx, budget):
    say(f"attention decode ctx={ctx} budget={budget}")
    B = 3
    wl = I.custom_workload("decode", batch=B, ctx=ctx, tq=1, budget=budget, seed=ctx + budget)
    x = I.make_inputs(wl)
    layer = oracle_layer(x)
    rows = [(b, ctx) for b in range(B)]
    ref = layer.rows(rows)
    qd, kd = _oracle_inputs_for_attention(x)
    sel = torch.from_numpy(np.stack([r.sel for r in ref])).cuda()
    out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 24), dtype=torch.float32, device="cuda")
    ws = qsa.decode_workspace(B, budget)
    qsa.sparse_attn_decode(qd[:, 0], kd, x.v.cuda(), sel, [ctx] * B, out, lse, ws)
    _check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref)


# ------------------------------------------------------------------ end to end

def test_end_to_end_prefill_T2048_budget64_every_row():
    wl = I.WORKLOADS["prefill_T2048_budget64"]
    say(f"end-to-end {wl.name}")
    x = I.make_inputs(wl)
    dp = DevicePrefill(x)
    dp.run()
    scores = dp.bufs.scores.cpu().numpy()
    sel = dp.bufs.sel.cpu().numpy()
    out = dp.out.float().cpu().numpy()
    lse = dp.lse.cpu().numpy()
    layer = oracle_layer(x)
    rows = [(0, t) for t in range(wl.tq)]
    compare_rows(layer, x, rows,
                 lambda b, t: scores[b, t, :t // 4], lambda b, t: sel[b, t],
                 lambda b, t: out[b, t], lambda b, t: lse[b, t])


def test_end_to_end_prefill_with_prefix_and_chunks():
    wl = I.custom_workload("prefill", batch=2, ctx=6001, tq=700, budget=64, n_needles=6, seed=77, chunk=256)
    say(f"end-to-end {wl.name}")
    x = I.make_inputs(wl)
    dp = DevicePrefill(x)
    dp.run()
    sel = dp.bufs.sel.cpu().numpy()
    out = dp.out.float().cpu().numpy()
    lse = dp.lse.cpu().numpy()
    layer = oracle_layer(x)
    rows = [(b, wl.ctx + i) for b in range(2) for i in range(0, wl.tq, 7)] + \
           [(int(b), int(t)) for b, t, _ in x.needles]
    rows = sorted(set(rows))
    compare_rows(layer, x, rows, None, lambda b, t: sel[b, t - wl.ctx],
                 lambda b, t: out[b, t - wl.ctx], lambda b, t: lse[b, t - wl.ctx])


def test_end_to_end_prefill_long_context_fused_select():
    """A chunk long enough for the fused index-select (its rows see > 16384
    blocks), sampled rows and every needle against the oracle."""
    wl = I.custom_workload("prefill", batch=1, ctx=70001, tq=1024, budget=512, n_needles=8, seed=5, chunk=512)
    say(f"end-to-end {wl.name}")
    x = I.make_inputs(wl)
    dp = DevicePrefill(x)
    dp.run()
    sel = dp.bufs.sel.cpu().numpy()
    out = dp.out.float().cpu().numpy()
    lse = dp.lse.cpu().numpy()
    n_flagged = int(dp.bufs.workspace[:4].view(torch.int32)[0].item())
    say(f"  rows that took the exact fallback in the last chunk: {n_flagged}")
    layer = oracle_layer(x)
    rows = [(0, wl.ctx + i) for i in range(0, wl.tq, 16)] + [(int(b), int(t)) for b, t, _ in x.needles]
    rows = sorted(set(rows))
    compare_rows(layer, x, rows, None, lambda b, t: sel[b, t - wl.ctx],
                 lambda b, t: out[b, t - wl.ctx], lambda b, t: lse[b, t - wl.ctx])


def test_end_to_end_decode_B32_ctx32K():
    wl = I.WORKLOADS["decode_B32_ctx32K"]
    say(f"end-to-end {wl.name}")
    x = I.make_inputs(wl)
    dd = DeviceDecode(x)
    dd.run()
    scores = dd.scores.cpu().numpy()
    sel = dd.sel.cpu().numpy()
    out = dd.out.float().cpu().numpy()
    lse = dd.lse.cpu().numpy()
    layer = oracle_layer(x)
    rows = [(b, wl.ctx) for b in range(wl.batch)]
    o = wl.ctx // 4
    compare_rows(layer, x, rows, lambda b, t: scores[b, 0, :o], lambda b, t: sel[b, 0],
                 lambda b, t: out[b], lambda b, t: lse[b])


def test_consecutive_decode_steps_match_the_oracle_rows():
    """Serving decode steps one token at a time (each appends its K, V and
    indexer-key rows and compresses the block it completes) give, row by
    row, the oracle's causal QSA output for those tokens."""
    B, ctx, S, budget = 2, 20001, 6, 512
    wl = I.custom_workload("prefill", batch=B, ctx=ctx, tq=S, budget=budget, n_needles=4, seed=31)
    say(f"consecutive decode steps {wl.name}")
    x = I.make_inputs(wl)
    dev = "cuda"
    L = ctx + S
    kc = torch.zeros((B, L, 2, 256), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(kc)
    ki = torch.zeros((B, L, 128), dtype=torch.bfloat16, device=dev)
    kc[:, :ctx] = x.k[:, :ctx].to(dev)
    qsa.rope_apply(kc[:, :ctx], [0] * B)
    v[:, :ctx] = x.v[:, :ctx].to(dev)
    ki[:, :ctx] = x.k_idx[:, :ctx].to(dev)
    kb = torch.zeros((B, L // 4 + 1, 128), dtype=torch.bfloat16, device=dev)
    qsa.compress_block_keys(ki, 0, ctx // 4, kb)
    ld = (L // 4 + 3) // 4 * 4
    ws = qsa.decode_step_workspace(B, budget)
    res = {}
    for s in range(S):
        t = ctx + s
        scores = torch.empty((B, 1, ld), dtype=torch.float32, device=dev)
        sel = torch.empty((B, 1, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
        qsa.decode_step(x.q[:, s:s + 1].contiguous().to(dev), x.k[:, t:t + 1].contiguous().to(dev),
                        x.q_idx[:, s:s + 1].contiguous().to(dev), ki, kc, v, kb, t, budget, out, lse, scores, sel,
                        ws, v_new=x.v[:, t:t + 1].contiguous().to(dev),
                        k_idx_new=x.k_idx[:, t:t + 1].contiguous().to(dev))
        torch.cuda.synchronize()
        for b in range(B):
            res[(b, t)] = (scores[b, 0, :t // 4].cpu().numpy(), sel[b, 0].cpu().numpy(),
                           out[b].float().cpu().numpy(), lse[b].cpu().numpy())
    rows = sorted(res)
    compare_rows(oracle_layer(x), x, rows, lambda b, t: res[(b, t)][0], lambda b, t: res[(b, t)][1],
                 lambda b, t: res[(b, t)][2], lambda b, t: res[(b, t)][3])


@pytest.mark.parametrize("ctx,n_steps,yarn", [(30001, 3, False), (270001, 2, True)],
                         ids=["ctx30001", "ctx270001_yarn"])
def test_multi_token_decode_steps_match_the_oracle_rows(ctx, n_steps, yarn):
    """Decode steps of 3 new tokens each (the shape of speculative
    verification), run back to back, give the oracle's causal QSA rows for
    every token; blocks completed inside a step are scored by its later
    tokens.  With yarn: the model card's static YaRN rotary past 262144."""
    B, tq, budget = 2, 3, 512
    dev_rope, o_yarn = (qsa.YARN, O.Yarn()) if yarn else (None, None)
    S = tq * n_steps
    wl = I.custom_workload("prefill", batch=B, ctx=ctx, tq=S, budget=budget, n_needles=4, seed=47)
    say(f"multi-token decode steps {wl.name}")
    x = I.make_inputs(wl)
    dev = "cuda"
    L = ctx + S
    kc = torch.zeros((B, L, 2, 256), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(kc)
    ki = torch.zeros((B, L, 128), dtype=torch.bfloat16, device=dev)
    kc[:, :ctx] = x.k[:, :ctx].to(dev)
    qsa.rope_apply(kc[:, :ctx], [0] * B, rope=dev_rope)
    v[:, :ctx] = x.v[:, :ctx].to(dev)
    ki[:, :ctx] = x.k_idx[:, :ctx].to(dev)
    kb = torch.zeros((B, L // 4 + 1, 128), dtype=torch.bfloat16, device=dev)
    qsa.compress_block_keys(ki, 0, ctx // 4, kb)
    ld = (L // 4 + 3) // 4 * 4
    ws = qsa.decode_step_workspace(B, budget, tq=tq)
    res = {}
    for st in range(n_steps):
        s0, t0 = tq * st, ctx + tq * st
        scores = torch.empty((B, tq, ld), dtype=torch.float32, device=dev)
        sel = torch.empty((B, tq, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, tq, 24, 256), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)
        sl = slice(s0, s0 + tq)
        qsa.decode_step(x.q[:, sl].contiguous().to(dev), x.k[:, t0:t0 + tq].contiguous().to(dev),
                        x.q_idx[:, sl].contiguous().to(dev), ki, kc, v, kb, t0, budget, out, lse, scores, sel, ws,
                        v_new=x.v[:, t0:t0 + tq].contiguous().to(dev),
                        k_idx_new=x.k_idx[:, t0:t0 + tq].contiguous().to(dev), rope=dev_rope)
        torch.cuda.synchronize()
        for b in range(B):
            for t in range(tq):
                p = t0 + t
                res[(b, p)] = (scores[b, t, :p // 4].cpu().numpy(), sel[b, t].cpu().numpy(),
                               out[b, t].float().cpu().numpy(), lse[b, t].cpu().numpy())
    rows = sorted(res)
    compare_rows(oracle_layer(x, o_yarn), x, rows, lambda b, t: res[(b, t)][0], lambda b, t: res[(b, t)][1],
                 lambda b, t: res[(b, t)][2], lambda b, t: res[(b, t)][3])


RAGGED = [([70001, 4099, 130000], 1, False), ([70001, 4099, 130000], 3, False),
          ([270001, 4099, 262142], 4, True)]


def check_appended_rows(x, pos, tq, k_rows, v_rows, ki_rows, kbar_of, yarn=None):
    """The rows a decode step appended for sequence b at pos[b] .. pos[b] + tq - 1:
    K rotated (within 1 bf16 ulp of the oracle's rotation, at least 99% equal),
    V and indexer keys bit for bit, and the key of every block a new token
    completes equal to the oracle's compression (bit for bit).
    k_rows(b) / v_rows(b) / ki_rows(b) -> the tq rows in the cache (CPU bf16);
    kbar_of(b, j) -> block key j of sequence b (CPU bf16 [128])."""
    same = total = 0
    for b, p in enumerate(pos):
        ref_k = O.rope_rotate(bits(x.k[b, p:p + tq]), np.arange(p, p + tq), yarn=yarn)
        ulp = bf16_ulp_diff(bits(k_rows(b)), ref_k)
        assert ulp.max() <= 1, (b, int(ulp.max()))
        same += int((ulp == 0).sum())
        total += ulp.size
        assert np.array_equal(bits(v_rows(b)), bits(x.v[b, p:p + tq])), b
        assert np.array_equal(bits(ki_rows(b)), bits(x.k_idx[b, p:p + tq])), b
        for t in range(p, p + tq):
            if t % 4 == 3:
                j = t // 4
                ref = O.compress_block_keys(bits(x.k_idx[b]), j, j + 1)[0]
                assert np.array_equal(bits(kbar_of(b, j)), ref), (b, j)
    assert same >= 0.99 * total, (same, total)


@pytest.mark.parametrize("pos,tq,yarn", RAGGED, ids=["tq1", "tq3", "tq4_yarn"])
def test_ragged_decode_step_matches_the_oracle_rows(pos, tq, yarn):
    """One serving decode step whose sequences sit at different positions
    (rows of other lengths' garbage past each sequence's end) against the
    oracle's causal rows: the appended rows and completed block keys, then
    scores, selection, output and LSE under the end-to-end protocol."""
    say(f"ragged decode step pos={pos} tq={tq} yarn={yarn}")
    dev_rope, o_yarn = (qsa.YARN, O.Yarn()) if yarn else (None, None)
    x = ragged_decode_inputs(pos, tq, seed=sum(pos) % 1000 + tq)
    d = DeviceRaggedDecode(x, tq, rope=dev_rope)
    ws = qsa.decode_step_workspace(len(pos), 512, tq=tq)
    qsa.decode_step(d.q_raw, d.k_new, d.q_idx, d.k_idx, d.k_cache, d.v_cache, d.kbar, pos, 512, d.out, d.lse,
                    d.scores, d.sel, ws, v_new=d.v_new, k_idx_new=d.k_idx_new, rope=dev_rope)
    torch.cuda.synchronize()
    check_appended_rows(x, pos, tq, lambda b: d.k_cache[b, pos[b]:pos[b] + tq].cpu(),
                        lambda b: d.v_cache[b, pos[b]:pos[b] + tq].cpu(),
                        lambda b: d.k_idx[b, pos[b]:pos[b] + tq].cpu(), lambda b, j: d.kbar[b, j].cpu(),
                        yarn=o_yarn)
    compare_result_rows(oracle_layer(x, o_yarn), x, d.results())


# ------------------------------------------------------------------ output gate

def _gate(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 3).to(torch.bfloat16)


def test_gated_attention_prefill_and_decode_with_oracle_selection():
    """The output gate fused into the prefill epilogue and the decode merge
    (1 and 3 tokens per sequence) against the oracle's gated rows; LSE is
    the ungated one."""
    ctx, tq, budget = 3000, 3, 512
    wl = I.custom_workload("prefill", batch=2, ctx=ctx, tq=tq, budget=budget, seed=91)
    say(f"gated attention {wl.name}")
    x = I.make_inputs(wl)
    gate = _gate((2, tq, 24, 256), 5)
    layer = O.OracleLayer(O.bits(x.q), O.bits(x.q_idx), O.bits(x.k), O.bits(x.v), O.bits(x.k_idx), x.q_pos0,
                          budget, gate=O.bits(gate))
    rows = [(b, ctx + i) for b in range(2) for i in range(tq)]
    ref = layer.rows(rows)
    qd, kd = _oracle_inputs_for_attention(x)
    sel = torch.from_numpy(np.stack([r.sel for r in ref]).reshape(2, tq, budget)).cuda()
    out = torch.empty((2, tq, 24, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, tq, 24), dtype=torch.float32, device="cuda")
    qsa.sparse_attn_prefill(qd, kd, x.v.cuda(), sel, [ctx, ctx], out, lse, gate=gate.cuda())
    _check_attention(out.float().cpu().numpy().reshape(-1, 24, 256), lse.cpu().numpy().reshape(-1, 24), ref)
    # decode form, all 3 tokens per sequence in one call
    out_d = torch.empty_like(out)
    lse_d = torch.empty_like(lse)
    ws = qsa.decode_workspace(2, budget, tq=tq)
    qsa.sparse_attn_decode(qd, kd, x.v.cuda(), sel, [ctx, ctx], out_d, lse_d, ws, gate=gate.cuda())
    _check_attention(out_d.float().cpu().numpy().reshape(-1, 24, 256), lse_d.cpu().numpy().reshape(-1, 24), ref)
    # one token per sequence
    out_1 = torch.empty((2, 24, 256), dtype=torch.bfloat16, device="cuda")
    lse_1 = torch.empty((2, 24), dtype=torch.float32, device="cuda")
    qsa.sparse_attn_decode(qd[:, 0].contiguous(), kd, x.v.cuda(), sel[:, 0].contiguous(), [ctx, ctx], out_1, lse_1,
                           qsa.decode_workspace(2, budget), gate=gate[:, 0].contiguous().cuda())
    ref1 = [ref[0], ref[tq]]
    _check_attention(out_1.float().cpu().numpy(), lse_1.cpu().numpy(), ref1)


def test_gated_prefill_layer_end_to_end():
    """A whole prefill chunk with the output gate against the oracle's gated
    rows under the end-to-end protocol."""
    wl = I.custom_workload("prefill", batch=1, ctx=2000, tq=300, budget=64, n_needles=4, seed=93, chunk=128)
    say(f"gated prefill layer {wl.name}")
    x = I.make_inputs(wl)
    gate = _gate((1, 300, 24, 256), 6)
    dp = DevicePrefill(x)
    dp.run(gate=gate.cuda())
    layer = O.OracleLayer(O.bits(x.q), O.bits(x.q_idx), O.bits(x.k), O.bits(x.v), O.bits(x.k_idx), x.q_pos0,
                          wl.budget, gate=O.bits(gate))
    sel = dp.bufs.sel.cpu().numpy()
    out = dp.out.float().cpu().numpy()
    lse = dp.lse.cpu().numpy()
    rows = [(0, 2000 + i) for i in range(0, 300, 7)]
    compare_rows(layer, x, rows, None, lambda b, t: sel[b, t - 2000], lambda b, t: out[b, t - 2000],
                 lambda b, t: lse[b, t - 2000])


# ------------------------------------------------------------------ static YaRN

def test_yarn_prefill_layer_end_to_end():
    """A prefill chunk past 262144 positions with the model card's static
    YaRN (factor 4 over 262144) against the oracle's YaRN rows under the
    end-to-end protocol; the cached prefix is rotated with the same table."""
    wl = I.custom_workload("prefill", batch=1, ctx=263000, tq=200, budget=512, n_needles=4, seed=95, chunk=128)
    say(f"yarn prefill layer {wl.name}")
    x = I.make_inputs(wl)
    dp = DevicePrefill(x, rope=qsa.YARN)
    dp.run()
    sel = dp.bufs.sel.cpu().numpy()
    out = dp.out.float().cpu().numpy()
    lse = dp.lse.cpu().numpy()
    rows = [(0, 263000 + i) for i in range(0, 200, 9)]
    compare_rows(oracle_layer(x, O.Yarn()), x, rows, None, lambda b, t: sel[b, t - 263000],
                 lambda b, t: out[b, t - 263000], lambda b, t: lse[b, t - 263000])


def test_decode_step_at_position_zero_returns_the_new_value_rows():
    """A sequence with nothing cached: the selection is the own block alone,
    which holds only the new token, so softmax gives that token weight 1.  At
    position 0 the rotation is the identity.  Every head of KV group g then
    returns the token's V row of group g bit for bit; the LSE is the scaled
    logit q.k, within 2^-15 sum |q k| (float32 accumulation of 256 bf16
    products); the selection is [0, -1, ...]."""
    say("decode_step at position 0")
    B, budget, L = 3, 64, 8
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator().manual_seed(5)
    q_raw = torch.randn((B, 1, 24, 256), generator=g).to(bf)
    k_new = torch.randn((B, 1, 2, 256), generator=g).to(bf)
    v_new = torch.randn((B, 1, 2, 256), generator=g).to(bf)
    q_idx = (torch.randn((B, 1, 4, 128), generator=g) / math.sqrt(128)).to(bf)
    k_idx_new = (torch.randn((B, 1, 128), generator=g) / math.sqrt(128)).to(bf)
    kc = torch.zeros((B, L, 2, 256), dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    ki = torch.zeros((B, L, 128), dtype=bf, device=dev)
    kb = torch.zeros((B, L // 4 + 1, 128), dtype=bf, device=dev)
    scores = torch.zeros((B, 1, 4), device=dev)
    sel = torch.empty((B, 1, budget), dtype=torch.int32, device=dev)
    out = torch.empty((B, 24, 256), dtype=bf, device=dev)
    lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(256)
    qsa.decode_step(q_raw.to(dev), k_new.to(dev), q_idx.to(dev), ki, kc, vc, kb, 0, budget, out, lse, scores, sel,
                    qsa.decode_step_workspace(B, budget), scale=scale, v_new=v_new.to(dev),
                    k_idx_new=k_idx_new.to(dev))
    torch.cuda.synchronize()
    assert sel[:, 0, 0].eq(0).all() and sel[:, 0, 1:].eq(-1).all()
    assert torch.equal(kc[:, 0].cpu().view(torch.int16), k_new[:, 0].view(torch.int16))   # identity rotation
    o = out.cpu()
    for h in range(24):
        assert torch.equal(o[:, h].view(torch.int16), v_new[:, 0, h // 12].view(torch.int16)), h
    qd = q_raw[:, 0].double()                                      # [B, 24, 256]
    kd = k_new[:, 0].double()                                      # [B, 2, 256]
    logit = torch.einsum("bhd,bhd->bh", qd, kd.repeat_interleave(12, dim=1))
    bound = 2.0 ** -15 * torch.einsum("bhd,bhd->bh", qd.abs(), kd.abs().repeat_interleave(12, dim=1)) + 1e-6
    assert (lse.cpu().double() - logit * scale).abs().le(bound * scale).all()


def test_prefill_from_position_zero_first_row_returns_its_value_row():
    """A prefill of the first 300 tokens: the rows of block 0 select the own
    block alone ([0, -1, ...]); row 0 attends only token 0, whose rotation is
    the identity, so every head of KV group g returns V[0, g] bit for bit and
    the LSE is the scaled logit q.k (within 2^-15 sum |q k|).  Two streams
    and two query chunks, so the side-stream order is on the path too."""
    say("prefill_layer from position 0")
    B, T, budget = 2, 300, 64
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator().manual_seed(8)
    q_raw = torch.randn((B, T, 24, 256), generator=g).to(bf)
    k_new = torch.randn((B, T, 2, 256), generator=g).to(bf)
    v = torch.randn((B, T, 2, 256), generator=g).to(bf)
    q_idx = (torch.randn((B, T, 4, 128), generator=g) / math.sqrt(128)).to(bf)
    k_idx = (torch.randn((B, T, 128), generator=g) / math.sqrt(128)).to(bf)
    kc = torch.zeros((B, T, 2, 256), dtype=bf, device=dev)
    kb = torch.zeros((B, T // 4 + 1, 128), dtype=bf, device=dev)
    out = torch.empty((B, T, 24, 256), dtype=bf, device=dev)
    lse = torch.empty((B, T, 24), dtype=torch.float32, device=dev)
    bufs = qsa.PrefillBuffers(B, T, 0, budget, 160)
    scale = 1.0 / math.sqrt(256)
    qsa.prefill_layer(q_raw.to(dev), k_new.to(dev), q_idx.to(dev), k_idx.to(dev), kc, v.to(dev), kb, 0, budget, out,
                      lse, bufs, torch.empty((B, T, 24, 256), dtype=bf, device=dev), side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    sel = bufs.sel.cpu()
    assert sel[:, :4, 0].eq(0).all() and sel[:, :4, 1:].eq(-1).all()
    assert torch.equal(kc[:, 0].cpu().view(torch.int16), k_new[:, 0].view(torch.int16))   # identity rotation
    o = out[:, 0].cpu()
    for h in range(24):
        assert torch.equal(o[:, h].view(torch.int16), v[:, 0, h // 12].view(torch.int16)), h
    qd = q_raw[:, 0].double()
    kd = k_new[:, 0].double().repeat_interleave(12, dim=1)
    logit = (qd * kd).sum(-1)
    bound = 2.0 ** -15 * (qd.abs() * kd.abs()).sum(-1) + 1e-6
    assert (lse[:, 0].cpu().double() - logit * scale).abs().le(bound * scale).all()
