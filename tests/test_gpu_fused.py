"""Fused fast paths against the primitive chain, bit for bit.

The fused decode index-select and the one-call decode step must produce the
same scores, selection, output and LSE bits as rope_apply + index_scores +
select_topk + sparse_attn_decode on the same inputs, including score patterns
that overflow the fused path's candidate capacity (exact fallback), and must
leave their workspace zeroed for the next call.  The fused prefill
index-select must give the selection of index_scores + select_topk on its
fast path, on every fallback trigger (tie floods, a sample that overstates
the tail) and on the shapes that bypass it, with a reused workspace.
"""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from block_sparse_long_12_amd import qsa
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

# the decode workspaces start with 16 control words for each of the most rows
# a call can have (256 sequences x 4 tokens); they must be zero between calls
CTRL_BYTES = 256 * 4 * 16 * 4


def _rand(shape, seed, sigma):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(torch.bfloat16)


def _kbar(kind, B, nblk, seed):
    if kind == "normal":
        return _rand((B, nblk, 128), seed, 1 / math.sqrt(512))
    if kind == "equal":          # every block scores the same: exact ties everywhere
        row = _rand((1, 1, 128), seed, 1 / math.sqrt(512))
        return row.expand(B, nblk, 128).contiguous()
    if kind == "few_values":     # 5 distinct keys: huge tie groups at the threshold
        rows = _rand((5, 128), seed, 1 / math.sqrt(512))
        idx = torch.from_numpy(np.random.default_rng(seed).integers(0, 5, (B, nblk)))
        return rows[idx]
    raise ValueError(kind)


CASES = [("normal", [1048576 // 16, 70001, 4096 + 3], 512), ("normal", [9000, 9001, 9002], 64),
         ("normal", [1048576, 1048575, 1048579], 512),      # own block 262144 / 262143: bitmap edge
         ("equal", [40000, 40000, 40000], 512), ("few_values", [50000, 12345, 8000], 512),
         ("normal", [100, 2047, 2048], 512), ("normal", [3, 50000, 7], 1), ("normal", [20000, 1, 20001], 2),
         ("normal", [200000, 262144, 300001], 512),       # long rows of different lengths
         ("normal", [1048576, 1048576, 1048576, 1048576], 1024),
         ("normal", [65536, 65537, 65540, 65543], 64),
         ("equal", [70000, 70000, 70000], 512),               # every key equal: the threshold bin overflows
         ("few_values", [80000, 66000], 512),                 # tie groups of thousands at the threshold
         ("normal", [28000] * 40, 2048),        # 40 rows: two-step scan waves keep > 64 (the exact key search)
         ("normal", [1048576] * 4, 2048)]       # the largest budget at 1M context


@pytest.mark.parametrize("kind,pos,budget", CASES, ids=[f"{k}-{p[0]}-{b}" for k, p, b in CASES])
def test_index_select_decode_matches_primitives(kind, pos, budget):
    say(f"index_select_decode {kind} pos={pos} budget={budget}")
    B = len(pos)
    nblk = max(1, max(pos) // 4)
    q = _rand((B, 1, 4, 128), sum(pos), 1 / math.sqrt(128)).cuda()
    kbar = _kbar(kind, B, nblk, budget).cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.full((B, 1, ld), float("nan"), device="cuda")
    sel_ref = torch.empty((B, 1, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos, s_ref)
    qsa.select_topk(s_ref, pos, budget, sel_ref)
    ws = qsa.index_select_workspace(B)
    for rep in range(2):                     # the second call reuses the workspace
        s_f = torch.full((B, 1, ld), float("nan"), device="cuda")
        sel_f = torch.empty((B, 1, budget), dtype=torch.int32, device="cuda")
        qsa.index_select_decode(q, kbar, pos, budget, s_f, sel_f, ws)
        torch.cuda.synchronize()
        for b in range(B):
            o = pos[b] // 4
            assert torch.equal(s_f[b, 0, :o].view(torch.int32), s_ref[b, 0, :o].view(torch.int32)), (rep, b)
        assert torch.equal(sel_f, sel_ref), rep
        # the control words (the head of the workspace) are left zeroed; the
        # candidate lists after them are scratch
        assert int(ws[:CTRL_BYTES].count_nonzero()) == 0, "control words not left zeroed"


# (kind, positions, budget, rows expected on the exact path): random scores
# at long context, one to four sequences and the largest budget, must all
# stay on the candidate lists (the scan's plan sizes the waves and the lists
# for them); equal keys send every row to the exact path
FAST_CASES = [("normal", [1048576], 512, 0), ("normal", [1048576, 1048579], 512, 0),
              ("normal", [1048576, 1000000, 1048575], 512, 0), ("normal", [1048576] * 4, 512, 0),
              ("normal", [1048576] * 4, 2048, 0), ("normal", [1048576], 2048, 0), ("normal", [262144], 512, 0),
              ("normal", [131072] * 8, 512, 0), ("normal", [32768] * 32, 512, 0),
              ("equal", [300000, 300000], 512, 2)]


def _boost_recent(q, kbar, pos, n_recent, sigmas):
    """Raise the scores of each sequence's n_recent most recent blocks by
    about `sigmas` standard deviations of its scores (the shape of attention
    that favours the local context), along the sequence's summed query."""
    qf = q.float().sum(dim=2)[:, 0]                          # [B, 128]: the 4 heads summed
    kb = kbar.float()
    for b, p in enumerate(pos):
        o = p // 4
        u = qf[b]
        sd = float(u.norm()) / math.sqrt(512)                 # score spread of N(0, 1/512) block keys
        kb[b, o - n_recent:o] += (sigmas * sd / float(u.dot(u))) * u
    return kb.to(torch.bfloat16)


@pytest.mark.parametrize("pos,budget", [([1048576, 1048576], 512), ([1048576], 2048), ([200000] * 4, 512)])
def test_index_select_decode_recovers_clustered_selections(pos, budget):
    """Selections concentrated in the most recent blocks: the scan's waves
    that hold them list too few, every row leaves the candidate lists, and
    the one-pass recovery over the stored row must still give the primitive
    chain's selection."""
    say(f"index_select_decode clustered B={len(pos)} pos={pos[0]} budget={budget}")
    B = len(pos)
    nblk = max(pos) // 4
    q = _rand((B, 1, 4, 128), 11 + sum(pos), 1 / math.sqrt(128))
    kbar = _boost_recent(q, _kbar("normal", B, nblk, budget + 3), pos, 3000, 4.0).cuda()
    q = q.cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.empty((B, 1, ld), device="cuda")
    sel_ref = torch.empty((B, 1, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos, s_ref)
    qsa.select_topk(s_ref, pos, budget, sel_ref)
    # most of each selection lies in the boosted blocks
    for b in range(B):
        o = pos[b] // 4
        assert int((sel_ref[b, 0] >= o - 3000).sum()) > budget // 2
    ws = qsa.index_select_workspace(B)
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    s_f = torch.empty_like(s_ref)
    sel_f = torch.empty_like(sel_ref)
    qsa.set_decode_fallback_counter(counter)
    try:
        qsa.index_select_decode(q, kbar, pos, budget, s_f, sel_f, ws)
        torch.cuda.synchronize()
    finally:
        qsa.set_decode_fallback_counter(None)
    assert torch.equal(sel_f, sel_ref)
    assert int(counter.item()) == B
    assert int(ws[:CTRL_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("kind,pos,budget,n_exact", FAST_CASES,
                         ids=[f"{k}-{len(p)}x{p[0]}-{b}" for k, p, b, _ in FAST_CASES])
def test_index_select_decode_stays_on_the_candidate_lists(kind, pos, budget, n_exact):
    say(f"index_select_decode fast path {kind} B={len(pos)} pos={pos[0]} budget={budget}")
    B = len(pos)
    nblk = max(pos) // 4
    q = _rand((B, 1, 4, 128), sum(pos) + 1, 1 / math.sqrt(128)).cuda()
    kbar = _kbar(kind, B, nblk, budget + 1).cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.empty((B, 1, ld), device="cuda")
    sel_ref = torch.empty((B, 1, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos, s_ref)
    qsa.select_topk(s_ref, pos, budget, sel_ref)
    ws = qsa.index_select_workspace(B)
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    s_f = torch.empty_like(s_ref)
    sel_f = torch.empty_like(sel_ref)
    qsa.set_decode_fallback_counter(counter)
    try:
        qsa.index_select_decode(q, kbar, pos, budget, s_f, sel_f, ws)
        torch.cuda.synchronize()
    finally:
        qsa.set_decode_fallback_counter(None)
    assert torch.equal(sel_f, sel_ref)
    assert int(counter.item()) == n_exact
    assert int(ws[:CTRL_BYTES].count_nonzero()) == 0


def test_scan_timing_hook_times_the_scan_and_changes_nothing():
    """With the measurement hook set, the decode index-select records the two
    events around its scan launch (a positive elapsed time no longer than the
    whole call) and returns the same scores and selection bit for bit."""
    say("scan timing hook")
    pos, budget = [70001, 130000], 512
    B, nblk = len(pos), max(pos) // 4
    q = _rand((B, 1, 4, 128), 5, 1 / math.sqrt(128)).cuda()
    kbar = _kbar("normal", B, nblk, 6).cuda()
    ld = (nblk + 3) // 4 * 4
    ws = qsa.index_select_workspace(B)
    outs = []
    for hooked in (False, True):
        s_f = torch.full((B, 1, ld), float("nan"), device="cuda")
        sel_f = torch.empty((B, 1, budget), dtype=torch.int32, device="cuda")
        b_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b_ev.record()
        e_ev.record()
        torch.cuda.synchronize()
        if hooked:
            qsa.set_scan_timing_events(b_ev, e_ev)
        try:
            c0.record()
            qsa.index_select_decode(q, kbar, pos, budget, s_f, sel_f, ws)
            c1.record()
            torch.cuda.synchronize()
        finally:
            qsa.set_scan_timing_events(None, None)
        if hooked:
            scan_ms, call_ms = b_ev.elapsed_time(e_ev), c0.elapsed_time(c1)
            assert 0.0 < scan_ms <= call_ms, (scan_ms, call_ms)
        outs.append((s_f, sel_f))
    for b in range(B):
        o = pos[b] // 4
        assert torch.equal(outs[0][0][b, 0, :o].view(torch.int32), outs[1][0][b, 0, :o].view(torch.int32))
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("ctx,budget,B", [(32768, 512, 8), (5001, 64, 3), (99, 512, 2), (131072, 512, 2)])
def test_decode_step_matches_primitives(ctx, budget, B):
    say(f"decode_step ctx={ctx} budget={budget} B={B}")
    wl = I.custom_workload("decode", batch=B, ctx=ctx, tq=1, budget=budget, n_needles=2, seed=ctx)
    x = I.make_inputs(wl)
    dev = "cuda"

    def caches():
        kc = x.k.to(dev)
        qsa.rope_apply(kc[:, :ctx], [0] * B)
        ki = x.k_idx.to(dev)
        kb = torch.zeros((B, max(1, (ctx + 1) // 4), 128), dtype=torch.bfloat16, device=dev)
        if ctx // 4:
            qsa.compress_block_keys(ki, 0, ctx // 4, kb)
        return kc, ki, kb

    ld = max(4, (ctx // 4 + 3) // 4 * 4)
    outs = []
    for fused in (False, True):
        kc, ki, kb = caches()
        v = x.v.to(dev)
        scores = torch.full((B, 1, ld), float("nan"), device=dev)
        sel = torch.empty((B, 1, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
        q_raw, k_new, q_idx = x.q.to(dev), x.k[:, ctx:ctx + 1].contiguous().to(dev), x.q_idx.to(dev)
        if fused:
            ws = qsa.decode_step_workspace(B, budget)
            for _ in range(2):
                qsa.decode_step(q_raw, k_new, q_idx, ki, kc, v, kb, ctx, budget, out, lse, scores, sel, ws)
        else:
            ws = qsa.decode_workspace(B, budget)
            qsa.decode_step_primitives(q_raw, k_new, q_idx, ki, kc, v, kb, ctx, budget, out, lse, scores, sel, ws,
                                       torch.empty_like(q_raw))
        torch.cuda.synchronize()
        outs.append((kc[:, ctx].clone(), scores[:, 0, :ctx // 4].clone(), sel.clone(), out.clone(), lse.clone()))
    for name, a, b in zip(("k row", "scores", "sel", "out", "lse"), outs[0], outs[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


# ---------------------------------------------------------------- prefill index-select

SAMPLE_RUNS, RUN_LEN = 256, 16    # the fused prefill index-select samples 256 runs of 16 blocks per row


def _run_starts(omin):
    """First block of each sampled run (spread evenly over [0, omin))."""
    return [r * (omin - RUN_LEN) // (SAMPLE_RUNS - 1) for r in range(SAMPLE_RUNS)]


def _prefill_kbar(kind, B, nblk, seed, pos0):
    if kind in ("normal", "equal", "few_values"):
        return _kbar(kind, B, nblk, seed)
    if kind == "sample_high":    # the sampled runs outrank the rest: the sample overstates the tail
        kb = _rand((B, nblk, 128), seed, 1 / math.sqrt(512)) * 0.01
        for b in range(B):
            for s in _run_starts(pos0[b] // 4):
                kb[b, s:s + RUN_LEN] = kb[b, s:s + RUN_LEN] * 100 + 0.05
        return kb.to(torch.bfloat16)
    raise ValueError(kind)


PREFILL_CASES = [
    ("normal", [70000, 70000], 700, 512, "fused"),
    ("normal", [70000, 91003], 333, 64, "fused"),
    ("normal", [80000], 1000, 1024, "fused"),
    ("normal", [80000], 200, 1025, "unfused"),
    ("normal", [30000], 300, 512, "unfused"),
    ("equal", [70000, 70000], 300, 512, "fallback"),
    # every one of 2600 rows flagged: the fallback redoes 5822 row tiles of
    # scores and 2600 row selections
    ("equal", [70000], 2600, 512, "fallback"),
    ("few_values", [66000], 500, 512, "either"),
    ("sample_high", [160000], 256, 512, "fallback"),
]


@pytest.mark.parametrize("kind,pos0,tq,budget,path", PREFILL_CASES,
                         ids=[f"{c[0]}-{c[1][0]}-{c[2]}-{c[3]}" for c in PREFILL_CASES])
def test_index_select_prefill_matches_primitives(kind, pos0, tq, budget, path):
    say(f"index_select_prefill {kind} pos0={pos0} tq={tq} budget={budget} ({path})")
    B = len(pos0)
    nblk = max((p + tq - 1) // 4 for p in pos0) + 1
    q = _rand((B, tq, 4, 128), tq + budget, 1 / math.sqrt(128)).cuda()
    if kind == "sample_high":    # every query row leans the same way so the high blocks rank first
        q = (q.float() * 0.1 + 0.05).to(torch.bfloat16)
    kbar = _prefill_kbar(kind, B, nblk, budget, pos0).cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.empty((B, tq, ld), device="cuda")
    sel_ref = torch.empty((B, tq, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos0, s_ref)
    qsa.select_topk(s_ref, pos0, budget, sel_ref)
    ws = qsa.index_select_prefill_workspace(B, tq)
    ws.fill_(0xA5)                                    # no initialisation is required
    for rep in range(2):                              # the second call reuses the workspace
        scratch = torch.empty((B, tq, ld), device="cuda")
        sel = torch.full((B, tq, budget), -7, dtype=torch.int32, device="cuda")
        qsa.index_select_prefill(q, kbar, pos0, budget, scratch, sel, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), (rep, int((sel != sel_ref).any(dim=-1).sum()))
        if path != "unfused":
            n_flagged = int(ws[:4].view(torch.int32)[0])
            say(f"  rows taking the exact fallback: {n_flagged} of {B * tq}")
            if path == "fused":
                assert n_flagged == 0
            elif path == "fallback":
                assert n_flagged > 0


def test_index_select_prefill_clustered_scores_stay_fused():
    """Every query shares a component along which the 3000 blocks before the
    chunk score about 4 standard deviations high (most selections then lie
    there, as with attention that favours the recent context): the sample of
    short runs spread over the blocks still sets thresholds that hold the
    selections, so no row takes the exact fallback."""
    pos0, tq, budget = [120000], 512, 512
    say(f"index_select_prefill clustered pos0={pos0} tq={tq} budget={budget}")
    B = len(pos0)
    nblk = (pos0[0] + tq - 1) // 4 + 1
    q = _rand((B, tq, 4, 128), 21, 1 / math.sqrt(128)).float()
    g = torch.Generator().manual_seed(22)
    c = torch.randn(128, generator=g)
    qn = float(q.sum(dim=2)[0].norm(dim=-1).mean())
    c = c / c.norm() * (0.5 * qn)
    q[:, :, 0, :] += c
    kb = _kbar("normal", B, nblk, 23).float()
    o = pos0[0] // 4
    kb[0, o - 3000:o] += (4.0 * qn / math.sqrt(512) / float(c.dot(c))) * c
    q, kbar = q.to(torch.bfloat16).cuda(), kb.to(torch.bfloat16).cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.empty((B, tq, ld), device="cuda")
    sel_ref = torch.empty((B, tq, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos0, s_ref)
    qsa.select_topk(s_ref, pos0, budget, sel_ref)
    assert float((sel_ref >= o - 3000).float().mean()) > 0.5     # the cluster holds most selections
    ws = qsa.index_select_prefill_workspace(B, tq)
    sel = torch.full((B, tq, budget), -7, dtype=torch.int32, device="cuda")
    qsa.index_select_prefill(q, kbar, pos0, budget, torch.empty((B, tq, ld), device="cuda"), sel, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_ref)
    assert int(ws[:4].view(torch.int32)[0]) == 0                 # rows on the exact fallback


def test_index_select_prefill_workspace_reuse_across_shapes():
    say("index_select_prefill: one workspace, shapes that change between calls")
    ws = qsa.index_select_prefill_workspace(2, 600)
    for (kind, pos0, tq, budget) in [("equal", [70000, 70000], 600, 512), ("normal", [72000], 250, 512),
                                     ("normal", [70000, 75000], 600, 300)]:
        B = len(pos0)
        nblk = max((p + tq - 1) // 4 for p in pos0) + 1
        q = _rand((B, tq, 4, 128), tq, 1 / math.sqrt(128)).cuda()
        kbar = _prefill_kbar(kind, B, nblk, 3, pos0).cuda()
        ld = (nblk + 3) // 4 * 4
        s_ref = torch.empty((B, tq, ld), device="cuda")
        sel_ref = torch.empty((B, tq, budget), dtype=torch.int32, device="cuda")
        qsa.index_scores(q, kbar, pos0, s_ref)
        qsa.select_topk(s_ref, pos0, budget, sel_ref)
        sel = torch.empty_like(sel_ref)
        qsa.index_select_prefill(q, kbar, pos0, budget, torch.empty_like(s_ref), sel, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), (kind, pos0, tq)


# ---------------------------------------------------------------- serving decode step

@pytest.mark.parametrize("pos,budget", [([4099, 9000, 4103], 512), ([20003, 7, 65539], 64), ([3, 1, 2], 8)])
def test_decode_step_appends_rows_and_compresses(pos, budget):
    """The one-call step with the new V and indexer-key rows and per-sequence
    positions equals the primitive chain bit for bit, including the rows it
    appends and the block key it writes when a new token completes a block."""
    say(f"decode_step serving pos={pos} budget={budget}")
    B = len(pos)
    L = max(pos) + 1
    wl = I.custom_workload("decode", batch=B, ctx=L - 1, tq=1, budget=budget, n_needles=0, seed=sum(pos))
    x = I.make_inputs(wl)
    dev = "cuda"
    g = torch.Generator().manual_seed(5)
    v_new = (torch.randn((B, 1, 2, 256), generator=g)).to(torch.bfloat16).to(dev)
    k_idx_new = (torch.randn((B, 1, 128), generator=g) / math.sqrt(128)).to(torch.bfloat16).to(dev)
    k_new = (torch.randn((B, 1, 2, 256), generator=g)).to(torch.bfloat16).to(dev)
    ld = max(4, (L // 4 + 3) // 4 * 4)
    outs = []
    for fused in (False, True):
        kc = x.k.to(dev)
        qsa.rope_apply(kc, [0] * B)
        v = x.v.to(dev)
        ki = x.k_idx.to(dev)
        for b in range(B):                            # the rows the step must write hold garbage
            kc[b, pos[b]] = 7.0
            v[b, pos[b]] = -3.0
            ki[b, pos[b]] = 5.0
        kb = torch.full((B, L // 4 + 1, 128), 9.0, dtype=torch.bfloat16, device=dev)
        for b in range(B):
            if pos[b] // 4:
                qsa.compress_block_keys(ki[b:b + 1], 0, pos[b] // 4, kb[b:b + 1])
        scores = torch.full((B, 1, ld), float("nan"), device=dev)
        sel = torch.empty((B, 1, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, 24, 256), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, 24), dtype=torch.float32, device=dev)
        q_raw, q_idx = x.q.to(dev), x.q_idx.to(dev)
        if fused:
            qsa.decode_step(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel,
                            qsa.decode_step_workspace(B, budget), v_new=v_new, k_idx_new=k_idx_new)
        else:
            qsa.decode_step_primitives(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel,
                                       qsa.decode_workspace(B, budget), torch.empty_like(q_raw), v_new=v_new,
                                       k_idx_new=k_idx_new)
        torch.cuda.synchronize()
        rows = [(kc[b, pos[b]].clone(), v[b, pos[b]].clone(), ki[b, pos[b]].clone(), kb[b].clone(),
                 scores[b, 0, :pos[b] // 4].clone(), sel[b].clone()) for b in range(B)]
        outs.append((rows, out.clone(), lse.clone()))
    (ra, oa, la), (rb, ob, lb) = outs
    for b in range(B):
        for name, a, c in zip(("k row", "v row", "k_idx row", "kbar", "scores", "sel"), ra[b], rb[b]):
            assert torch.equal(a.view(torch.uint8), c.view(torch.uint8)), (b, name)
        assert torch.equal(rb[b][1], v_new[b, 0]) and torch.equal(rb[b][2], k_idx_new[b, 0]), b
        if (pos[b] + 1) % 4 == 0:                     # the completed block was written, the next one not
            assert not torch.equal(rb[b][3][pos[b] // 4], torch.full_like(rb[b][3][0], 9.0)), b
    assert torch.equal(oa.view(torch.uint8), ob.view(torch.uint8))
    assert torch.equal(la.view(torch.uint8), lb.view(torch.uint8))


# ---------------------------------------------------------------- several decode tokens per sequence

MULTI_STEP_CASES = [([4097, 9000, 70001], 4, 512, False), ([4099, 8191], 2, 512, False),
                    ([131069, 131072], 3, 512, False), ([1, 6], 4, 8, False),
                    ([262143, 300001], 3, 512, True), ([5, 9000], 2, 64, True),
                    # the most rows a step takes (256 sequences of 4 tokens: one attention split
                    # per row), the shorter rows keeping every candidate
                    ([2000 + 7 * b for b in range(256)], 4, 512, False)]


@pytest.mark.parametrize("pos,tq,budget,yarn", MULTI_STEP_CASES,
                         ids=[f"B{len(c[0])}-pos{c[0][0]}-tq{c[1]}-b{c[2]}{'-yarn' if c[3] else ''}"
                              for c in MULTI_STEP_CASES])
def test_multi_token_decode_step_matches_primitives(pos, tq, budget, yarn):
    """tq new tokens per sequence in one step (one pass over the block keys
    scores every token) equal the primitive chain bit for bit: the appended
    rows, the key of every block a new token completes (a later token of the
    same step scores it), scores, selections, outputs and LSEs.  yarn: the
    step rotates q and the new K rows with the static-YaRN table."""
    say(f"multi-token decode_step pos={pos} tq={tq} budget={budget} yarn={yarn}")
    rope = qsa.YARN if yarn else None
    B = len(pos)
    L = max(pos) + tq
    dev = "cuda"
    g = torch.Generator().manual_seed(11 + tq)
    bf = torch.bfloat16
    k_cpu = torch.randn((B, L, 2, 256), generator=g).to(bf)
    v_cpu = torch.randn((B, L, 2, 256), generator=g).to(bf)
    ki_cpu = (torch.randn((B, L, 128), generator=g) / math.sqrt(128)).to(bf)
    q_raw = torch.randn((B, tq, 24, 256), generator=g).to(bf).to(dev)
    q_idx = (torch.randn((B, tq, 4, 128), generator=g) / math.sqrt(128)).to(bf).to(dev)
    k_new = torch.randn((B, tq, 2, 256), generator=g).to(bf).to(dev)
    v_new = torch.randn((B, tq, 2, 256), generator=g).to(bf).to(dev)
    k_idx_new = (torch.randn((B, tq, 128), generator=g) / math.sqrt(128)).to(bf).to(dev)
    gate = (torch.randn((B, tq, 24, 256), generator=g) * 3).to(bf).to(dev)    # the output gate too
    ld = max(4, ((L - 1) // 4 + 3) // 4 * 4)
    outs = []
    for fused in (False, True):
        kc, v, ki = k_cpu.to(dev), v_cpu.to(dev), ki_cpu.to(dev)
        qsa.rope_apply(kc, [0] * B, rope=rope)
        kb = torch.full((B, L // 4 + 1, 128), 9.0, dtype=bf, device=dev)
        for b in range(B):
            if pos[b] // 4:
                qsa.compress_block_keys(ki[b:b + 1], 0, pos[b] // 4, kb[b:b + 1])
        scores = torch.full((B, tq, ld), float("nan"), device=dev)
        sel = torch.empty((B, tq, budget), dtype=torch.int32, device=dev)
        out = torch.empty((B, tq, 24, 256), dtype=bf, device=dev)
        lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)
        if fused:
            ws = qsa.decode_step_workspace(B, budget, tq=tq)
            for _ in range(2):                        # the second call reuses the workspace
                qsa.decode_step(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel, ws,
                                v_new=v_new, k_idx_new=k_idx_new, gate=gate, rope=rope)
            assert int(ws[:CTRL_BYTES].count_nonzero()) == 0
        else:
            qsa.decode_step_primitives(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel,
                                       qsa.decode_workspace(B, budget, tq=tq), torch.empty_like(q_raw),
                                       v_new=v_new, k_idx_new=k_idx_new, gate=gate, rope=rope)
        torch.cuda.synchronize()
        per = []
        for b in range(B):
            rows = slice(pos[b], pos[b] + tq)
            per.append((kc[b, rows].clone(), v[b, rows].clone(), ki[b, rows].clone(), kb[b].clone(),
                        [scores[b, t, :(pos[b] + t) // 4].clone() for t in range(tq)], sel[b].clone()))
        outs.append((per, out.clone(), lse.clone()))
    (pa, oa, la), (pb, ob, lb) = outs
    for b in range(B):
        for name, a, c in zip(("k rows", "v rows", "k_idx rows", "kbar", "", "sel"), pa[b], pb[b]):
            if name:
                assert torch.equal(a.view(torch.uint8), c.view(torch.uint8)), (b, name)
        for t in range(tq):
            assert torch.equal(pa[b][4][t].view(torch.int32), pb[b][4][t].view(torch.int32)), (b, t, "scores")
        for x in range(pos[b], pos[b] + tq):          # every completed block was written
            if x % 4 == 3:
                assert not torch.equal(pb[b][3][x // 4], torch.full_like(pb[b][3][0], 9.0)), (b, x)
    assert torch.equal(oa.view(torch.uint8), ob.view(torch.uint8))
    assert torch.equal(la.view(torch.uint8), lb.view(torch.uint8))


@pytest.mark.parametrize("pos,tq,budget", [([70001, 262141], 4, 512), ([5000, 5001, 5002], 3, 64),
                                            # the most rows a call takes: 256 sequences of 4 tokens
                                            ([8000 + 37 * b for b in range(256)], 4, 512)],
                         ids=["B2-tq4", "B3-tq3", "B256-tq4"])
def test_multi_token_index_select_decode_matches_primitives(pos, tq, budget):
    say(f"multi-token index_select_decode pos={pos} tq={tq}")
    B = len(pos)
    nblk = (max(pos) + tq - 1) // 4
    q = _rand((B, tq, 4, 128), sum(pos) + tq, 1 / math.sqrt(128)).cuda()
    kbar = _kbar("normal", B, max(1, nblk), budget).cuda()
    ld = (nblk + 3) // 4 * 4
    s_ref = torch.full((B, tq, ld), float("nan"), device="cuda")
    sel_ref = torch.empty((B, tq, budget), dtype=torch.int32, device="cuda")
    qsa.index_scores(q, kbar, pos, s_ref)
    qsa.select_topk(s_ref, pos, budget, sel_ref)
    ws = qsa.index_select_workspace(B, tq=tq)
    s_f = torch.full((B, tq, ld), float("nan"), device="cuda")
    sel_f = torch.empty((B, tq, budget), dtype=torch.int32, device="cuda")
    qsa.index_select_decode(q, kbar, pos, budget, s_f, sel_f, ws)
    torch.cuda.synchronize()
    for b in range(B):
        for t in range(tq):
            o = (pos[b] + t) // 4
            assert torch.equal(s_f[b, t, :o].view(torch.int32), s_ref[b, t, :o].view(torch.int32)), (b, t)
    assert torch.equal(sel_f, sel_ref)


def test_decode_step_workspace_reused_across_shapes():
    """One decode-step workspace (sized for the largest call) serves steps
    whose row counts grow and shrink (B x tq = 2, 12, 4, 12): every call
    equals the primitive chain bit for bit and leaves the control words
    zeroed, so a call with more rows never reads what a smaller one left."""
    dev, bf, budget = "cuda", torch.bfloat16, 512
    shapes = [([70001, 4099], 1), ([9000, 70001, 4099, 30000], 3), ([4099, 70001], 2), ([30000, 9000, 4099, 70001], 3)]
    ws = qsa.decode_step_workspace(4, budget, tq=3)
    for i, (pos, tq) in enumerate(shapes):
        say(f"decode_step reuse {i}: pos={pos} tq={tq}")
        B = len(pos)
        L = max(pos) + tq
        g = torch.Generator().manual_seed(100 + i)
        k_cpu = torch.randn((B, L, 2, 256), generator=g).to(bf)
        v_cpu = torch.randn((B, L, 2, 256), generator=g).to(bf)
        ki_cpu = (torch.randn((B, L, 128), generator=g) / math.sqrt(128)).to(bf)
        q_raw = torch.randn((B, tq, 24, 256), generator=g).to(bf).to(dev)
        q_idx = (torch.randn((B, tq, 4, 128), generator=g) / math.sqrt(128)).to(bf).to(dev)
        k_new = torch.randn((B, tq, 2, 256), generator=g).to(bf).to(dev)
        ld = max(4, ((L - 1) // 4 + 3) // 4 * 4)
        res = []
        for fused in (False, True):
            kc, v, ki = k_cpu.to(dev), v_cpu.to(dev), ki_cpu.to(dev)
            qsa.rope_apply(kc, [0] * B)
            kb = torch.zeros((B, L // 4 + 1, 128), dtype=bf, device=dev)
            for b in range(B):
                qsa.compress_block_keys(ki[b:b + 1], 0, pos[b] // 4, kb[b:b + 1])
            scores = torch.full((B, tq, ld), float("nan"), device=dev)
            sel = torch.empty((B, tq, budget), dtype=torch.int32, device=dev)
            lead = (B,) if tq == 1 else (B, tq)        # one token: [B, 24, 256] outputs
            out = torch.empty(lead + (24, 256), dtype=bf, device=dev)
            lse = torch.empty(lead + (24,), dtype=torch.float32, device=dev)
            if fused:
                qsa.decode_step(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel, ws)
            else:
                qsa.decode_step_primitives(q_raw, k_new, q_idx, ki, kc, v, kb, pos, budget, out, lse, scores, sel,
                                           qsa.decode_workspace(B, budget, tq=tq), torch.empty_like(q_raw))
            torch.cuda.synchronize()
            res.append((sel.clone(), out.clone(), lse.clone(),
                        [scores[b, t, :(pos[b] + t) // 4].clone() for b in range(B) for t in range(tq)]))
        (sa, oa, la, ca), (sb, ob, lb, cb) = res
        assert torch.equal(sa, sb), i
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), i
        assert torch.equal(la, lb), i
        for x, y in zip(ca, cb):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), i
        assert int(ws[:CTRL_BYTES].count_nonzero()) == 0, i
