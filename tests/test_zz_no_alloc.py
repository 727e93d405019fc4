"""The allocation-free decode step (qsa_decode_step_noalloc, the library's
static per-GPU scratch instead of a workspace) against qsa_decode_step with
its own zeroed workspace: scores, selection, output, LSE and the rows and
block keys it appends, bit for bit, on two calls in a row -- the second with
a smaller input, so it also meets what the first left in the shared scratch."""

import math

import pytest
import torch

from block_sparse_long_12_amd import qsa
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

bf = torch.bfloat16


def _case(pos, tq, seed):
    B = len(pos)
    L = max(pos) + tq
    g = torch.Generator().manual_seed(seed)
    c = dict(
        k=torch.randn((B, L, 2, 256), generator=g).to(bf), v=torch.randn((B, L, 2, 256), generator=g).to(bf),
        ki=(torch.randn((B, L, 128), generator=g) / math.sqrt(128)).to(bf),
        q=torch.randn((B, tq, 24, 256), generator=g).to(bf),
        q_idx=(torch.randn((B, tq, 4, 128), generator=g) / math.sqrt(128)).to(bf),
        k_new=torch.randn((B, tq, 2, 256), generator=g).to(bf), v_new=torch.randn((B, tq, 2, 256), generator=g).to(bf),
        ki_new=(torch.randn((B, tq, 128), generator=g) / math.sqrt(128)).to(bf),
        gate=(torch.randn((B, tq, 24, 256), generator=g) * 3).to(bf))
    return B, L, c


def _run(pos, tq, c, B, L, noalloc, rope):
    dev = "cuda"
    kc, v, ki = c["k"].to(dev), c["v"].to(dev), c["ki"].to(dev)
    qsa.rope_apply(kc, [0] * B, rope=rope)
    kb = torch.zeros((B, L // 4 + 1, 128), dtype=bf, device=dev)
    for b in range(B):
        qsa.compress_block_keys(ki[b:b + 1], 0, pos[b] // 4, kb[b:b + 1])
    ld = max(4, ((L - 1) // 4 + 3) // 4 * 4)
    scores = torch.full((B, tq, ld), float("nan"), device=dev)
    sel = torch.empty((B, tq, 512), dtype=torch.int32, device=dev)
    out = torch.empty((B, tq, 24, 256), dtype=bf, device=dev)
    lse = torch.empty((B, tq, 24), dtype=torch.float32, device=dev)
    args = (c["q"].to(dev), c["k_new"].to(dev), c["q_idx"].to(dev), ki, kc, v, kb, pos, 512, out, lse, scores, sel)
    kw = dict(v_new=c["v_new"].to(dev), k_idx_new=c["ki_new"].to(dev), gate=c["gate"].to(dev), rope=rope)
    if noalloc:
        qsa.decode_step_noalloc(*args, **kw)
    else:
        qsa.decode_step(*args, qsa.decode_step_workspace(B, 512, tq=tq), **kw)
    torch.cuda.synchronize()
    rows = [(kc[b, pos[b]:pos[b] + tq], v[b, pos[b]:pos[b] + tq], ki[b, pos[b]:pos[b] + tq], kb[b])
            for b in range(B)]
    sc = [scores[b, t, :(pos[b] + t) // 4] for b in range(B) for t in range(tq)]
    return sel, out, lse, sc, rows


@pytest.mark.parametrize("calls", [
    [([70001, 4099, 130000, 9000], 3, False), ([4099, 70003], 1, False)],
    [([262143, 300001], 4, True), ([9001], 2, True)],
], ids=["plain", "yarn"])
def test_noalloc_decode_step_equals_decode_step_on_consecutive_calls(calls):
    for i, (pos, tq, yarn) in enumerate(calls):
        say(f"noalloc call {i}: pos={pos} tq={tq} yarn={yarn}")
        rope = qsa.YARN if yarn else None
        B, L, c = _case(pos, tq, seed=7 + i + tq)
        a = _run(pos, tq, c, B, L, False, rope)
        b = _run(pos, tq, c, B, L, True, rope)
        assert torch.equal(a[0], b[0]), "sel"
        assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16)), "out"
        assert torch.equal(a[2], b[2]), "lse"
        for x, y in zip(a[3], b[3]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), "scores"
        for ra, rb in zip(a[4], b[4]):
            for x, y in zip(ra, rb):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "appended rows / block keys"


def test_noalloc_rejects_shapes_beyond_its_scratch():
    B, tq = 64, 4
    dev = "cuda"
    q = torch.zeros((B, tq, 24, 256), dtype=bf, device=dev)
    kc = torch.zeros((B, 8192 + tq, 2, 256), dtype=bf, device=dev)
    with pytest.raises(qsa.QSAError, match="static"):
        qsa.decode_step_noalloc(q, torch.zeros((B, tq, 2, 256), dtype=bf, device=dev),
                                torch.zeros((B, tq, 4, 128), dtype=bf, device=dev), None, kc, torch.zeros_like(kc),
                                torch.zeros((B, 2049, 128), dtype=bf, device=dev), 8192, 512,
                                torch.empty_like(q), None, torch.empty((B, tq, 2052), device=dev),
                                torch.empty((B, tq, 512), dtype=torch.int32, device=dev))
