"""Parity at the full sizes of the benchmark configurations, run the way
bench.py times them (the same entry points, query chunking and buffers):
seeded samples of query rows plus every planted needle of the prefills, and
every row of the 1M-context decode, against the oracle row by row with the
end-to-end protocol of gpu_common.compare_rows."""

import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from tests.gpu_common import DeviceDecode, DevicePrefill, compare_rows, oracle_layer, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _prefill_sampled(name: str, n_rows: int):
    wl = I.WORKLOADS[name]
    assert wl.batch == 1
    say(f"full-size {wl.name}: generating inputs")
    x = I.make_inputs(wl)
    dp = DevicePrefill(x)
    say(f"  running the layer ({wl.tq} new tokens, {wl.chunk}-query chunks)")
    dp.run()
    rows = sorted(set(I.sample_rows(wl, n_rows) + [(int(b), int(t)) for b, t, _ in x.needles]))
    at = {r: k for k, r in enumerate(rows)}
    idx = torch.tensor([t - wl.ctx for _, t in rows], device="cuda")
    sel = dp.bufs.sel[0].index_select(0, idx).cpu().numpy()
    out = dp.out[0].index_select(0, idx).float().cpu().numpy()
    lse = dp.lse[0].index_select(0, idx).cpu().numpy()
    del dp
    torch.cuda.empty_cache()
    say(f"  oracle on {len(rows)} rows")
    layer = oracle_layer(x)
    compare_rows(layer, x, rows, None, lambda b, t: sel[at[(b, t)]], lambda b, t: out[at[(b, t)]],
                 lambda b, t: lse[at[(b, t)]])


def test_full_size_prefill_1M_context_chunk_sampled_rows():
    _prefill_sampled("prefill_prefix943718_chunk104858", 48)


def test_full_size_prefill_T131072_sampled_rows():
    _prefill_sampled("prefill_T131072", 64)


def test_full_size_decode_B4_ctx1M_every_row():
    wl = I.WORKLOADS["decode_B4_ctx1M"]
    say(f"full-size {wl.name}: generating inputs")
    x = I.make_inputs(wl)
    dd = DeviceDecode(x)
    dd.run()
    o = wl.ctx // 4
    scores = dd.scores[:, 0, :o].cpu().numpy()
    sel = dd.sel.cpu().numpy()
    out = dd.out.float().cpu().numpy()
    lse = dd.lse.cpu().numpy()
    del dd
    torch.cuda.empty_cache()
    layer = oracle_layer(x)
    rows = [(b, wl.ctx) for b in range(wl.batch)]
    compare_rows(layer, x, rows, lambda b, t: scores[b], lambda b, t: sel[b, 0],
                 lambda b, t: out[b], lambda b, t: lse[b])
