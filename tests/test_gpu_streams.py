"""The two-stream prefill order (each query chunk's index-select on a second
stream, its attention on the caller's stream after an event of that
selection) against the one-stream order: selections and outputs bit for bit.
"""

import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from block_sparse_long_12_amd import qsa
from tests.gpu_common import DevicePrefill, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,ctx,T,chunk,budget", [(1, 40000, 2048, 512, 64), (2, 12000, 1500, 512, 512),
                                                   (1, 70000, 1536, 512, 512)],     # fused index-select path
                         ids=["exact-ctx40000", "exact-ctx12000", "fused-ctx70000"])
def test_two_stream_prefill_matches_one_stream(B, ctx, T, chunk, budget):
    say(f"two-stream prefill B={B} ctx={ctx} T={T} chunk={chunk} budget={budget}")
    x = I.make_inputs(I.custom_workload("prefill", B, ctx, T, budget, seed=11, chunk=chunk))
    dp = DevicePrefill(x)
    dp.run()
    sel1, out1, lse1 = dp.bufs.sel.clone(), dp.out.clone(), dp.lse.clone()
    dp2 = DevicePrefill(x)
    side = torch.cuda.Stream()
    qsa.prefill_layer(dp2.q_raw, dp2.k_new, dp2.q_idx, dp2.k_idx, dp2.k_cache, dp2.v_cache, dp2.kbar, ctx, budget,
                      dp2.out, dp2.lse, dp2.bufs, dp2.q_rot, side_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(dp2.bufs.sel, sel1)
    assert torch.equal(dp2.out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(dp2.lse, lse1)
