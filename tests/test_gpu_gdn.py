"""Gated DeltaNet token mixer on the GPU against the float64 oracle.

Prefill runs the chunk-parallel form (bf16 matrix-core products with fp32
accumulation, an fp32 inverse of the triangular system, fp32 state).  Its
tolerance comes from that arithmetic: tests/gdn_emulation.py rounds to bf16
wherever the kernel does (normalised q and k, P, -Wk, the state as a
matrix-core operand, W and its decayed copy, the output), and on these very
inputs that model lies at most 0.049 x rms(o) from the exact recurrence
(mean 0.0029 x rms; state 0.034 / 0.0018 x rms), flat in the length because
the decay forgets old errors (tests/test_gdn_emulation.py, CPU).  The bounds
below are 0.08 / 0.008 x rms for outputs and 0.06 / 0.006 x rms for the state.
Each prefill is also held to the model itself: the GPU may not stray further
from it than the model strays from the exact recurrence.
The decode step applies the recurrence itself in fp32, so only the bf16
rounding of its output (2^-9 relative) and fp32 sums separate it from the
oracle.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from block_sparse_long_12_amd import qsa
from oracle import gdn_oracle as G
from tests import gdn_emulation as E
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _close(got, ref, what, max_rel=0.08, mean_rel=0.008):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(np.asarray(got, np.float64) - ref)
    say(f"  {what}: max {float(err.max()) / rms:.4f} rms, mean {float(err.mean()) / rms:.5f} rms")
    assert err.max() <= max_rel * rms and err.mean() <= mean_rel * rms, \
        (what, float(err.max()) / rms, float(err.mean()) / rms)


def _near_model(got, x, b, heads, what):
    """The GPU outputs / final state of sequence b against the rounding model
    on the same inputs: max |GPU - model| at most max |model - exact|."""
    q, k, v = (G.bf16_to_f64(_bits(t[b])) for t in (x.q, x.k, x.v))
    r = E.emulate(q, k, v, x.g[b].numpy(), x.beta[b].numpy(), x.s0[b].double().numpy(), heads)
    for h in heads:
        qp, kp = G.prepare_qk(q[:, h // 3], k[:, h // 3])
        o_ref, s_ref = G.gated_delta_rule(qp, kp, v[:, h], x.g[b, :, h].double().numpy(),
                                          x.beta[b, :, h].double().numpy(), x.s0[b, h].double().numpy())
        o_gpu, s_gpu = got(h)
        o_mod, s_mod = r[h]
        for name, g_, m_, e_ in (("outputs", o_gpu, o_mod, o_ref), ("state", s_gpu, s_mod, s_ref)):
            d_gm = float(np.abs(np.asarray(g_, np.float64) - m_).max())
            d_me = float(np.abs(m_ - e_).max())
            say(f"  {what} b={b} head {h} {name}: |gpu - model| {d_gm:.3g}, |model - exact| {d_me:.3g}")
            assert d_gm <= d_me, (what, b, h, name, d_gm, d_me)


def _dev(x):
    return [t.cuda() for t in (x.q, x.k, x.v, x.g, x.beta)]


def _oracle(x, lo=0, hi=None):
    sl = slice(lo, hi)
    return G.gdn_layer(_bits(x.q[:, sl]), _bits(x.k[:, sl]), _bits(x.v[:, sl]), x.g[:, sl].numpy(),
                       x.beta[:, sl].numpy(), x.s0.numpy())


@pytest.mark.parametrize("B,T", [(2, 1), (2, 63), (2, 64), (1, 130), (2, 700)])
def test_gdn_prefill_matches_the_oracle(B, T):
    say(f"gdn prefill B={B} T={T}")
    x = I.make_gdn_inputs(B, T, seed=T)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    out = torch.empty_like(v)
    qsa.gdn_prefill(q, k, v, g, beta, state, out, qsa.gdn_prefill_workspace(B, T))
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    o_gpu, s_gpu = out.float().cpu().numpy(), state.cpu().numpy()
    _close(o_gpu, o_ref, "outputs")
    _close(s_gpu, s_ref, "state", 0.06, 0.006)
    for b in range(B):
        _near_model(lambda h: (o_gpu[b, :, h], s_gpu[b, h]), x, b, [0, 1, 23, 47], f"T={T}")


def test_gdn_prefill_calls_chain_through_the_state():
    """Two calls of 130 and 170 tokens equal one of 300 (both held to the oracle)."""
    B, T = 1, 300
    say("gdn prefill in two calls")
    x = I.make_gdn_inputs(B, T, seed=5)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    out = torch.empty_like(v)
    ws = qsa.gdn_prefill_workspace(B, 170)
    for lo, hi in ((0, 130), (130, 300)):
        qsa.gdn_prefill(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], g[:, lo:hi], beta[:, lo:hi], state,
                        out[:, lo:hi], ws)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _close(out.float().cpu().numpy(), o_ref, "outputs")
    _close(state.cpu().numpy(), s_ref, "state", 0.06, 0.006)


def test_gdn_decode_steps_match_the_oracle():
    B, steps = 3, 4
    say("gdn decode")
    x = I.make_gdn_inputs(B, steps, seed=21, state_sigma=0.3)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    outs = []
    for t in range(steps):
        o = torch.empty((B, 48, 128), dtype=torch.bfloat16, device="cuda")
        qsa.gdn_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), g[:, t].contiguous(),
                       beta[:, t].contiguous(), state, o)
        outs.append(o)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    got = torch.stack(outs, 1).float().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(o_ref) + 1e-6
    assert np.all(np.abs(got - o_ref) <= bound), float(np.max(np.abs(got - o_ref) - bound))
    s = state.cpu().numpy()
    assert np.allclose(s, s_ref, rtol=1e-5, atol=1e-5 * float(np.sqrt(np.mean(s_ref ** 2))))


def test_gdn_prefill_then_decode():
    B, T, steps = 2, 130, 3
    say("gdn prefill then decode")
    x = I.make_gdn_inputs(B, T + steps, seed=31)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    out = torch.empty_like(v)
    qsa.gdn_prefill(q[:, :T], k[:, :T], v[:, :T], g[:, :T], beta[:, :T], state, out[:, :T],
                    qsa.gdn_prefill_workspace(B, T))
    for t in range(T, T + steps):
        o = torch.empty((B, 48, 128), dtype=torch.bfloat16, device="cuda")
        qsa.gdn_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), g[:, t].contiguous(),
                       beta[:, t].contiguous(), state, o)
        out[:, t] = o
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _close(out.float().cpu().numpy(), o_ref, "outputs")
    _close(state.cpu().numpy(), s_ref, "state", 0.06, 0.006)


def test_gdn_prefill_over_several_workspace_segments():
    """32838 tokens (513 chunks: two workspace segments) on one sequence;
    two V heads (first and last) held to the oracle on the final state, the
    last chunk and a sample of tokens."""
    B, T = 1, 512 * 64 + 70
    say(f"gdn prefill T={T}")
    x = I.make_gdn_inputs(B, T, seed=41)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    out = torch.empty_like(v)
    qsa.gdn_prefill(q, k, v, g, beta, state, out, qsa.gdn_prefill_workspace(B, T))
    torch.cuda.synchronize()
    qf = G.bf16_to_f64(_bits(x.q[0]))
    kf = G.bf16_to_f64(_bits(x.k[0]))
    rows = np.r_[np.arange(0, T, 997), np.arange(T - 64, T)]
    for h in (0, 47):
        qp, kp = G.prepare_qk(qf[:, h // 3], kf[:, h // 3])
        o_ref, s_ref = G.gated_delta_rule(qp, kp, G.bf16_to_f64(_bits(x.v[0, :, h])), x.g[0, :, h].double().numpy(),
                                          x.beta[0, :, h].double().numpy(), x.s0[0, h].double().numpy())
        got = out[0, :, h].float().cpu().numpy()
        _close(got[rows], o_ref[rows], f"outputs head {h}")
        _close(state[0, h].cpu().numpy(), s_ref, f"state head {h}", 0.06, 0.006)


def test_gdn_prefill_over_four_segments_equals_chained_calls():
    """98374 tokens (1538 chunks: three full workspace segments of 512 chunks
    and a 2-chunk tail, so segment s + 1's prep writes the workspace half
    segment s - 1's state pass read) equal four chained calls of at most 512 chunks (each a
    single segment) bit for bit, outputs and state; two heads are held to
    the oracle and to the rounding model."""
    B, T = 1, 3 * 512 * 64 + 70
    say(f"gdn prefill T={T}, one call against chained calls")
    x = I.make_gdn_inputs(B, T, seed=43)
    q, k, v, g, beta = _dev(x)
    state = x.s0.cuda()
    out = torch.empty_like(v)
    qsa.gdn_prefill(q, k, v, g, beta, state, out, qsa.gdn_prefill_workspace(B, T))
    state_c = x.s0.cuda()
    out_c = torch.empty_like(v)
    seg = 512 * 64
    ws = qsa.gdn_prefill_workspace(B, seg)
    for lo in range(0, T, seg):
        hi = min(T, lo + seg)
        qsa.gdn_prefill(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], g[:, lo:hi], beta[:, lo:hi], state_c,
                        out_c[:, lo:hi], ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(state.view(torch.int32), state_c.view(torch.int32))
    qf = G.bf16_to_f64(_bits(x.q[0]))
    kf = G.bf16_to_f64(_bits(x.k[0]))
    rows = np.r_[np.arange(0, T, 1999), np.arange(T - 64, T)]
    o_all = out[0].float().cpu().numpy()
    s_all = state[0].cpu().numpy()
    for h in (7, 40):
        qp, kp = G.prepare_qk(qf[:, h // 3], kf[:, h // 3])
        o_ref, s_ref = G.gated_delta_rule(qp, kp, G.bf16_to_f64(_bits(x.v[0, :, h])), x.g[0, :, h].double().numpy(),
                                          x.beta[0, :, h].double().numpy(), x.s0[0, h].double().numpy())
        _close(o_all[rows, h], o_ref[rows], f"outputs head {h}")
        _close(s_all[h], s_ref, f"state head {h}", 0.06, 0.006)
    _near_model(lambda h: (o_all[:, h], s_all[h]), x, 0, [7, 40], f"T={T}")
