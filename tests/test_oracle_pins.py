"""Pins of the CPU oracle against facts other than itself.

Each test fixes the oracle to something independent of its own code: values
derived by hand (tests/golden), closed forms, a library routine for a special
case (dense causal attention), or brute force on tiny inputs in plain Python.
"""

import cmath
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

from block_sparse_long_12_amd import inputs as I
from oracle import qsa_oracle as O

GOLD = Path(__file__).parent / "golden"


def _gold(name):
    return json.loads((GOLD / name).read_text())


def _bf16_bits_of_hex(h):
    return O.f64_to_bf16(np.array([float.fromhex(h)]))[0]


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_golden():
    for c in _gold("bf16_rounding.json")["cases"]:
        got = O.f64_to_bf16(np.array([float.fromhex(c["value"])]))[0]
        assert got == int(c["bits"], 16), c


def test_bf16_rounding_matches_torch_cast():
    # torch's float32 -> bf16 cast is an independent round-to-nearest-even
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), ref)


def test_bf16_roundtrip_every_normal_pattern():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (pats >> 7) & 0xFF
    ok = ((exp > 0) & (exp < 0xFF)) | ((pats & 0x7FFF) == 0)
    pats = pats[ok]
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(pats)), pats)


# ---------------------------------------------------------------- rotary

def _rand_bf16(shape, seed, sigma=1.0):
    t = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * sigma)
    return O.bits(t.to(torch.bfloat16))


def test_rope_position_zero_is_identity():
    x = _rand_bf16((5, 3, 256), 1)
    assert np.array_equal(O.rope_rotate(x, np.zeros(5, np.int64)), x)


def test_rope_leaves_dims_past_the_slice():
    x = _rand_bf16((7, 2, 256), 2)
    y = O.rope_rotate(x, np.arange(7) * 1000 + 3)
    assert np.array_equal(y[..., 64:], x[..., 64:])
    assert not np.array_equal(y[..., :64], x[..., :64])


def test_rope_complex_form():
    # rotate-half pair (i, i+32) as the complex number a + ib turned by e^{i pos w_i},
    # w_i = theta^(-i/32), theta = 1e7 and 64 rotary dims (model card rope_parameters:
    # rope_theta 1e7, partial_rotary_factor 0.25 of head dim 256)
    assert 0.25 * 256 == 64
    x = O.bf16_to_f64(_rand_bf16((4, 2, 256), 3))
    pos = np.array([0, 1, 4097, 1048575])
    y = O.rope_rotate_f64(x, pos)
    for ti, p in enumerate(pos):
        for h in range(2):
            for i in range(32):
                w = 1e7 ** (-i / 32.0)
                z = complex(x[ti, h, i], x[ti, h, 32 + i]) * cmath.exp(1j * p * w)
                assert abs(y[ti, h, i] - z.real) < 1e-9 and abs(y[ti, h, 32 + i] - z.imag) < 1e-9


def test_rope_relative_position():
    # <R(m) q, R(n) k> = <R(m - n) q, k> on the rotary slice
    q = O.bf16_to_f64(_rand_bf16((1, 1, 256), 4))
    k = O.bf16_to_f64(_rand_bf16((1, 1, 256), 5))
    for m, n in [(5, 3), (1000, 17), (262144, 1), (1048575, 943718)]:
        lhs = np.dot(O.rope_rotate_f64(q, np.array([m]))[0, 0, :64], O.rope_rotate_f64(k, np.array([n]))[0, 0, :64])
        rhs = np.dot(O.rope_rotate_f64(q, np.array([m - n]))[0, 0, :64], k[0, 0, :64])
        assert abs(lhs - rhs) < 1e-8


def test_rope_preserves_pair_norms():
    x = O.bf16_to_f64(_rand_bf16((3, 24, 256), 6))
    y = O.rope_rotate_f64(x, np.array([7, 99999, 1048576]))
    nx = x[..., :32] ** 2 + x[..., 32:64] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:64] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-12)


def test_rope_rounding_is_single_step():
    x = _rand_bf16((16, 2, 256), 7)
    pos = np.arange(16) * 65537
    assert np.array_equal(O.rope_rotate(x, pos), O.f64_to_bf16(O.rope_rotate_f64(O.bf16_to_f64(x), pos)))



# ---------------------------------------------------------------- static YaRN

def test_yarn_table_for_the_model_card_config_by_hand():
    # model card "Processing Ultra-Long Texts": theta 1e7, factor 4, original 262144,
    # 64 rotary dims.  Pair i turns 262144 * 1e7^(-i/32) / (2 pi) times over the original
    # context; that count is 32 at i = 32 ln(262144 / 64 pi) / ln 1e7 = 14.24 and 1 at
    # i = 32 ln(262144 / 2 pi) / ln 1e7 = 21.12, so the ramp runs from pair 14 to pair 22.
    assert 14 < 32 * math.log(262144 / (64 * math.pi)) / math.log(1e7) < 14.5
    assert 21 < 32 * math.log(262144 / (2 * math.pi)) / math.log(1e7) < 21.5
    inv, m = O.yarn_inv_freq(O.Yarn(factor=4.0, original_max=262144))
    w = np.array([1e7 ** (-i / 32.0) for i in range(32)])
    assert np.allclose(inv[:15], w[:15], rtol=1e-14, atol=0)          # pairs 0..14 kept
    assert np.allclose(inv[22:], w[22:] / 4, rtol=1e-14, atol=0)      # pairs 22..31 divided by 4
    for i in range(15, 22):                                            # linear blend in i
        g = (i - 14) / 8.0
        assert math.isclose(inv[i], w[i] * (1 - g) + w[i] / 4 * g, rel_tol=1e-14)
    assert math.isclose(m, 1 + 0.1 * math.log(4.0), rel_tol=1e-15)


@pytest.mark.parametrize("theta,factor,orig", [(1e7, 4.0, 262144), (1e7, 2.0, 262144),
                                               (1e4, 8.0, 4096), (5e5, 3.0, 32768), (1e7, 1.5, 1 << 20)])
def test_yarn_matches_the_transformers_routine(theta, factor, orig):
    # an independent implementation of the frameworks' static YaRN (float32 there)
    tr = pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    cfg = tr.PretrainedConfig()
    cfg.hidden_size, cfg.num_attention_heads, cfg.head_dim = 24 * 256, 24, 256
    cfg.max_position_embeddings = int(orig * factor)
    cfg.rope_parameters = {"rope_type": "yarn", "rope_theta": theta, "partial_rotary_factor": 0.25,
                           "factor": factor, "original_max_position_embeddings": orig}
    ref_inv, ref_m = ROPE_INIT_FUNCTIONS["yarn"](cfg, torch.device("cpu"))
    inv, m = O.yarn_inv_freq(O.Yarn(factor=factor, original_max=orig), theta=theta)
    assert np.allclose(inv, ref_inv.double().numpy(), rtol=2e-6, atol=0)
    assert math.isclose(m, ref_m, rel_tol=1e-12)


def test_yarn_factor_one_is_plain_rotary():
    x = O.bf16_to_f64(_rand_bf16((3, 2, 256), 8))
    pos = np.array([1, 300000, 1048575])
    assert np.array_equal(O.rope_rotate_f64(x, pos, yarn=O.Yarn(factor=1.0)), O.rope_rotate_f64(x, pos))


def test_yarn_rotation_complex_form_and_norms():
    # each pair turned by e^{i p w'_i} and scaled by 1 + 0.1 ln 4; dims past 64 untouched
    yarn = O.Yarn()
    inv, _ = O.yarn_inv_freq(yarn)
    mf = 1 + 0.1 * math.log(4.0)
    x = O.bf16_to_f64(_rand_bf16((3, 2, 256), 9))
    pos = np.array([0, 262145, 1048575])
    y = O.rope_rotate_f64(x, pos, yarn=yarn)
    assert np.array_equal(y[..., 64:], x[..., 64:])
    for ti, p in enumerate(pos):
        for i in range(32):
            z = complex(x[ti, 0, i], x[ti, 0, 32 + i]) * cmath.exp(1j * p * inv[i]) * mf
            assert abs(y[ti, 0, i] - z.real) < 1e-9 and abs(y[ti, 0, 32 + i] - z.imag) < 1e-9
    nx = x[..., :32] ** 2 + x[..., 32:64] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:64] ** 2
    assert np.allclose(ny, nx * mf * mf, rtol=1e-12, atol=1e-12)


def test_yarn_relative_position():
    # <Y(m) q, Y(n) k> = <Y(m - n) q, Y(0) k>: the scaled rotation still depends on m - n only
    yarn = O.Yarn()
    q = O.bf16_to_f64(_rand_bf16((1, 1, 256), 10))
    k = O.bf16_to_f64(_rand_bf16((1, 1, 256), 11))
    for m, n in [(5, 3), (262144, 1), (1048575, 943718)]:
        lhs = np.dot(O.rope_rotate_f64(q, np.array([m]), yarn=yarn)[0, 0, :64],
                     O.rope_rotate_f64(k, np.array([n]), yarn=yarn)[0, 0, :64])
        rhs = np.dot(O.rope_rotate_f64(q, np.array([m - n]), yarn=yarn)[0, 0, :64],
                     O.rope_rotate_f64(k, np.array([0]), yarn=yarn)[0, 0, :64])
        assert abs(lhs - rhs) < 1e-8

# ---------------------------------------------------------------- compression

def test_compress_golden():
    for c in _gold("compress_cases.json")["cases"]:
        keys = np.array([_bf16_bits_of_hex(h) for h in c["keys"]], np.uint16)
        k = np.repeat(keys[:, None], 3, axis=1)          # [4 tokens, 3 dims]
        got = O.compress_block_keys(k, 0, 1)
        assert np.all(got == int(c["bits"], 16)), c


def test_compress_close_to_exact_mean():
    k = _rand_bf16((4096, 128), 8, sigma=1 / math.sqrt(128))
    got = O.bf16_to_f64(O.compress_block_keys(k, 0, 1024))
    exact = O.bf16_to_f64(k).reshape(1024, 4, 128).mean(axis=1)
    ref = O.bf16_to_f64(O.f64_to_bf16(exact))
    assert np.mean(got == ref) > 0.999
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= ulp)


def test_compress_block_range_and_complete_blocks_only():
    k = _rand_bf16((4 * 10 + 3, 128), 9)
    full = O.compress_block_keys(k, 0, 10)
    assert full.shape == (10, 128)
    assert np.array_equal(O.compress_block_keys(k, 3, 7), full[3:7])
    assert O.compress_block_keys(k, 5, 5).shape == (0, 128)


# ---------------------------------------------------------------- scores

def test_scores_bruteforce_tiny():
    q = _rand_bf16((3, 4, 128), 10, sigma=1 / math.sqrt(128))
    kb = _rand_bf16((9, 128), 11, sigma=1 / math.sqrt(128))
    got = O.index_scores(q, O.bf16_to_f64(kb))
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(kb)
    for r in range(3):
        for j in range(9):
            terms = [float(qf[r, h, d]) * float(kf[j, d]) for h in range(4) for d in range(128)]
            assert got[r, j] == np.float32(math.fsum(terms))


def test_scores_are_the_correctly_rounded_sum_on_many_entries():
    """2400 entries, rows of very different magnitudes: each score is the
    float32 rounding of the exact sum of its 512 products (math.fsum), the
    float64 product sum inside the oracle being far finer than that
    rounding."""
    q = _rand_bf16((40, 4, 128), 31)
    kb = _rand_bf16((60, 128), 32)
    q = O.f64_to_bf16(O.bf16_to_f64(q) * np.float64(2.0) ** np.arange(-20, 20)[:, None, None])  # exact scaling
    got = O.index_scores(q, O.bf16_to_f64(kb))
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(kb)
    for r in range(40):
        for j in range(60):
            terms = (qf[r, :, :] * kf[j][None, :]).ravel().tolist()
            assert got[r, j] == np.float32(math.fsum(terms)), (r, j)


def test_scores_basis_queries_pick_key_entries():
    kb = _rand_bf16((6, 128), 12)
    q = np.zeros((1, 4, 128), np.uint16)
    dims = [5, 17, 17, 127]
    for h, d in enumerate(dims):
        q[0, h, d] = 0x3F80                              # 1.0
    got = O.index_scores(q, O.bf16_to_f64(kb))[0]
    kf = O.bf16_to_f64(kb)
    for j in range(6):
        assert got[j] == np.float32(sum(kf[j, d] for d in dims))


def test_scores_invariant_to_head_order():
    q = _rand_bf16((2, 4, 128), 13)
    kb = O.bf16_to_f64(_rand_bf16((50, 128), 14))
    assert np.array_equal(O.index_scores(q, kb), O.index_scores(q[:, ::-1].copy(), kb))


# ---------------------------------------------------------------- selection

def _select_bruteforce(scores, t, budget):
    o = t // 4
    def key(j):
        s = float(scores[j])
        return (1 if math.isnan(s) else 0, -(0.0 if math.isnan(s) else s), j)
    chosen = sorted(range(o), key=key)[:min(budget - 1, o)] + [o]
    return sorted(chosen) + [-1] * (budget - len(chosen))


def test_select_golden():
    for c in _gold("select_cases.json")["cases"]:
        s = np.array([float(x) for x in c["scores"]], np.float32)
        assert O.select_blocks(s, c["t"], c["budget"]).tolist() == c["sel"], c


def test_select_bruteforce_random_rows():
    rng = np.random.default_rng(15)
    for trial in range(300):
        t = int(rng.integers(0, 200))
        budget = int(rng.integers(1, 70))
        o = t // 4
        if trial % 3 == 0:   # coarse values: many exact ties
            s = rng.integers(-3, 4, o).astype(np.float32) * np.float32(0.5)
        else:
            s = rng.standard_normal(o).astype(np.float32)
        assert O.select_blocks(s, t, budget).tolist() == _select_bruteforce(s, t, budget)


def test_select_budget_covering_everything_keeps_all():
    s = np.random.default_rng(16).standard_normal(100).astype(np.float32)
    got = O.select_blocks(s, 403, 512)
    assert got[:101].tolist() == list(range(101)) and np.all(got[101:] == -1)


# ---------------------------------------------------------------- attention

def _sdpa_dense_causal(q, k, v, scale):
    """Dense causal GQA by torch's SDPA in float64; q [T,Hq,D], k/v [T,Hkv,D]."""
    group = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(group, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).repeat_interleave(group, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_layer_equals_dense_causal_attention_when_budget_covers_everything():
    wl = I.custom_workload("prefill", batch=1, ctx=0, tq=61, budget=64, seed=21)
    x = I.make_inputs(wl)
    B = O.bits
    layer = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget)
    res = layer.rows([(0, t) for t in range(61)])
    pos = np.arange(61)
    q = O.bf16_to_f64(O.rope_rotate(B(x.q)[0], pos))
    k = O.bf16_to_f64(O.rope_rotate(B(x.k)[0], pos))
    v = O.bf16_to_f64(B(x.v)[0])
    ref = _sdpa_dense_causal(q, k, v, 1 / 16)
    got = np.stack([r.out for r in res])
    assert np.max(np.abs(got - ref)) < 1e-12


def test_lse_matches_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(22)
    q = rng.standard_normal((24, 256))
    k = rng.standard_normal((37, 2, 256))
    v = rng.standard_normal((37, 2, 256))
    _, lse = O.attend(q, k, v, 1 / 16)
    for h in range(24):
        assert abs(lse[h] - logsumexp(k[:, h // 12, :] @ q[h] / 16)) < 1e-12


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((24, 256)) * 3
    k = rng.standard_normal((100, 2, 256))
    out, _ = O.attend(q, k, np.ones((100, 2, 256)), 1 / 16)
    assert np.max(np.abs(out - 1.0)) < 1e-12


def test_attention_invariant_to_order_of_selected_blocks():
    wl = I.custom_workload("prefill", batch=1, ctx=0, tq=400, budget=16, seed=24)
    x = I.make_inputs(wl)
    B = O.bits
    layer = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget)
    rows = [(0, 397), (0, 250)]
    base = layer.rows(rows)
    rng = np.random.default_rng(0)
    perm = {r: rng.permutation(res.sel) for r, res in zip(rows, base)}
    again = layer.rows(rows, sel_override=perm)
    for a, b in zip(base, again):
        assert np.max(np.abs(a.out - b.out)) < 1e-12


def test_attention_bruteforce_with_explicit_mask_tiny():
    # tiny dims: Hq 4, Hkv 2, D 8; the attended set is given as a 0/1 mask row
    rng = np.random.default_rng(25)
    T, Hq, Hkv, D = 23, 4, 2, 8
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    t = 21
    sel = np.array([1, 3, 5, -1])             # own block of t=21 is 5
    mask = [0] * T
    for j in (1, 3):
        for n in range(4 * j, 4 * j + 4):
            mask[n] = 1
    for n in range(20, t + 1):
        mask[n] = 1
    tok = O.expand_tokens(sel, t)
    assert tok.tolist() == [n for n in range(T) if mask[n]]
    out, lse = O.attend(q, k[tok], v[tok], 0.5)
    for h in range(Hq):
        g = h // 2
        logit = [sum(q[h, d] * k[n, g, d] for d in range(D)) * 0.5 if mask[n] else None for n in range(T)]
        mx = max(x for x in logit if x is not None)
        w = [math.exp(x - mx) if x is not None else 0.0 for x in logit]
        z = sum(w)
        for d in range(D):
            ref = sum(w[n] * v[n, g, d] for n in range(T)) / z
            assert abs(out[h, d] - ref) < 1e-12
        assert abs(lse[h] - (mx + math.log(z))) < 1e-12


# ---------------------------------------------------------------- pipeline

def test_planted_needles_are_selected():
    wl = I.WORKLOADS["prefill_T2048_budget64"]
    x = I.make_inputs(wl)
    B = O.bits
    layer = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget)
    assert len(x.needles) == 8
    res = layer.rows([(int(b), int(t)) for b, t, _ in x.needles])
    for (b, t, j), r in zip(x.needles, res):
        assert j in r.sel
        assert r.scores[j] == r.scores.max() and r.scores[j] > 4.0


def test_generator_is_deterministic_and_thread_independent():
    wl = I.custom_workload("prefill", batch=2, ctx=8, tq=40, budget=8, n_needles=3, seed=5)
    a = I.make_inputs(wl, threads=1)
    b = I.make_inputs(wl, threads=4)
    for name in ("q", "q_idx", "k", "v", "k_idx"):
        assert torch.equal(getattr(a, name).view(torch.int16), getattr(b, name).view(torch.int16))
    assert np.array_equal(a.needles, b.needles)
    assert float(a.q.float().std()) == pytest.approx(1.0, rel=0.05)
    assert float(a.q_idx.float().std()) == pytest.approx(1 / math.sqrt(128), rel=0.05)


# ---------------------------------------------------------------- output gate

def _gate_bits(values):
    return O.f64_to_bf16(np.asarray(values, np.float64))


def test_output_gate_special_values():
    """sigmoid(0) = 1/2 halves the output exactly; large logits pass it
    (sigmoid(30) = 1 - 9.4e-14) or block it (sigmoid(-30) = 9.4e-14)."""
    out = np.array([[1.5, -2.25, 3.0e-3, 7.0]])
    assert np.array_equal(O.output_gate(out, _gate_bits(np.zeros((1, 4)))), out / 2)
    up = O.output_gate(out, _gate_bits(np.full((1, 4), 30.0)))
    down = O.output_gate(out, _gate_bits(np.full((1, 4), -30.0)))
    assert np.allclose(up, out, rtol=1e-12, atol=0) and np.all(np.abs(down) <= 1e-12 * np.abs(out))


def test_output_gate_is_the_logistic_function():
    """Against scipy's logistic function on random logits, and the symmetry
    sigmoid(g) + sigmoid(-g) = 1: gating with g and with -g sums to the
    ungated output."""
    from scipy.special import expit
    rng = np.random.default_rng(3)
    out = rng.standard_normal((24, 256))
    g_bits = _gate_bits(rng.standard_normal((24, 256)) * 4)
    g = O.bf16_to_f64(g_bits)
    assert np.allclose(O.output_gate(out, g_bits), out * expit(g), rtol=1e-14, atol=1e-300)
    both = O.output_gate(out, g_bits) + O.output_gate(out, O.f64_to_bf16(-g))
    assert np.allclose(both, out, rtol=1e-13, atol=1e-15)


def test_layer_gate_scales_outputs_and_leaves_lse():
    wl = I.custom_workload("prefill", batch=1, ctx=40, tq=6, budget=8, seed=5)
    x = I.make_inputs(wl)
    B = O.bits
    g = np.random.default_rng(4).standard_normal((1, 6, 24, 256))
    g_bits = _gate_bits(g)
    plain = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget)
    gated = O.OracleLayer(B(x.q), B(x.q_idx), B(x.k), B(x.v), B(x.k_idx), x.q_pos0, wl.budget, gate=g_bits)
    rows = [(0, 40 + i) for i in range(6)]
    for i, (a, c) in enumerate(zip(plain.rows(rows), gated.rows(rows))):
        s = 1.0 / (1.0 + np.exp(-O.bf16_to_f64(g_bits[0, i])))
        assert np.allclose(c.out, a.out * s, rtol=1e-14, atol=1e-300)
        assert np.array_equal(c.lse, a.lse) and np.array_equal(c.sel, a.sel)
