"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutant replaces one oracle function (on the CPU, inside this test only)
with a subtly wrong variant -- a dropped term, a wrong sign, index or
operand -- and runs the pins that should notice.  A mutant that no pin
rejects would mean the oracle is not pinned where it matters.
"""

import numpy as np
import pytest

from oracle import qsa_oracle as O
from tests import test_oracle_pins as P


def _compress_sum_not_mean(k_idx_bits, b0, b1):
    n = b1 - b0
    k = O.bf16_to_f64(k_idx_bits[4 * b0: 4 * b1]).astype(np.float32).reshape(n, 4, -1)
    return O.f64_to_bf16((((k[:, 0] + k[:, 1]) + k[:, 2]) + k[:, 3]).astype(np.float64))


def _compress_three_keys(k_idx_bits, b0, b1):
    n = b1 - b0
    k = O.bf16_to_f64(k_idx_bits[4 * b0: 4 * b1]).astype(np.float32).reshape(n, 4, -1)
    return O.f64_to_bf16(((k[:, 0] + k[:, 1] + k[:, 2]) * np.float32(0.25)).astype(np.float64))


def _compress_exact_mean(k_idx_bits, b0, b1):
    n = b1 - b0
    k = O.bf16_to_f64(k_idx_bits[4 * b0: 4 * b1]).reshape(n, 4, -1)
    return O.f64_to_bf16(k.mean(axis=1))


def _rope_factory(sign=1.0, interleaved=False, theta=O.ROPE_THETA, rot=64):
    def f(x, positions, rot_dim=64, th=O.ROPE_THETA, yarn=None):
        half = rot // 2
        ang = np.asarray(positions, np.float64)[:, None] * (theta ** (-2.0 * np.arange(half) / rot))[None]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :] * sign
        out = np.array(x, dtype=np.float64, copy=True)
        if interleaved:
            a, b = x[..., 0:rot:2], x[..., 1:rot:2]
            out[..., 0:rot:2] = a * c - b * s
            out[..., 1:rot:2] = b * c + a * s
        else:
            a, b = x[..., :half], x[..., half:rot]
            out[..., :half] = a * c - b * s
            out[..., half:rot] = b * c + a * s
        return out
    return f


def _yarn_factory(reverse=False, no_mscale=False, round_ends=False, times_s=False):
    def f(yarn, rot_dim=64, theta=O.ROPE_THETA):
        w = O.rope_inv_freq(rot_dim, theta)
        s, L = yarn.factor, yarn.original_max
        at = lambda rho: (rot_dim / 2) * np.log(L / (2 * np.pi * rho)) / np.log(theta)
        lo = np.round(at(32.0)) if round_ends else np.floor(at(32.0))
        hi = np.round(at(1.0)) if round_ends else np.ceil(at(1.0))
        ramp = np.clip((np.arange(rot_dim // 2) - lo) / (hi - lo), 0, 1)
        if reverse:
            ramp = 1 - ramp
        interp = w * s if times_s else w / s
        return interp * ramp + w * (1 - ramp), (1.0 if no_mscale else 0.1 * np.log(s) + 1)
    return f


def _select_factory(tie_high=False, own_outside_budget=False, keep_neg_zero=False):
    def f(scores_row, t, budget):
        o = t // 4
        keep = min(budget if own_outside_budget else budget - 1, o)
        s = np.asarray(scores_row[:o], np.float64)
        isnan = np.isnan(s)
        s = np.where(isnan, 0.0, s)
        if not keep_neg_zero:
            s = s + 0.0
        idx = np.arange(o)
        if tie_high:
            idx = -idx
        if keep_neg_zero:
            # distinguish -0.0 from +0.0 by the sign bit
            sb = np.signbit(s) & (s == 0)
            order = np.lexsort((idx, sb, -s, isnan))
        else:
            order = np.lexsort((idx, -s, isnan))
        chosen = np.sort(np.append(order[:keep], o)).astype(np.int32)
        out = np.full(max(budget, chosen.size), -1, np.int32)
        out[:chosen.size] = chosen
        return out[:budget] if chosen.size <= budget else out
    return f


def _attend_factory(mod_groups=False, no_scale=False):
    def f(q, k, v, scale):
        hq, hkv = q.shape[0], k.shape[1]
        out = np.zeros((hq, q.shape[1]))
        lse = np.zeros(hq)
        for h in range(hq):
            g = (h % hkv) if mod_groups else h // (hq // hkv)
            logits = (k[:, g, :] @ q[h]) * (1.0 if no_scale else scale)
            m = logits.max()
            p = np.exp(logits - m)
            out[h] = (p @ v[:, g, :]) / p.sum()
            lse[h] = m + np.log(p.sum())
        return out, lse
    return f


def _expand_no_causal_cut(sel, t):
    blocks = np.asarray(sel)[np.asarray(sel) >= 0].astype(np.int64)
    return (4 * blocks[:, None] + np.arange(4)[None, :]).reshape(-1)


MUTANTS = [
    ("compress: sum instead of mean", "compress_block_keys", _compress_sum_not_mean,
     [P.test_compress_golden]),
    ("compress: drops the 4th key", "compress_block_keys", _compress_three_keys,
     [P.test_compress_golden]),
    ("compress: exact mean instead of the float32 token-order sum", "compress_block_keys",
     _compress_exact_mean, [P.test_compress_golden]),
    ("rope: wrong rotation direction", "rope_rotate_f64", _rope_factory(sign=-1.0),
     [P.test_rope_complex_form]),
    ("rope: interleaved pairs (2i, 2i+1)", "rope_rotate_f64", _rope_factory(interleaved=True),
     [P.test_rope_complex_form]),
    ("rope: theta 1e4", "rope_rotate_f64", _rope_factory(theta=1e4), [P.test_rope_complex_form]),
    ("rope: 128 rotary dims", "rope_rotate_f64", _rope_factory(rot=128),
     [P.test_rope_leaves_dims_past_the_slice, P.test_rope_complex_form]),
    ("yarn: ramp reversed (high frequencies interpolated)", "yarn_inv_freq", _yarn_factory(reverse=True),
     [P.test_yarn_table_for_the_model_card_config_by_hand]),
    ("yarn: no factor on cos and sin", "yarn_inv_freq", _yarn_factory(no_mscale=True),
     [P.test_yarn_table_for_the_model_card_config_by_hand, P.test_yarn_rotation_complex_form_and_norms]),
    ("yarn: ramp ends rounded to nearest", "yarn_inv_freq", _yarn_factory(round_ends=True),
     [P.test_yarn_table_for_the_model_card_config_by_hand]),
    ("yarn: frequencies multiplied by s", "yarn_inv_freq", _yarn_factory(times_s=True),
     [P.test_yarn_table_for_the_model_card_config_by_hand]),
    ("select: ties to the higher index", "select_blocks", _select_factory(tie_high=True),
     [P.test_select_golden]),
    ("select: own block outside the budget", "select_blocks", _select_factory(own_outside_budget=True),
     [P.test_select_golden]),
    ("select: -0.0 ranked below +0.0", "select_blocks", _select_factory(keep_neg_zero=True),
     [P.test_select_golden]),
    ("attention: KV head h % 2 instead of h // 12", "attend", _attend_factory(mod_groups=True),
     [P.test_layer_equals_dense_causal_attention_when_budget_covers_everything]),
    ("attention: softmax scale dropped", "attend", _attend_factory(no_scale=True),
     [P.test_layer_equals_dense_causal_attention_when_budget_covers_everything]),
    ("attention: own block not cut at the query", "expand_tokens", _expand_no_causal_cut,
     [P.test_layer_equals_dense_causal_attention_when_budget_covers_everything]),
    ("gate: sigmoid of the wrong sign", "output_gate",
     lambda out, g: out / (1.0 + np.exp(O.bf16_to_f64(g))),
     [P.test_output_gate_special_values, P.test_output_gate_is_the_logistic_function]),
    ("gate: tanh instead of the logistic function", "output_gate",
     lambda out, g: out * np.tanh(O.bf16_to_f64(g)),
     [P.test_output_gate_special_values, P.test_output_gate_is_the_logistic_function]),
    ("gate: multiplies by the logit", "output_gate",
     lambda out, g: out * O.bf16_to_f64(g),
     [P.test_output_gate_special_values, P.test_output_gate_is_the_logistic_function]),
]


@pytest.mark.parametrize("name,attr,impl,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, attr, impl, pins):
    monkeypatch.setattr(O, attr, impl)
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"no pin rejects the mutant: {name}"


def test_scores_dropping_a_head_is_caught(monkeypatch):
    orig = O.index_scores

    def three_heads(q_idx_bits, kbar_f64):
        return orig(q_idx_bits[:, :3], kbar_f64)

    monkeypatch.setattr(O, "index_scores", three_heads)
    with pytest.raises(AssertionError):
        P.test_scores_bruteforce_tiny()


def test_scores_transposed_operand_is_caught(monkeypatch):
    def per_dim_sum(q_idx_bits, kbar_f64):
        q = O.bf16_to_f64(q_idx_bits)
        # sums the key over dims and the query over heads separately: wrong contraction
        return (q.sum(axis=(1, 2))[:, None] * kbar_f64.sum(axis=1)[None, :]).astype(np.float32)

    monkeypatch.setattr(O, "index_scores", per_dim_sum)
    with pytest.raises(AssertionError):
        P.test_scores_bruteforce_tiny()
