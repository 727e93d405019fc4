"""Pins of the Gated DeltaNet oracle against facts other than itself.

Hand-derived single writes, the pure-decay closed form, the delta rule's
exact overwrite of associations, the chunk-parallel (UT-transform) form of
the same recurrence solved with a library linear solve, normalisation and
head-grouping invariants, and state carry across calls; then planted
mistakes that these pins must reject.
"""

import math

import numpy as np
import pytest

from oracle import gdn_oracle as G


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(n, i):
    e = np.zeros(n)
    e[i] = 1.0
    return e


# ---------------------------------------------------------------- closed forms

def test_single_write_from_zero_by_hand():
    # k = 2 e0 (normalised: e0), q = 5 e0 (normalised and scaled: e0 / sqrt(128)),
    # beta 0.5, g -0.3 (the decay meets an empty state): S1 = 0.5 e0 v^T and
    # o1 = S1^T q = 0.5 v / sqrt(128)
    v = _rng(1).standard_normal(128)
    q, k = G.prepare_qk((5 * _unit(128, 0))[None], (2 * _unit(128, 0))[None])
    o, s = G.gated_delta_rule(q, k, v[None], np.array([-0.3]), np.array([0.5]), np.zeros((128, 128)))
    s_hand = np.zeros((128, 128))
    s_hand[0] = 0.5 * v
    assert np.allclose(s, s_hand, atol=1e-15)
    assert np.allclose(o[0], 0.5 * v / math.sqrt(128), atol=1e-15)


def test_no_write_is_pure_decay():
    # beta = 0: S_t = exp(g_1 + ... + g_t) S_0 and o_t = S_t^T q_t
    r = _rng(2)
    T = 9
    q, k = G.prepare_qk(r.standard_normal((T, 128)), r.standard_normal((T, 128)))
    s0 = r.standard_normal((128, 128))
    g = -r.uniform(0, 0.5, T)
    o, s = G.gated_delta_rule(q, k, r.standard_normal((T, 128)), g, np.zeros(T), s0)
    cg = np.cumsum(g)
    for t in range(T):
        assert np.allclose(o[t], math.exp(cg[t]) * (s0.T @ q[t]), rtol=1e-12, atol=1e-12)
    assert np.allclose(s, math.exp(cg[-1]) * s0, rtol=1e-12, atol=1e-12)


def test_delta_rule_overwrites_associations():
    # no decay, beta = 1, orthonormal keys: writing (ka, v1), (kb, v2), (ka, v3)
    # leaves S = ka v3^T + kb v2^T exactly, so reading ka gives v3
    r = _rng(3)
    v = r.standard_normal((3, 128))
    ka, kb = _unit(128, 7), _unit(128, 40)
    q, k = G.prepare_qk(np.stack([ka, kb, ka]), np.stack([ka, kb, ka]))
    o, s = G.gated_delta_rule(q, k, v, np.zeros(3), np.ones(3), np.zeros((128, 128)))
    assert np.allclose(s, np.outer(ka, v[2]) + np.outer(kb, v[1]), atol=1e-14)
    assert np.allclose(o[2], v[2] / math.sqrt(128), atol=1e-14)


def test_full_strength_write_is_read_back_exactly():
    # alpha = 1, beta = 1: (I - k k^T) S + k v^T maps the unit key k to v whatever S held
    r = _rng(4)
    T = 12
    q, k = G.prepare_qk(r.standard_normal((T, 128)), r.standard_normal((T, 128)))
    q[-1] = k[-1] / math.sqrt(128)
    g = -r.uniform(0, 0.2, T)
    g[-1] = 0.0
    beta = r.uniform(0, 1, T)
    beta[-1] = 1.0
    v = r.standard_normal((T, 128))
    o, s = G.gated_delta_rule(q, k, v, g, beta, r.standard_normal((128, 128)))
    assert np.allclose(s.T @ k[-1], v[-1], atol=1e-12)
    assert np.allclose(o[-1], v[-1] / math.sqrt(128), atol=1e-12)


# ---------------------------------------------------------------- chunk-parallel form

def _chunked(q, k, v, g, beta, s0, C):
    """The same recurrence over chunks of C tokens (UT transform): within a
    chunk with cumulative log decay c_i, the written rows w solve
    (I + A) w = beta v - beta exp(c) (k S_0), A_ij = beta_i exp(c_i - c_j) k_i.k_j (j < i);
    then o = exp(c) (q S_0) + (M * q k^T) w with M_ij = exp(c_i - c_j) (j <= i), and
    S = exp(c_C) S_0 + k^T (exp(c_C - c) w)."""
    s = np.array(s0, copy=True)
    out = np.zeros((q.shape[0], v.shape[1]))
    for c0 in range(0, q.shape[0], C):
        sl = slice(c0, min(q.shape[0], c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        c = np.cumsum(g[sl])
        n = len(c)
        diff = c[:, None] - c[None, :]
        A = np.tril(b[:, None] * np.exp(np.where(np.tril(np.ones((n, n)), -1) > 0, diff, 0.0)) * (K @ K.T), -1)
        rhs = b[:, None] * V - (b * np.exp(c))[:, None] * (K @ s)
        w = np.linalg.solve(np.eye(n) + A, rhs)
        M = np.tril(np.exp(np.where(np.tril(np.ones((n, n))) > 0, diff, 0.0)))
        out[sl] = np.exp(c)[:, None] * (Q @ s) + (M * (Q @ K.T)) @ w
        s = math.exp(c[-1]) * s + K.T @ (np.exp(c[-1] - c)[:, None] * w)
    return out, s


@pytest.mark.parametrize("T,C", [(50, 16), (64, 64), (7, 64), (130, 32)])
def test_chunked_form_equals_the_recurrence(T, C):
    r = _rng(T + C)
    q, k = G.prepare_qk(r.standard_normal((T, 128)), r.standard_normal((T, 128)))
    v = r.standard_normal((T, 128))
    g = -r.uniform(0, 1.0, T)
    beta = r.uniform(0, 1, T)
    s0 = r.standard_normal((128, 128)) * 0.3
    o1, s1 = G.gated_delta_rule(q, k, v, g, beta, s0)
    o2, s2 = _chunked(q, k, v, g, beta, s0, C)
    assert np.allclose(o1, o2, rtol=1e-9, atol=1e-10)
    assert np.allclose(s1, s2, rtol=1e-9, atol=1e-10)


# ---------------------------------------------------------------- layer invariants

def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32).__rshift__(16).astype(np.uint16)


def _layer_inputs(T, seed):
    r = _rng(seed)
    q = _bits(r.standard_normal((1, T, 16, 128)))
    k = _bits(r.standard_normal((1, T, 16, 128)))
    v = _bits(r.standard_normal((1, T, 48, 128)))
    g = -r.uniform(0, 0.5, (1, T, 48)).astype(np.float32)
    beta = r.uniform(0, 1, (1, T, 48)).astype(np.float32)
    s0 = (r.standard_normal((1, 48, 128, 128)) * 0.1).astype(np.float32)
    return q, k, v, g, beta, s0


def test_value_heads_share_query_key_heads_in_groups_of_three():
    q, k, v, g, beta, s0 = _layer_inputs(6, 5)
    for h in (1, 2, 3):                      # heads 0..3 with identical values, gates and state
        v[:, :, h], g[:, :, h], beta[:, :, h], s0[:, h] = v[:, :, 0], g[:, :, 0], beta[:, :, 0], s0[:, 0]
    o, s = G.gdn_layer(q, k, v, g, beta, s0)
    assert np.array_equal(o[:, :, 1], o[:, :, 0]) and np.array_equal(o[:, :, 2], o[:, :, 0])
    assert not np.allclose(o[:, :, 3], o[:, :, 0])          # head 3 reads Q/K head 1


def test_query_and_key_scale_does_not_matter():
    q, k, v, g, beta, s0 = _layer_inputs(5, 6)
    o1, s1 = G.gdn_layer(q, k, v, g, beta, s0)
    q2 = _bits(G.bf16_to_f64(q) * 4.0)            # exact in bf16
    k2 = _bits(G.bf16_to_f64(k) * 0.25)
    o2, s2 = G.gdn_layer(q2, k2, v, g, beta, s0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_state_carries_across_calls():
    q, k, v, g, beta, s0 = _layer_inputs(10, 7)
    o, s = G.gdn_layer(q, k, v, g, beta, s0)
    oa, sa = G.gdn_layer(q[:, :4], k[:, :4], v[:, :4], g[:, :4], beta[:, :4], s0)
    ob, sb = G.gdn_layer(q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], sa)
    assert np.allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-12)
    assert np.allclose(sb, s, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _rule(decay_erase=True, sign=-1.0, read_before=False, transposed=False):
    def f(q, k, v, g, beta, s0):
        s = np.array(s0, copy=True)
        out = np.zeros((q.shape[0], v.shape[1]))
        for t in range(q.shape[0]):
            a = np.exp(g[t])
            if read_before:
                out[t] = s.T @ q[t]
            erase = sign * beta[t] * np.outer(k[t], k[t] @ s)
            s = (a * (s + erase) if decay_erase else a * s + erase) + beta[t] * np.outer(k[t], v[t])
            if not read_before:
                out[t] = (s @ q[t]) if transposed else (s.T @ q[t])
        return out, s
    return f


RULE_PINS = [test_single_write_from_zero_by_hand, test_no_write_is_pure_decay,
             test_delta_rule_overwrites_associations, test_full_strength_write_is_read_back_exactly,
             lambda: test_chunked_form_equals_the_recurrence(50, 16)]

MUTANTS = [
    ("erase term not decayed", "gated_delta_rule", _rule(decay_erase=False), RULE_PINS),
    ("erase with the wrong sign", "gated_delta_rule", _rule(sign=1.0), RULE_PINS),
    ("output read before the write", "gated_delta_rule", _rule(read_before=True), RULE_PINS),
    ("output S q instead of S^T q", "gated_delta_rule", _rule(transposed=True), RULE_PINS),
    ("q not scaled", "prepare_qk",
     lambda q, k, normalize=True: (G.l2_normalize(q), G.l2_normalize(k)),
     [test_single_write_from_zero_by_hand]),
    ("q, k not normalised", "prepare_qk",
     lambda q, k, normalize=True: (q / math.sqrt(q.shape[-1]), k),
     [test_single_write_from_zero_by_hand, test_query_and_key_scale_does_not_matter]),
]


@pytest.mark.parametrize("name,attr,impl,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, attr, impl, pins):
    monkeypatch.setattr(G, attr, impl)
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):
            caught = True
    assert caught, f"no pin rejects the mutant: {name}"


def test_head_grouping_mutant_is_caught(monkeypatch):
    orig = G.gdn_layer

    def modulo_heads(q_bits, k_bits, v_bits, g, beta, s0, normalize=True):
        # V head h reading Q/K head h % 16 instead of h // 3
        qq = np.stack([q_bits[:, :, h % 16] for h in range(48)], axis=2)
        kk = np.stack([k_bits[:, :, h % 16] for h in range(48)], axis=2)
        return orig(qq, kk, v_bits, g, beta, s0, normalize)

    monkeypatch.setattr(G, "gdn_layer", modulo_heads)
    with pytest.raises(AssertionError):
        test_value_heads_share_query_key_heads_in_groups_of_three()
