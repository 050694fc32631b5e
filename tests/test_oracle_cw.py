"""Pins of the oracle's channel-wise decay decode (Kimi Delta Attention).

The Kimi Linear section of "Seven Architectures Replacing KV Cache With
Bounded Mutable State" replaces Gated DeltaNet's scalar forget gate with one
decay per key channel and applies the delta correction to the decayed state.
Pinned here by: equal channels reduce to the (separately pinned) scalar
oracle; a one-hot key rewrites exactly its own row while every other row only
decays by its own rate; the delta-rule invariant on the decayed state (which
fails for the erase-then-decay order); the zero-decay limit; slot rules.
"""
import numpy as np
import pytest

import oracle

RULES = ["linear", "gated", "delta", "gated_delta"]


def case(seed, B=3, Hqk=2, Hv=4, dk=5, dv=3, n_slots=8):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hqk, dk))
    k = r.standard_normal((B, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, Hv, dv))
    g = -np.abs(r.standard_normal((B, Hv, dk)))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, Hv))))
    pool = r.standard_normal((n_slots, Hv, dk, dv))
    return q, k, v, g, beta, pool


@pytest.mark.parametrize("rule", RULES)
def test_equal_channels_reduce_to_scalar_decay(rule):
    q, k, v, g, beta, pool = case(1)
    gs = g[:, :, 0]
    g_eq = np.repeat(gs[:, :, None], g.shape[2], axis=2)
    rs, ws = np.array([0, 5, -1], np.int32), np.array([2, 6, 7], np.int32)
    o1, p1, c1 = oracle.decode(q, k, v, gs, beta, pool, rs, ws, rule=rule, scale=0.7)
    o2, p2, c2 = oracle.decode_cw(q, k, v, g_eq, beta, pool, rs, ws, rule=rule, scale=0.7)
    assert c1 == c2 == 0
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2, p1, rtol=1e-12, atol=1e-13)


def test_one_hot_key_rewrites_only_its_row():
    # k = e_i, beta = 1: row i of the new state is v; every other row m is alpha_m S_m
    q, k, v, g, beta, pool = case(2, B=1, Hqk=1, Hv=1, dk=6, dv=4, n_slots=1)
    i = 3
    k = np.zeros_like(k)
    k[0, 0, i] = 1.0
    beta = np.ones_like(beta)
    _, after, _ = oracle.decode_cw(q, k, v, g, beta, pool, rule="gated_delta")
    S0, S1 = pool[0, 0], after[0, 0]
    np.testing.assert_allclose(S1[i], v[0, 0], rtol=1e-14, atol=1e-14)
    for m in range(6):
        if m != i:
            np.testing.assert_allclose(S1[m], np.exp(g[0, 0, m]) * S0[m], rtol=1e-14)


def test_delta_invariant_on_the_decayed_state():
    # unit k, beta = 1: the new state maps k to v whatever the per-channel decay
    q, k, v, g, beta, pool = case(3, B=2, n_slots=2)
    beta = np.ones_like(beta)
    _, after, _ = oracle.decode_cw(q, k, v, g, beta, pool, rule="gated_delta")
    for b in range(2):
        for h in range(4):
            kk = k[b, h * 2 // 4]
            np.testing.assert_allclose(after[b, h].T @ kk, v[b, h], rtol=1e-12, atol=1e-12)
    # the erase-then-decay order does not keep it: the channels decay differently
    S, kk, a = pool[0, 0], k[0, 0], np.exp(g[0, 0])
    other = np.diag(a) @ (np.eye(len(kk)) - np.outer(kk, kk)) @ S + np.outer(kk, v[0, 0])
    assert np.max(np.abs(other.T @ kk - v[0, 0])) > 1e-3


def test_zero_decay_keeps_only_the_new_write():
    q, k, v, g, beta, pool = case(4, B=2, n_slots=2)
    g = np.full_like(g, -800.0)   # exp underflows to 0 in every channel
    o, after, _ = oracle.decode_cw(q, k, v, g, beta, pool, rule="gated_delta", scale=1.0)
    for b in range(2):
        for h in range(4):
            kk, qq = k[b, h // 2], q[b, h // 2]
            np.testing.assert_allclose(after[b, h], beta[b, h] * np.outer(kk, v[b, h]), atol=1e-14)
            np.testing.assert_allclose(o[b, h], beta[b, h] * (kk @ qq) * v[b, h], atol=1e-14)


def test_slots_and_rounding():
    q, k, v, g, beta, pool = case(5)
    rs, ws = np.array([0, 9, 1], np.int32), np.array([3, 4, 5], np.int32)
    o, after, code = oracle.decode_cw(q, k, v, g, beta, pool, rs, ws, round_state=True)
    assert code == 1                      # request 1 read past the pool: skipped
    assert not o[1].any()
    np.testing.assert_array_equal(after[4], pool[4])
    np.testing.assert_array_equal(after[3], oracle.round_bf16(after[3]))
    _, exact, _ = oracle.decode_cw(q, k, v, g, beta, pool, rs, ws, round_state=False)
    np.testing.assert_array_equal(after[3], oracle.round_bf16(exact[3]))
