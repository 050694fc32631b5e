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


# --------------------------------------------------------------------------
# sequences (the prefill recurrence) with a channel-wise decay

from fractions import Fraction  # noqa: E402

from chunk_model import chunked_sequence_cw  # noqa: E402


def seq_case(seed, lengths, Hqk=1, Hv=2, dk=6, dv=4, n_slots=6, g_scale=1.0):
    r = np.random.default_rng(seed)
    N = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = r.standard_normal((N, Hqk, dk))
    k = r.standard_normal((N, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((N, Hv, dv))
    g = -np.abs(r.standard_normal((N, Hv, dk))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((N, Hv))))
    pool = r.standard_normal((n_slots, Hv, dk, dv)) * 0.3
    return cu, q, k, v, g, beta, pool


@pytest.mark.parametrize("rule", RULES)
def test_sequences_equal_channels_are_the_scalar_sequences(rule):
    cu, q, k, v, g, beta, pool = seq_case(11, [5, 0, 9])
    gs = g[:, :, 0]
    geq = np.repeat(gs[:, :, None], g.shape[2], axis=2)
    rs, ws = np.array([1, -1, 2], np.int32), np.array([3, 4, 5], np.int32)
    o1, p1, _ = oracle.sequences(cu, q, k, v, gs, beta, pool, rs, ws, rule=rule, scale=0.6)
    o2, p2, _ = oracle.sequences_cw(cu, q, k, v, geq, beta, pool, rs, ws, rule=rule, scale=0.6)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2, p1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("rule", RULES)
def test_sequences_equal_decode_steps(rule):
    """T decode tokens on one slot = one sequence of T tokens."""
    cu, q, k, v, g, beta, pool = seq_case(12, [7])
    p = pool.copy()
    outs = []
    for t in range(7):
        o, p, _ = oracle.decode_cw(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                   beta[t:t + 1], p, [0], [0], rule=rule)
        outs.append(o)
    os_, ps, _ = oracle.sequences_cw(cu, q, k, v, g, beta, pool, [0], [0], rule=rule)
    np.testing.assert_allclose(np.concatenate(outs), os_, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p[0], ps[0], rtol=1e-12, atol=1e-13)


def test_sequences_delta_invariant_every_token():
    """With beta = 1 and unit keys the new state reads back v_t at k_t after
    every token: M_t^T k_t = v_t (the write reads the decayed state)."""
    T = 6
    _, q, k, v, g, beta, pool = seq_case(13, [T])
    beta[:] = 1.0
    p = pool.copy()
    for t in range(T):
        _, p, _ = oracle.sequences_cw(np.array([0, 1], np.int32), q[t:t + 1], k[t:t + 1],
                                      v[t:t + 1], g[t:t + 1], beta[t:t + 1], p, [0], [0])
        for h in range(2):
            np.testing.assert_allclose(p[0, h].T @ k[t, 0], v[t, h], rtol=1e-12, atol=1e-12)


def test_sequences_exact_rational_with_on_off_channels():
    """Channels that keep everything (g = 0) or forget everything (g = -inf)
    make every weight 0 or 1, so with dyadic inputs the recurrence is exact
    rational arithmetic: the oracle must equal a Fraction computation."""
    T, dk, dv = 4, 3, 2
    r = np.random.default_rng(14)
    q = r.integers(-4, 5, (T, 1, dk)) / 4.0
    k = r.integers(-4, 5, (T, 1, dk)) / 4.0
    v = r.integers(-4, 5, (T, 1, dv)) / 4.0
    beta = np.full((T, 1), 0.5)
    g = np.zeros((T, 1, dk))
    g[1, 0, 0] = -np.inf
    g[2, 0, 2] = -np.inf
    g[3, 0, 1] = -np.inf
    cu = np.array([0, T], np.int32)
    o, p, _ = oracle.sequences_cw(cu, q, k, v, g, beta, np.zeros((1, 1, dk, dv)), [-1], [0])
    S = [[Fraction(0)] * dv for _ in range(dk)]
    for t in range(T):
        a = [Fraction(0) if np.isneginf(g[t, 0, i]) else Fraction(1) for i in range(dk)]
        S = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
        kk = [Fraction(x) for x in k[t, 0]]
        read = [sum(S[i][j] * kk[i] for i in range(dk)) for j in range(dv)]
        d = [Fraction(beta[t, 0]) * (Fraction(v[t, 0, j]) - read[j]) for j in range(dv)]
        S = [[S[i][j] + kk[i] * d[j] for j in range(dv)] for i in range(dk)]
        want = [sum(S[i][j] * Fraction(q[t, 0, i]) for i in range(dk)) for j in range(dv)]
        assert [Fraction(x) for x in o[t, 0]] == want, t
    assert [[Fraction(x) for x in row] for row in p[0, 0]] == S


def test_sequences_split_through_checkpoint():
    cu, q, k, v, g, beta, pool = seq_case(15, [11])
    o, p, _ = oracle.sequences_cw(cu, q, k, v, g, beta, pool, [0], [1])
    T1 = 4
    o1, p1, _ = oracle.sequences_cw(np.array([0, T1], np.int32), q[:T1], k[:T1], v[:T1], g[:T1],
                                    beta[:T1], pool, [0], [2])
    o2, p2, _ = oracle.sequences_cw(np.array([0, 11 - T1], np.int32), q[T1:], k[T1:], v[T1:],
                                    g[T1:], beta[T1:], p1, [2], [1])
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2[1], p[1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("C,sub", [(16, 16), (64, 16), (64, 64), (8, 4)])
def test_chunked_cw_model_matches_token_recurrence(rule, C, sub):
    """The chunk algebra the GPU chain uses (per-channel scalings, the
    end-of-column-tile reference below the diagonal, direct weights on it)
    equals the token recurrence, including ragged tails and gates so strong
    (g down to -60 per token) that any single chunk-wide reference would
    overflow."""
    lengths = [70, 33]
    cu, q, k, v, g, beta, pool = seq_case(16, lengths, Hv=1, dk=8, dv=5)
    g[5:9, 0, 2] = -60.0
    g[40:43, 0, 6] = -25.0
    o, p, _ = oracle.sequences_cw(cu, q, k, v, g, beta, pool, [0, 1], [2, 3], rule=rule, scale=0.9)
    for s_, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        om, Mm = chunked_sequence_cw(pool[s_, 0], q[a:b, 0], k[a:b, 0], v[a:b, 0], g[a:b, 0],
                                     beta[a:b, 0], rule, C, scale=0.9, sub=sub)
        np.testing.assert_allclose(om, o[a:b, 0], rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(Mm, p[2 + s_, 0], rtol=1e-9, atol=1e-11)
