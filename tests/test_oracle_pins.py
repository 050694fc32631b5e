"""Pins of the FP64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: exact
rational arithmetic, explicit transition matrices, invariants of the delta
rule, textbook closed forms, and library rounding.  Page citations name the
page title and section.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

RULES = ["linear", "gated", "delta", "gated_delta"]
ERASE = {"linear": False, "gated": False, "delta": True, "gated_delta": True}
DECAY = {"linear": False, "gated": True, "delta": False, "gated_delta": True}


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_problem(seed, T, Hqk, Hv, dk, dv, state_std=0.3):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((T, Hqk, dk)))
    k = unit(r.standard_normal((T, Hqk, dk)))
    v = r.standard_normal((T, Hv, dv))
    g = -np.log1p(np.exp(r.standard_normal((T, Hv))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, Hv))))
    M0 = r.standard_normal((1, Hv, dk, dv)) * state_std
    return q, k, v, g, beta, M0


def run_tokens(q, k, v, g, beta, M0, rule, scale=1.0):
    """Run T tokens of one sequence through the oracle's prefill recurrence."""
    T = q.shape[0]
    cu = np.array([0, T], np.int32)
    o, pool, code = oracle.sequences(cu, q, k, v, g, beta, M0, [0], [0], rule=rule, scale=scale)
    assert code == 0
    return o, pool[0]


# --------------------------------------------------------------------------
# exact rational brute force with explicit transition matrices
# ("Seven Architectures ...", section Gated DeltaNet-2: S_t = Diag(alpha)(I - b k k^T) S_{t-1}
#  + w k v^T, reduced to Gated DeltaNet by tying alpha, b, w to scalars)

def _fr_matmul(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


@pytest.mark.parametrize("rule", RULES)
def test_exact_rational_transition_matrices(rule):
    dk, dv, T = 3, 2, 4
    F = Fraction
    ks = [[F(1), F(0), F(0)], [F(3, 5), F(4, 5), F(0)], [F(0), F(0), F(1)], [F(2, 3), F(1, 3), F(2, 3)]]
    qs = [[F(0), F(1), F(0)], [F(1), F(0), F(0)], [F(2, 3), F(2, 3), F(1, 3)], [F(0), F(3, 5), F(4, 5)]]
    vs = [[F(1), F(-2)], [F(1, 2), F(3)], [F(-1), F(1, 4)], [F(5, 4), F(-3, 8)]]
    a = [F(1, 2), F(3, 4), F(7, 8), F(1, 4)]
    b = [F(1, 2), F(1, 4), F(3, 4), F(1)]
    M = [[F(1, 8), F(-1, 4)], [F(0), F(1, 2)], [F(3, 8), F(1, 16)]]
    M0 = [row[:] for row in M]
    outs = []
    for t in range(T):
        at = a[t] if DECAY[rule] else F(1)
        bt = b[t] if ERASE[rule] else F(0)
        wt = b[t] if ERASE[rule] else F(1)
        At = [[at * ((1 if i == j else 0) - bt * ks[t][i] * ks[t][j]) for j in range(dk)]
              for i in range(dk)]
        M = _fr_matmul(At, M)
        M = [[M[i][j] + wt * ks[t][i] * vs[t][j] for j in range(dv)] for i in range(dk)]
        outs.append([sum(M[i][j] * qs[t][i] for i in range(dk)) for j in range(dv)])
    fl = lambda x: np.array([[float(e) for e in row] for row in x])
    q = fl(qs)[:, None, :]
    k = fl(ks)[:, None, :]
    v = fl(vs)[:, None, :]
    g = np.log(np.array([float(x) for x in a]))[:, None]
    beta = np.array([float(x) for x in b])[:, None]
    o, Mt = run_tokens(q, k, v, g, beta, fl(M0)[None, None], rule)
    np.testing.assert_allclose(o[:, 0, :], fl(outs), rtol=0, atol=1e-14)
    np.testing.assert_allclose(Mt[0], fl(M), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# fully unrolled sum: M_T = (prod A) M0 + sum_s (prod_{r>s} A_r) w_s k_s v_s^T

@pytest.mark.parametrize("rule", RULES)
def test_unrolled_sum(rule):
    T, dk, dv = 10, 8, 6
    q, k, v, g, beta, M0 = rand_problem(1, T, 1, 1, dk, dv)
    a = np.exp(g[:, 0]) if DECAY[rule] else np.ones(T)
    bt = beta[:, 0] if ERASE[rule] else np.zeros(T)
    wt = beta[:, 0] if ERASE[rule] else np.ones(T)
    A = [a[t] * (np.eye(dk) - bt[t] * np.outer(k[t, 0], k[t, 0])) for t in range(T)]
    P = np.eye(dk)
    for t in range(T):
        P = A[t] @ P
    MT = P @ M0[0, 0]
    for s in range(T):
        Ps = np.eye(dk)
        for r in range(s + 1, T):
            Ps = A[r] @ Ps
        MT = MT + Ps @ (wt[s] * np.outer(k[s, 0], v[s, 0]))
    _, Mt = run_tokens(q, k, v, g, beta, M0, rule)
    np.testing.assert_allclose(Mt[0], MT, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants of the delta rule

@pytest.mark.parametrize("rule", ["delta", "gated_delta"])
def test_delta_rule_writes_exactly(rule):
    """With a = beta = 1 and unit k, the new state maps k_t to v_t: M_t^T k_t = v_t."""
    T, dk, dv = 12, 16, 8
    q, k, v, g, beta, M0 = rand_problem(2, T, 1, 1, dk, dv)
    g[:] = 0.0
    beta[:] = 1.0
    # read out with q_t = k_t, so o_t = M_t^T k_t
    o, _ = run_tokens(k.copy(), k, v, g, beta, M0, rule)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


@pytest.mark.parametrize("rule", RULES)
def test_erase_acts_only_along_k(rule):
    """For x orthogonal to k_t: M_t^T x = a_t M_{t-1}^T x, whatever beta is."""
    dk, dv = 16, 8
    q, k, v, g, beta, M0 = rand_problem(3, 1, 1, 1, dk, dv)
    x = np.random.default_rng(4).standard_normal(dk)
    x -= (x @ k[0, 0]) * k[0, 0]
    o, _ = run_tokens(x[None, None, :], k, v, g, beta, M0, rule)
    a = math.exp(g[0, 0]) if DECAY[rule] else 1.0
    np.testing.assert_allclose(o[0, 0], a * (M0[0, 0].T @ x), rtol=0, atol=1e-13)


def test_frozen_state():
    """a = 1, beta = 0 under gated_delta leaves the state unchanged: o_t = M0^T q_t."""
    T, dk, dv = 9, 16, 16
    q, k, v, g, beta, M0 = rand_problem(5, T, 2, 2, dk, dv)
    g[:] = 0.0
    beta[:] = 0.0
    o, Mt = run_tokens(q, k, v, g, beta, M0, "gated_delta")
    assert np.array_equal(Mt, M0[0])
    for h in range(2):
        np.testing.assert_allclose(o[:, h], q[:, h] @ M0[0, h], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# textbook closed forms of plain and decayed linear attention (O(T^2) brute force)

@pytest.mark.parametrize("rule", ["linear", "gated"])
def test_linear_attention_closed_form(rule):
    """o_t = (prod_{r<=t} a_r) M0^T q_t + sum_{s<=t} (prod_{s<r<=t} a_r) (k_s . q_t) v_s."""
    T, dk, dv = 14, 8, 5
    q, k, v, g, beta, M0 = rand_problem(6, T, 1, 1, dk, dv)
    a = np.exp(g[:, 0]) if rule == "gated" else np.ones(T)
    o, _ = run_tokens(q, k, v, g, beta, M0, rule, scale=0.75)
    for t in range(T):
        ref = np.prod(a[:t + 1]) * (M0[0, 0].T @ q[t, 0])
        for s in range(t + 1):
            ref = ref + np.prod(a[s + 1:t + 1]) * (k[s, 0] @ q[t, 0]) * v[s, 0]
        np.testing.assert_allclose(o[t, 0], 0.75 * ref, rtol=0, atol=1e-13)


def test_single_token_closed_form():
    """M1 = a M0 + beta k (v - a M0^T k)^T, o1 = a M0^T q + beta (k.q)(v - a M0^T k);
    from a zero state o1 = beta (k.q) v."""
    dk, dv = 12, 7
    q, k, v, g, beta, M0 = rand_problem(7, 1, 1, 1, dk, dv)
    a = math.exp(g[0, 0])
    b = beta[0, 0]
    kk, qq, vv, M = k[0, 0], q[0, 0], v[0, 0], M0[0, 0]
    resid = vv - a * (M.T @ kk)
    o, Mt = run_tokens(q, k, v, g, beta, M0, "gated_delta")
    np.testing.assert_allclose(Mt[0], a * M + b * np.outer(kk, resid), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], a * (M.T @ qq) + b * (kk @ qq) * resid, rtol=0, atol=1e-14)
    o0, _ = run_tokens(q, k, v, g, beta, np.zeros_like(M0), "gated_delta")
    np.testing.assert_allclose(o0[0, 0], b * (kk @ qq) * vv, rtol=0, atol=1e-15)


def test_residual_form_equals_literal_form():
    """The kernel's algebra: a(I - b k k^T)M + b k v^T = aM + b k (v - a M^T k)^T and
    M'^T q = a M^T q + (k.q) b (v - a M^T k) (Kimi Linear section of "Seven
    Architectures ..." with a scalar decay; "Gated DeltaNet", Engineering details)."""
    r = np.random.default_rng(8)
    dk, dv = 16, 16
    M = r.standard_normal((dk, dv))
    k = unit(r.standard_normal(dk))
    q = unit(r.standard_normal(dk))
    v = r.standard_normal(dv)
    a, b = 0.8, 0.3
    lit = a * (np.eye(dk) - b * np.outer(k, k)) @ M + b * np.outer(k, v)
    delta = b * (v - a * (M.T @ k))
    res = a * M + np.outer(k, delta)
    np.testing.assert_allclose(lit, res, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lit.T @ q, a * (M.T @ q) + (k @ q) * delta, rtol=0, atol=1e-14)
    # and the oracle agrees with the literal form
    o, Mt = run_tokens(q[None, None], k[None, None], v[None, None], np.log([[a]]), np.array([[b]]),
                       M[None, None], "gated_delta")
    np.testing.assert_allclose(Mt[0], lit, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# grouped heads, decode vs prefill, split invariance, slots

def test_grouped_heads_contiguous():
    """State head h reads q/k head floor(h * Hqk / Hv): with Hv = 2 Hqk, heads 2j and 2j+1
    share q/k head j.  Same result as explicitly repeating q, k per state head."""
    T, Hqk, Hv, dk, dv = 6, 2, 4, 8, 8
    q, k, v, g, beta, M0 = rand_problem(9, T, Hqk, Hv, dk, dv)
    o1, M1 = run_tokens(q, k, v, g, beta, M0, "gated_delta")
    qr = np.repeat(q, 2, axis=1)
    kr = np.repeat(k, 2, axis=1)
    o2, M2 = run_tokens(qr, kr, v, g, beta, M0, "gated_delta")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(M1, M2)


@pytest.mark.parametrize("rule", RULES)
def test_decode_steps_equal_sequence(rule):
    T, Hqk, Hv, dk, dv = 7, 1, 2, 8, 4
    q, k, v, g, beta, M0 = rand_problem(10, T, Hqk, Hv, dk, dv)
    o_seq, M_seq = run_tokens(q, k, v, g, beta, M0, rule)
    pool = M0.copy()
    for t in range(T):
        o_t, pool, code = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                        beta[t:t + 1], pool, [0], [0], rule=rule)
        assert code == 0
        np.testing.assert_array_equal(o_t[0], o_seq[t])
    np.testing.assert_array_equal(pool[0], M_seq)


def test_split_invariance_through_checkpoint_slot():
    """prefill(T) == prefill(T1) -> checkpoint slot -> prefill(T2) (the checkpoint read slot
    of the "Recurrent state" glossary, Why it matters)."""
    T, T1, Hqk, Hv, dk, dv = 20, 8, 1, 2, 8, 8
    q, k, v, g, beta, M0 = rand_problem(11, T, Hqk, Hv, dk, dv)
    o_full, M_full = run_tokens(q, k, v, g, beta, M0, "gated_delta")
    pool = np.zeros((3, Hv, dk, dv))
    pool[0] = M0[0]
    cu = np.array([0, T1], np.int32)
    o1, pool, _ = oracle.sequences(cu, q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], pool, [0], [2])
    cu = np.array([0, T - T1], np.int32)
    o2, pool, _ = oracle.sequences(cu, q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], pool, [2], [1])
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(pool[1], M_full, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(pool[0], M0[0])  # the source checkpoint is untouched


def test_slot_semantics():
    B, Hqk, Hv, dk, dv, n_slots = 4, 1, 2, 4, 4, 10
    q, k, v, g, beta, _ = rand_problem(12, B, Hqk, Hv, dk, dv)
    pool = np.random.default_rng(13).standard_normal((n_slots, Hv, dk, dv))
    read = np.array([3, -1, 5, 7], np.int32)
    write = np.array([0, 1, -1, 7], np.int32)
    o, after, code = oracle.decode(q, k, v, g, beta, pool, read, write)
    assert code == 0
    for s in range(n_slots):
        if s not in (0, 1, 7):
            assert np.array_equal(after[s], pool[s]), s
    # read -1 starts from zero; write -1 stores nothing but still produces o
    zero_pool = np.zeros((1, Hv, dk, dv))
    o1, p1, _ = oracle.decode(q[1:2], k[1:2], v[1:2], g[1:2], beta[1:2], zero_pool, [0], [0])
    np.testing.assert_array_equal(o[1], o1[0])
    np.testing.assert_array_equal(after[1], p1[0])
    o2, _, _ = oracle.decode(q[2:3], k[2:3], v[2:3], g[2:3], beta[2:3], pool[5:6], [0], [0])
    np.testing.assert_array_equal(o[2], o2[0])
    # an out-of-range slot skips that request only
    bad = np.array([3, 10, 5, 7], np.int32)
    o3, after3, code3 = oracle.decode(q, k, v, g, beta, pool, bad, write)
    assert code3 == 1
    assert np.array_equal(after3[1], pool[1]) and np.all(o3[1] == 0)
    np.testing.assert_array_equal(after3[0], after[0])


# --------------------------------------------------------------------------
# the chunked algebra the prefill uses, against the token recurrence

@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("C", [4, 16, 64])
def test_chunked_form_matches_token_recurrence(rule, C):
    from chunk_model import chunked_sequence
    T, dk, dv = 150, 16, 12
    q, k, v, g, beta, M0 = rand_problem(14, T, 1, 1, dk, dv)
    o_ref, M_ref = run_tokens(q, k, v, g, beta, M0, rule, scale=0.5)
    o, M = chunked_sequence(M0[0, 0], q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], rule, C,
                            scale=0.5)
    np.testing.assert_allclose(o, o_ref[:, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(M, M_ref[0], rtol=0, atol=1e-11)


# --------------------------------------------------------------------------
# BF16 rounding of the stored state ("Recurrent state", Why it matters)

def test_round_bf16_matches_torch_on_float32_values():
    r = np.random.default_rng(15)
    bits = r.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # exact ties: a BF16 value plus half a unit in the last place
    base = r.integers(0, 2**16, size=5000, dtype=np.uint64).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1.17549435e-38,
                         3.3895314e38, 3.4028235e38, 1.0, 1.00390625, 1.01171875],
                        np.float32)
    allx = np.concatenate([x, ties, specials])
    ref = torch.from_numpy(allx).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(allx.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.isnan(oracle.round_bf16(np.array([np.nan])))[0]


def test_round_bf16_is_direct_not_via_float32():
    # 1 + 2^-8 + 2^-40 is just above the midpoint between 1 and 1 + 2^-7, so the nearest
    # BF16 value is 1 + 2^-7; rounding through float32 first would land on the tie and
    # then round to even (1.0).
    x = 1.0 + 2.0**-8 + 2.0**-40
    assert oracle.round_bf16(np.array([x]))[0] == 1.0 + 2.0**-7
    assert oracle.round_bf16(np.array([1.0 + 2.0**-8]))[0] == 1.0        # tie -> even
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0**-8]))[0] == 1.0 + 2.0**-6  # tie -> even


def test_state_rounded_to_bf16_where_stored():
    """BF16 storage: a decode step stores round(M_1); a sequence stores only round(M_T)
    (the state stays in high precision between tokens of one call)."""
    T, Hqk, Hv, dk, dv = 5, 1, 2, 8, 8
    q, k, v, g, beta, M0 = rand_problem(16, T, Hqk, Hv, dk, dv)
    M0 = torch.from_numpy(M0).to(torch.bfloat16).double().numpy()
    _, p_exact, _ = oracle.decode(q[:1], k[:1], v[:1], g[:1], beta[:1], M0, [0], [0])
    _, p_round, _ = oracle.decode(q[:1], k[:1], v[:1], g[:1], beta[:1], M0, [0], [0],
                                  round_state=True)
    want = torch.from_numpy(p_exact).float().to(torch.bfloat16).double().numpy()
    # the exact state is far from any tie, so rounding via float32 agrees here
    np.testing.assert_array_equal(p_round, want)
    assert not np.array_equal(p_round, p_exact)
    cu = np.array([0, T], np.int32)
    _, s_exact, _ = oracle.sequences(cu, q, k, v, g, beta, M0, [0], [0])
    _, s_round, _ = oracle.sequences(cu, q, k, v, g, beta, M0, [0], [0], round_state=True)
    np.testing.assert_array_equal(s_round, oracle.round_bf16(s_exact))
