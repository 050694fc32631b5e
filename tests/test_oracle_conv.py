"""Pins of the oracle's decode-side conv step (conv window kept in slots).

The short conv is part of a Gated DeltaNet layer ("Gated DeltaNet" glossary,
Engineering details), so a decode token's conv window is the raw inputs of
the tokens before it.  Pinned here to the prefill front-end (itself pinned by
brute force in test_oracle_frontend.py): decoding a sequence token by token
from an empty window reproduces the front-end over the whole sequence, and
the window left behind equals the sequence's last raw inputs.  Closed forms
pin the tap order and the slot rules.
"""
import math

import numpy as np

import oracle

K = 4


def raw(seed, N, Hqk, Hv, dk, dv):
    r = np.random.default_rng(seed)
    return dict(
        q_raw=r.standard_normal((N, Hqk * dk)), k_raw=r.standard_normal((N, Hqk * dk)),
        v_raw=r.standard_normal((N, Hv * dv)), wq=r.standard_normal((Hqk * dk, K)) * 0.5,
        wk=r.standard_normal((Hqk * dk, K)) * 0.5, wv=r.standard_normal((Hv * dv, K)) * 0.5,
        a_raw=r.standard_normal((N, Hv)), b_raw=r.standard_normal((N, Hv)))


def step(x, rows, pool, rs, ws, Hqk, Hv, eps=1e-6):
    sel = lambda a: a[rows]
    return oracle.conv_decode(sel(x["q_raw"]), sel(x["k_raw"]), sel(x["v_raw"]), x["wq"], x["wk"],
                              x["wv"], sel(x["a_raw"]), sel(x["b_raw"]), pool,
                              np.asarray(rs, np.int32), np.asarray(ws, np.int32),
                              Hqk=Hqk, Hv=Hv, eps=eps)


def test_token_by_token_equals_frontend_and_leaves_the_tail():
    Hqk, Hv, dk, dv = 2, 4, 3, 2
    cu = np.array([0, 1, 3, 8, 14], np.int32)   # lengths 1, 2, 5, 6: shorter and longer than K-1
    N = int(cu[-1])
    x = raw(3, N, Hqk, Hv, dk, dv)
    q, k, v, g, beta = oracle.frontend(cu, x["q_raw"], x["k_raw"], x["v_raw"], x["wq"], x["wk"],
                                       x["wv"], x["a_raw"], x["b_raw"], Hqk=Hqk, Hv=Hv)
    tail = oracle.conv_tail(cu, x["q_raw"], x["k_raw"], x["v_raw"], K)
    C = 2 * Hqk * dk + Hv * dv
    for s in range(len(cu) - 1):
        pool = np.full((2, K - 1, C), 7.0)   # slot 0 live, slot 1 untouched
        for t in range(cu[s], cu[s + 1]):
            first = t == cu[s]
            qd, kd, vd, gd, bd, pool, code = step(x, [t], pool, [-1 if first else 0], [0], Hqk, Hv)
            assert code == 0
            np.testing.assert_allclose(qd[0], q[t], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(kd[0], k[t], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(vd[0], v[t], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(gd[0], g[t], rtol=1e-15)
            np.testing.assert_allclose(bd[0], beta[t], rtol=1e-15)
        np.testing.assert_array_equal(pool[0], tail[s])
        np.testing.assert_array_equal(pool[1], np.full((K - 1, C), 7.0))


def test_tail_is_the_last_raw_inputs_zero_padded():
    Hqk, Hv, dk, dv = 1, 1, 2, 2
    cu = np.array([0, 2, 6], np.int32)
    x = raw(4, 6, Hqk, Hv, dk, dv)
    tail = oracle.conv_tail(cu, x["q_raw"], x["k_raw"], x["v_raw"], K)
    rows = np.concatenate([x["q_raw"], x["k_raw"], x["v_raw"]], axis=1)
    np.testing.assert_array_equal(tail[0, 0], np.zeros(rows.shape[1]))   # before token 0
    np.testing.assert_array_equal(tail[0, 1:], rows[0:2])
    np.testing.assert_array_equal(tail[1], rows[3:6])


def test_one_hot_taps_select_the_window_entry():
    # tap j alone: the v output is SiLU of the window entry j (j = 0 oldest, K-1 current)
    Hqk, Hv, dk, dv = 1, 2, 2, 3
    x = raw(5, 1, Hqk, Hv, dk, dv)
    C = 2 * Hqk * dk + Hv * dv
    hist = np.random.default_rng(6).standard_normal((1, K - 1, C))
    window_v = np.concatenate([hist[0, :, 2 * Hqk * dk:], x["v_raw"]], axis=0)  # [K, Hv*dv]
    silu = lambda s: s / (1.0 + np.exp(-s))
    for j in range(K):
        xj = dict(x)
        xj["wv"] = np.zeros_like(x["wv"])
        xj["wv"][:, j] = 1.0
        _, _, vd, _, _, _, _ = step(xj, [0], hist, [0], [-1], Hqk, Hv)
        np.testing.assert_allclose(vd.reshape(-1), silu(window_v[j]), rtol=1e-15)


def test_worked_example_one_channel():
    # taps (1, 2, 3, 4) over history (1, 0, -1) and input 0.5: 1 + 0 - 3 + 2 = 0 -> SiLU 0;
    # all-ones taps over history (0.5, 0.25, 0) and input 1: 1.75 * sigmoid(1.75)
    Hqk, Hv, dk, dv = 1, 1, 1, 1
    base = dict(q_raw=np.ones((1, 1)), k_raw=np.ones((1, 1)), wq=np.ones((1, K)),
                wk=np.ones((1, K)), a_raw=np.zeros((1, 1)), b_raw=np.zeros((1, 1)))
    hist = np.zeros((1, K - 1, 3))
    hist[0, :, 2] = [1.0, 0.0, -1.0]
    x = dict(base, v_raw=np.array([[0.5]]), wv=np.array([[1.0, 2.0, 3.0, 4.0]]))
    _, _, vd, g, beta, _, _ = step(x, [0], hist, [0], [-1], Hqk, Hv)
    assert vd[0, 0, 0] == 0.0
    assert g[0, 0] == -math.log(2.0) and beta[0, 0] == 0.5   # -softplus(0), sigmoid(0)
    hist[0, :, 2] = [0.5, 0.25, 0.0]
    x = dict(base, v_raw=np.array([[1.0]]), wv=np.ones((1, K)))
    _, _, vd, _, _, pool, _ = step(x, [0], hist, [0], [0], Hqk, Hv)
    assert math.isclose(vd[0, 0, 0], 1.75 / (1.0 + math.exp(-1.75)), rel_tol=1e-15)
    np.testing.assert_array_equal(pool[0, :, 2], [0.25, 0.0, 1.0])   # the window slid by one


def test_batch_routes_slots_and_skips_bad_requests():
    Hqk, Hv, dk, dv = 2, 2, 4, 2
    B, n_slots = 4, 6
    x = raw(7, B, Hqk, Hv, dk, dv)
    C = 2 * Hqk * dk + Hv * dv
    pool0 = np.random.default_rng(8).standard_normal((n_slots, K - 1, C))
    rs, ws = [3, -1, 0, 5], [3, 1, -1, 2]
    out = step(x, list(range(B)), pool0, rs, ws, Hqk, Hv)
    assert out[6] == 0
    expect_pool = pool0.copy()
    for r in range(B):   # each request alone gives the same outputs and slot contents
        one = step(x, [r], pool0, [rs[r]], [ws[r]], Hqk, Hv)
        for a, b in zip(out[:5], one[:5]):
            np.testing.assert_array_equal(a[r], b[0])
        if ws[r] >= 0:
            expect_pool[ws[r]] = one[5][ws[r]]
    np.testing.assert_array_equal(out[5], expect_pool)
    # request 1 had no history: its window is zeros then its own input
    fresh = step(x, [1], np.zeros((1, K - 1, C)), [0], [-1], Hqk, Hv)
    np.testing.assert_array_equal(out[2][1], fresh[2][0])
    # a slot index out of range skips that request only
    bad = step(x, list(range(B)), pool0, [3, -1, 6, 5], ws, Hqk, Hv)
    assert bad[6] == 1
    assert not bad[0][2].any() and not bad[2][2].any()
    np.testing.assert_array_equal(bad[0][0], out[0][0])
    np.testing.assert_array_equal(bad[5][3], out[5][3])


def frontend_of(x, cu, Hqk, Hv, init=None):
    return oracle.frontend(cu, x["q_raw"], x["k_raw"], x["v_raw"], x["wq"], x["wk"], x["wv"],
                           x["a_raw"], x["b_raw"], Hqk=Hqk, Hv=Hv, conv_init=init)


def part(x, a, b):
    return {n: (x[n][a:b] if n not in ("wq", "wk", "wv") else x[n]) for n in x}


def test_resumed_frontend_equals_the_whole_sequence():
    """A sequence cut into three parts, each resumed from the window the
    previous one left (the middle part shorter than K-1 tokens, so its window
    keeps rows of the first part's), gives the whole sequence's front-end
    bit for bit."""
    Hqk, Hv, dk, dv = 2, 2, 3, 2
    T, T1, T2 = 11, 5, 7
    x = raw(9, T, Hqk, Hv, dk, dv)
    whole = frontend_of(x, np.array([0, T], np.int32), Hqk, Hv)
    init = None
    outs = []
    for a, b in ((0, T1), (T1, T2), (T2, T)):
        xp = part(x, a, b)
        cu = np.array([0, b - a], np.int32)
        outs.append(frontend_of(xp, cu, Hqk, Hv, init))
        init = oracle.conv_tail(cu, xp["q_raw"], xp["k_raw"], xp["v_raw"], K, conv_init=init)
    for i in range(5):
        np.testing.assert_array_equal(np.concatenate([o[i] for o in outs]), whole[i])
    # the last window is the whole sequence's tail
    np.testing.assert_array_equal(init, oracle.conv_tail(np.array([0, T], np.int32), x["q_raw"],
                                                         x["k_raw"], x["v_raw"], K))


def test_resumed_frontend_equals_decode_steps():
    """T tokens from a stored window W through the front-end equal T
    conv-decode steps starting from a slot holding W."""
    Hqk, Hv, dk, dv = 1, 2, 4, 3
    T = 6
    x = raw(10, T, Hqk, Hv, dk, dv)
    C = 2 * Hqk * dk + Hv * dv
    W = np.random.default_rng(11).standard_normal((1, K - 1, C))
    q, k, v, g, beta = frontend_of(x, np.array([0, T], np.int32), Hqk, Hv, W)
    pool = W.copy()
    for t in range(T):
        qd, kd, vd, gd, bd, pool, code = step(x, [t], pool, [0], [0], Hqk, Hv)
        assert code == 0
        np.testing.assert_allclose(qd[0], q[t], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(kd[0], k[t], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(vd[0], v[t], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(pool[0], oracle.conv_tail(np.array([0, T], np.int32),
                                                            x["q_raw"], x["k_raw"], x["v_raw"],
                                                            K, conv_init=W)[0])


def test_oldest_tap_reads_the_stored_window():
    """With only the oldest tap set, output t of a resumed sequence is SiLU of
    the raw input three tokens back: window rows 0, 1, 2 for its first three
    tokens, then its own inputs."""
    Hqk, Hv, dk, dv = 1, 1, 2, 2
    T = 5
    x = raw(12, T, Hqk, Hv, dk, dv)
    for n in ("wq", "wk", "wv"):
        x[n] = np.zeros_like(x[n])
        x[n][:, 0] = 1.0
    C = 2 * Hqk * dk + Hv * dv
    W = np.random.default_rng(13).standard_normal((1, K - 1, C))
    _, _, v, _, _ = frontend_of(x, np.array([0, T], np.int32), Hqk, Hv, W)
    silu = lambda s: s / (1.0 + np.exp(-s))
    vch = slice(2 * Hqk * dk, C)
    for t in range(T):
        src = W[0, t, vch] if t < K - 1 else x["v_raw"][t - (K - 1)]
        np.testing.assert_allclose(v[t].reshape(-1), silu(src), rtol=1e-15)


def test_windows_stay_with_their_sequences():
    """A batch of sequences (one empty, one shorter than the window) with
    windows of their own equals each sequence run alone with its window; the
    windows left behind keep the older rows of short sequences."""
    Hqk, Hv, dk, dv = 1, 2, 2, 2
    lengths = [4, 0, 2, 6]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = int(cu[-1])
    x = raw(14, N, Hqk, Hv, dk, dv)
    C = 2 * Hqk * dk + Hv * dv
    W = np.random.default_rng(15).standard_normal((len(lengths), K - 1, C))
    got = frontend_of(x, cu, Hqk, Hv, W)
    tail = oracle.conv_tail(cu, x["q_raw"], x["k_raw"], x["v_raw"], K, conv_init=W)
    for s, L in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        xs = part(x, a, b)
        one = frontend_of(xs, np.array([0, L], np.int32), Hqk, Hv, W[s:s + 1])
        for i in range(5):
            np.testing.assert_array_equal(got[i][a:b], one[i])
        rows = np.concatenate([W[s], np.concatenate([xs["q_raw"], xs["k_raw"], xs["v_raw"]], 1)])
        np.testing.assert_array_equal(tail[s], rows[-(K - 1):])
