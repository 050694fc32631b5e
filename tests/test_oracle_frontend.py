"""Pins of the oracle's front-end (causal depthwise conv + SiLU, L2 norm, gates).

The conv is fused with the layer on the "Gated DeltaNet" glossary page
(Engineering details); its width, SiLU and the q/k normalisation come from the
prefill workload description.  Checked here by brute force on tiny inputs,
by causality and sequence isolation, and by closed forms at chosen points.
"""
import math

import numpy as np

import oracle


def tiny(seed, N, Hqk, Hv, dk, dv, K=4):
    r = np.random.default_rng(seed)
    return dict(
        q_raw=r.standard_normal((N, Hqk * dk)), k_raw=r.standard_normal((N, Hqk * dk)),
        v_raw=r.standard_normal((N, Hv * dv)), wq=r.standard_normal((Hqk * dk, K)) * 0.5,
        wk=r.standard_normal((Hqk * dk, K)) * 0.5, wv=r.standard_normal((Hv * dv, K)) * 0.5,
        a_raw=r.standard_normal((N, Hv)), b_raw=r.standard_normal((N, Hv)))


def run(cu, x, Hqk, Hv, eps=1e-6):
    return oracle.frontend(np.asarray(cu, np.int32), x["q_raw"], x["k_raw"], x["v_raw"], x["wq"],
                           x["wk"], x["wv"], x["a_raw"], x["b_raw"], Hqk=Hqk, Hv=Hv, eps=eps)


def test_conv_silu_norm_brute_force():
    N, Hqk, Hv, dk, dv, K = 11, 2, 4, 3, 2, 4
    cu = [0, 5, 11]
    x = tiny(1, N, Hqk, Hv, dk, dv, K)
    q, k, v, g, beta = run(cu, x, Hqk, Hv)

    def ref_conv(raw, w):
        out = np.zeros_like(raw)
        for s in range(len(cu) - 1):
            for t in range(cu[s], cu[s + 1]):
                for c in range(raw.shape[1]):
                    acc = 0.0
                    for j in range(K):  # tap j sees the token j - (K-1) steps away
                        src = t - (K - 1) + j
                        if src >= cu[s]:
                            acc += w[c, j] * raw[src, c]
                    out[t, c] = acc / (1.0 + math.exp(-acc))  # SiLU
        return out

    yq, yk, yv = ref_conv(x["q_raw"], x["wq"]), ref_conv(x["k_raw"], x["wk"]), ref_conv(x["v_raw"], x["wv"])
    for t in range(N):
        for h in range(Hqk):
            for y, got in ((yq, q), (yk, k)):
                seg = y[t, h * dk:(h + 1) * dk]
                np.testing.assert_allclose(got[t, h], seg / math.sqrt(seg @ seg + 1e-6), atol=1e-14)
    np.testing.assert_allclose(v.reshape(N, -1), yv, atol=1e-14)
    np.testing.assert_allclose(g, -np.log1p(np.exp(x["a_raw"])), atol=1e-14)
    np.testing.assert_allclose(beta, 1.0 / (1.0 + np.exp(-x["b_raw"])), atol=1e-15)


def test_gate_closed_forms():
    N, Hqk, Hv, dk, dv = 3, 1, 1, 2, 2
    x = tiny(2, N, Hqk, Hv, dk, dv)
    x["a_raw"][:, 0] = [0.0, 800.0, -800.0]
    x["b_raw"][:, 0] = [0.0, 800.0, -800.0]
    _, _, _, g, beta = run([0, N], x, Hqk, Hv)
    assert g[0, 0] == -math.log(2.0)          # softplus(0) = ln 2
    assert g[1, 0] == -800.0                   # softplus(x) -> x, no overflow
    assert g[2, 0] == 0.0 or abs(g[2, 0]) < 1e-300  # softplus(-800) underflows to 0
    assert beta[0, 0] == 0.5 and beta[1, 0] == 1.0 and beta[2, 0] == 0.0


def test_unit_norm_and_eps():
    N, Hqk, Hv, dk, dv = 6, 2, 2, 8, 4
    x = tiny(3, N, Hqk, Hv, dk, dv)
    q, k, _, _, _ = run([0, N], x, Hqk, Hv, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-14)
    # with eps the squared norm is s / (s + eps)
    x["q_raw"] *= 1e-3
    qe, _, _, _, _ = run([0, N], x, Hqk, Hv, eps=1e-6)
    q0, _, _, _, _ = run([0, N], x, Hqk, Hv, eps=0.0)
    # q0 is the unit vector; qe = y / sqrt(s + eps) so |qe|^2 = s/(s+eps) < 1
    n2 = np.sum(qe**2, axis=-1)
    assert np.all(n2 < 1.0) and np.all(n2 > 0.0)
    np.testing.assert_allclose(qe / np.sqrt(n2)[..., None], q0, atol=1e-12)


def test_causality():
    N, Hqk, Hv, dk, dv = 16, 1, 2, 4, 4
    x = tiny(4, N, Hqk, Hv, dk, dv)
    base = run([0, N], x, Hqk, Hv)
    t = 9
    for key in ("q_raw", "k_raw", "v_raw"):
        y = {kk: vv.copy() for kk, vv in x.items()}
        y[key][t] += 5.0
        pert = run([0, N], y, Hqk, Hv)
        for a, b in zip(base[:3], pert[:3]):
            np.testing.assert_array_equal(a[:t], b[:t])       # the past is untouched
        idx = ("q_raw", "k_raw", "v_raw").index(key)
        assert not np.array_equal(base[idx][t], pert[idx][t])  # the token itself moves
        np.testing.assert_array_equal(base[idx][t + 4:], pert[idx][t + 4:])  # window is 4 wide


def test_no_leak_across_sequences():
    N, Hqk, Hv, dk, dv = 12, 1, 1, 4, 4
    cu = [0, 5, 12]
    x = tiny(5, N, Hqk, Hv, dk, dv)
    base = run(cu, x, Hqk, Hv)
    y = {kk: vv.copy() for kk, vv in x.items()}
    for key in ("q_raw", "k_raw", "v_raw"):
        y[key][:5] = 123.0
    pert = run(cu, y, Hqk, Hv)
    for a, b in zip(base, pert):
        np.testing.assert_array_equal(a[5:], b[5:])
    # and the second sequence equals running it alone
    solo = {kk: (vv[5:] if kk in ("q_raw", "k_raw", "v_raw", "a_raw", "b_raw") else vv)
            for kk, vv in x.items()}
    alone = run([0, 7], solo, Hqk, Hv)
    for a, b in zip(base, alone):
        np.testing.assert_array_equal(a[5:], b)
