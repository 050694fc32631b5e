"""Float64 NumPy model of the chunked (WY-style) form of the recurrence.

This is the algebra the GPU prefill implements, written out plainly so that
tests can check it against the token-by-token oracle before trusting any
kernel built on it.  It is NOT the oracle and the oracle does not use it.

Within a chunk of n tokens with initial state M0 (d_k x d_v), write the
per-token update as M_r = a_r M_{r-1} + k_r u_r^T with
u_r = beta_r (v_r - a_r M_{r-1}^T k_r) (the residual form of the Kimi Delta
Attention update with a scalar decay, "Seven Architectures ...", section Kimi
Linear).  With G = cumsum(log a), gamma = exp(G):

  (I + A) U = diag(beta) V - diag(beta*gamma) K M0,
  A[r, s] = beta_r exp(G_r - G_s) (k_r . k_s)   for s < r, else 0
  U = U' - W M0,  U' = T diag(beta) V,  W = T diag(beta*gamma) K,  T = (I + A)^-1
  O = diag(gamma) Q M0 + (L o Q K^T) U,  L[r, s] = exp(G_r - G_s) for s <= r
  M_n = gamma_n M0 + (diag(exp(G_n - G)) K)^T U
"""
import numpy as np

ERASE = {"linear": False, "gated": False, "delta": True, "gated_delta": True}
DECAY = {"linear": False, "gated": True, "delta": False, "gated_delta": True}


def chunk_step(M0, q, k, v, g, beta, rule):
    n = q.shape[0]
    G = np.cumsum(g) if DECAY[rule] else np.zeros(n)
    gamma = np.exp(G)
    D = G[:, None] - G[None, :]
    low_strict = np.tril(np.ones((n, n)), -1)
    low_incl = np.tril(np.ones((n, n)))
    Ldec = np.exp(np.where(low_incl > 0, D, 0.0)) * low_incl
    if ERASE[rule]:
        A = beta[:, None] * np.exp(np.where(low_strict > 0, D, 0.0)) * (k @ k.T) * low_strict
        T = np.linalg.inv(np.eye(n) + A)
        Up = T @ (beta[:, None] * v)
        W = T @ ((beta * gamma)[:, None] * k)
    else:
        Up = v.copy()
        W = np.zeros_like(k)
    U = Up - W @ M0
    O = gamma[:, None] * (q @ M0) + (Ldec * (q @ k.T)) @ U
    Kt = np.exp(G[-1] - G)[:, None] * k
    Mn = gamma[-1] * M0 + Kt.T @ U
    return O, Mn


def chunked_sequence(M0, q, k, v, g, beta, rule, C, scale=1.0):
    """Run one head of one sequence chunk by chunk.  Returns (o [T, d_v], M_T)."""
    T = q.shape[0]
    M = M0.copy()
    outs = []
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        O, M = chunk_step(M, q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], rule)
        outs.append(O)
    o = np.concatenate(outs, axis=0) if outs else np.zeros((0, M0.shape[1]))
    return scale * o, M


def chunk_step_cw(M0, q, k, v, g, beta, rule, sub=16):
    """The chunked form with one decay per key channel (Kimi Delta Attention,
    "Seven Architectures ...", Kimi Linear section), as the GPU chain forms
    it.  g: [n, d_k] log-decays.  Per channel i, G[:, i] = cumsum(g[:, i]);
    the scalar form's gamma-weighted rows become per-channel scalings:

      K_g = K o e^G,  Q_g = Q o e^G,  K_e = K o e^(G_n - G)
      A[r, s] = beta_r sum_i k_ri k_si e^(G_ri - G_si)      (s < r)
      P[r, s] =        sum_i q_ri k_si e^(G_ri - G_si)      (s <= r)
      (I + A) U = diag(beta) (V - K_g M0)   (delta rules; else U = V)
      O = Q_g M0 + P U,   M_n = diag(e^(G_n)) M0 + K_e^T U

    A and P are formed in sub x sub tiles.  Below the diagonal, tile (I, J)
    factors the weight through the last token m of column tile J:
    e^(G_r - G_s) = e^(G_r - G_m) e^(G_m - G_s), both factors <= 1 for r > m >= s,
    so a product of two scaled matrices (the MFMA form) neither overflows nor
    loses a weight that is O(1).  Diagonal tiles have no such reference and
    take the weight of every (r, s, i) directly."""
    n, dk = k.shape
    decay, erase = DECAY[rule], ERASE[rule]
    G = np.cumsum(g, axis=0) if decay else np.zeros((n, dk))
    Kg, Qg = k * np.exp(G), q * np.exp(G)
    Ke = k * np.exp(G[-1] - G)
    A = np.zeros((n, n))
    P = np.zeros((n, n))
    for I in range(0, n, sub):
        for J in range(0, I + 1, sub):
            rI, rJ = slice(I, min(n, I + sub)), slice(J, min(n, J + sub))
            if I > J:
                m = min(n, J + sub) - 1
                L = np.exp(G[rI] - G[m])          # <= 1
                R = np.exp(G[m] - G[rJ])          # <= 1
                A[rI, rJ] = (k[rI] * L) @ (k[rJ] * R).T
                P[rI, rJ] = (q[rI] * L) @ (k[rJ] * R).T
            else:
                for r in range(I, min(n, I + sub)):
                    for s in range(J, r + 1):
                        w = np.exp(G[r] - G[s])
                        P[r, s] = np.sum(q[r] * k[s] * w)
                        if s < r:
                            A[r, s] = np.sum(k[r] * k[s] * w)
    if erase:
        A = beta[:, None] * A
        U = np.linalg.solve(np.eye(n) + A, beta[:, None] * (v - Kg @ M0))
    else:
        U = v.copy()
    O = Qg @ M0 + P @ U
    Mn = np.exp(G[-1])[:, None] * M0 + Ke.T @ U
    return O, Mn


def chunked_sequence_cw(M0, q, k, v, g, beta, rule, C, scale=1.0, sub=16):
    """One head of one sequence chunk by chunk with a per-channel decay."""
    T = q.shape[0]
    M = M0.copy()
    outs = []
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        O, M = chunk_step_cw(M, q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], rule, sub)
        outs.append(O)
    o = np.concatenate(outs, axis=0) if outs else np.zeros((0, M0.shape[1]))
    return scale * o, M
