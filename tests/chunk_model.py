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
