"""Independent formulations used to pin the oracle (test side only).

Nothing here is imported by the oracle or by the HIP path.  Each function
computes a quantity the oracle also computes, by a different route:

* ``product_form_exact``: the closed product form of the gated delta rule in
  exact rational arithmetic (``fractions.Fraction``), for tiny T and d.
* ``chunked_form``: the chunked WY/UT evaluation of the same recurrence
  (the "chunked" FLA operation named in LightLLM #1097, Highlights), in fp64.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


# ------------------------------------------------------------ exact product form
def _mat_mul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][k] * B[k][j] for k in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _mat_add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _scale(A, s):
    return [[a * s for a in r] for r in A]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _outer(u, v):
    return [[a * b for b in v] for a in u]


def product_form_exact(alpha, beta, K, V, Q, S0):
    """Gated delta rule by its unrolled product form, exactly.

    With A_t = alpha_t (I - beta_t k_t k_t^T) (a d_k x d_k matrix):
        S_T = S_0 A_1 ... A_T + sum_t beta_t v_t k_t^T A_{t+1} ... A_T
        o_t = S_t q_t
    alpha, beta: lists of Fractions (length T); K, Q: lists of d_k-vectors;
    V: list of d_v-vectors; S0: d_v x d_k.  Returns (o list, S_T).
    """
    T = len(alpha)
    dk = len(K[0])
    A = [_scale(_mat_add(_eye(dk), _scale(_outer(K[t], K[t]), -beta[t])), alpha[t]) for t in range(T)]
    o, S_t = [], None
    for t_end in range(1, T + 1):
        S = S0
        for t in range(t_end):
            S = _mat_mul(S, A[t])
        for t in range(t_end):
            term = _scale(_outer(V[t], K[t]), beta[t])
            for s in range(t + 1, t_end):
                term = _mat_mul(term, A[s])
            S = _mat_add(S, term)
        o.append([sum((S[i][j] * Q[t_end - 1][j] for j in range(dk)), Fraction(0)) for i in range(len(S))])
        S_t = S
    return o, S_t


# ------------------------------------------------------------- chunked form
def chunked_form(q, k, v, g, beta, S0, chunk, scale=1.0):
    """Chunked WY/UT evaluation of the gated delta rule for one head, fp64.

    q, k [T, d_k] normalised; v [T, d_v]; g, beta [T]; S0 [d_v, d_k].
    Per chunk of n <= chunk tokens with incoming S0 and G = cumsum(g):
      A_ij = beta_i exp(G_i - G_j) k_i.k_j (i > j), T = (I + A)^-1
      W = T diag(beta e^G) K,  U~ = T diag(beta) V,  U = U~ - W S0^T
      O = diag(e^G) Q S0^T + (M o Q K^T) U,  M_ij = exp(G_i - G_j) (j <= i)
      S = e^{G_n} S0 + U^T diag(e^{G_n - G}) K
    Every exponent is a non-positive difference, masked before exp.
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    S = np.array(S0, np.float64)
    T = len(g)
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        Q, K, Vc, gc, bc = q[sl], k[sl], v[sl], g[sl], beta[sl]
        n = len(gc)
        G = np.cumsum(gc)
        diff = G[:, None] - G[None, :]
        lower = np.tril(np.ones((n, n), bool), -1)
        lower_eq = np.tril(np.ones((n, n), bool), 0)
        A = np.where(lower, bc[:, None] * np.exp(np.where(lower, diff, 0.0)) * (K @ K.T), 0.0)
        Tm = np.linalg.inv(np.eye(n) + A)
        W = Tm @ (bc[:, None] * np.exp(G)[:, None] * K)
        Ut = Tm @ (bc[:, None] * Vc)
        U = Ut - W @ S.T
        M = np.where(lower_eq, np.exp(np.where(lower_eq, diff, 0.0)), 0.0)
        o[sl] = scale * (np.exp(G)[:, None] * (Q @ S.T) + (M * (Q @ K.T)) @ U)
        S = np.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
    return o, S
