"""Chunkwise (WY / UT-transform) form of the gated delta rule, fp64, numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is not the
oracle: the oracle is the sequential token-by-token definition in
``gdn_oracle.c``.  This module restates, independently, the blocked algebra a
fast implementation relies on, so that a test can show on tiny inputs that
the blocked form reaches the same numbers as the definition.

Source of the idea: the course page "Chapitre 16 - Assembler un systeme de
type Kimi K3", section 16.2 (prefill of recurrent layers works block by
block with large matrix products inside each block and the state handed on
from block to block; its example cuts 256 prompt tokens into 4 blocks of
64).  The pages give no algebra for it; the derivation below is ours.

Derivation (state stored as M = S^T, [Dk][Dv]): one token maps
    M_t = a_t (I - b_t k_t k_t^T) M_{t-1} + b_t k_t v_t^T.
Inside a chunk with rows r = 0..n-1, entry state M0, g_r = sum_{i<=r} log a_i
and gamma_r = exp(g_r), unrolling gives
    M_r = gamma_r M0 + sum_{i<=r} exp(g_r - g_i) k_i u_i^T
for "pseudo-values" u_i that satisfy the unit lower-triangular system
    u_r + b_r sum_{i<r} exp(g_r - g_i) (k_r . k_i) u_i = b_r (v_r - gamma_r M0^T k_r).
Writing A_ri = b_r exp(g_r - g_i) (k_r . k_i) for i < r and T = (I + A)^-1:
    U = T diag(b) (V - diag(gamma) K M0)                       ("fused" grouping)
      = T diag(b) V - T diag(b gamma) K M0 = U~ - W M0          ("wy" grouping)
    O = diag(gamma) Q M0 + (P o (Q K^T)) U,  P_ri = exp(g_r - g_i) for i <= r
    M_n = gamma_{n-1} M0 + K^T diag(exp(g_{n-1} - g)) U.
Every exponent used is <= 0.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunked_head(q, k, v, log_alpha, beta, M0=None, C: int = 64, form: str = "fused"):
    """One head.  q, k: [T, Dk]; v: [T, Dv]; log_alpha, beta: [T]; M0: [Dk, Dv].
    Returns (o [T, Dv], M [Dk, Dv]) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    la = np.asarray(log_alpha, np.float64)
    be = np.asarray(beta, np.float64)
    T, Dk = q.shape
    Dv = v.shape[1]
    M = np.zeros((Dk, Dv)) if M0 is None else np.array(M0, np.float64)
    o = np.zeros((T, Dv))
    for s in range(0, T, C):
        e = min(s + C, T)
        n = e - s
        Q, K, V, b = q[s:e], k[s:e], v[s:e], be[s:e]
        g = np.cumsum(la[s:e])
        gamma = np.exp(g)
        diff = g[:, None] - g[None, :]
        lower = np.tril(np.ones((n, n), dtype=bool))
        E = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)   # exp(g_r - g_i), i <= r
        strict = np.tril(np.ones((n, n), dtype=bool), -1)
        A = np.where(strict, b[:, None] * E * (K @ K.T), 0.0)
        I_plus_A = np.eye(n) + A
        if form == "fused":
            rhs = b[:, None] * (V - gamma[:, None] * (K @ M))
            U = solve_triangular(I_plus_A, rhs, lower=True, unit_diagonal=True)
        elif form == "wy":
            W = solve_triangular(I_plus_A, (b * gamma)[:, None] * K, lower=True, unit_diagonal=True)
            Ut = solve_triangular(I_plus_A, b[:, None] * V, lower=True, unit_diagonal=True)
            U = Ut - W @ M
        else:
            raise ValueError(form)
        o[s:e] = gamma[:, None] * (Q @ M) + (E * (Q @ K.T)) @ U
        M = gamma[-1] * M + K.T @ (np.exp(g[-1] - g)[:, None] * U)
    return o, M


def decode_single_pass(M, q, k, v, log_alpha, beta):
    """One token from state M ([Dk, Dv]) with one read of M:
    u = M^T k, w = M^T q, d = b (v - a u), M' = a M + k d^T, o = a w + (k . q) d.
    (o equals M'^T q: M'^T q = a M^T q + d (k . q).)"""
    M = np.asarray(M, np.float64)
    a = np.exp(log_alpha)
    u = M.T @ k
    w = M.T @ q
    d = beta * (v - a * u)
    return a * w + (k @ q) * d, a * M + np.outer(k, d)
