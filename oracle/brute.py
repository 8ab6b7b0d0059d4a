"""TEST INFRASTRUCTURE ONLY: brute-force forms used to pin the oracle.

1. explicit transition products ("Gated Delta Network（GDN）", §4.1(a),
   eqs. 7-8; "TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.1, paper eq. 10):
       S_r = S_0 P_r + H_r ,  P_r = prod_{i<=r} A_i ,
       H_r = sum_{i<=r} beta_i v_i k_i^T prod_{j=i+1..r} A_j ,
   with the K-by-K transition A_i = alpha_i (I - beta_i k_i k_i^T) (scalar
   gate) or Diag(gamma_i) (I - beta_i k_i k_i^T) (per-key gate).  Every
   product is formed from scratch (O(r^2) matrix products), in the paper
   orientation S in R^{V x K}; only for tiny inputs.
2. the ungated WY recursions (§2.2.2-2.2.3 of the TileLang page, eqs. 4-5):
       w_r = beta_r (k_r - sum_{i<r} w_i (k_i^T k_r)),
       u_r = beta_r (v_r - sum_{i<r} u_i (k_i^T k_r)),
   so that P = I - W^T K and H = U^T K.
"""
from __future__ import annotations

import numpy as np

from .recurrence import as_f64


def transition(k, beta, g, per_key):
    K = k.shape[0]
    house = np.eye(K) - beta * np.outer(k, k)
    if per_key:
        return np.diag(np.exp(g)) @ house
    return np.exp(g) * house


def brute_force_forward(q, k, v, beta, g, scale, h0=None, gate="scalar"):
    """Single sequence, single head: q, k [L, K]; v [L, V]; beta [L];
    g [L] or [L, K]; h0 [K, V] (kernel orientation) or None.
    Returns (o [L, V], hL [K, V])."""
    q, k, v, beta, g = (as_f64(x) for x in (q, k, v, beta, g))
    L, K = k.shape
    V = v.shape[1]
    per_key = gate == "per_key"
    S0 = as_f64(h0).T if h0 is not None else np.zeros((V, K))
    A = [transition(k[i], beta[i], g[i], per_key) for i in range(L)]

    def prod(lo, hi):          # A_lo A_{lo+1} ... A_{hi-1}
        P = np.eye(K)
        for i in range(lo, hi):
            P = P @ A[i]
        return P

    o = np.zeros((L, V))
    S = S0
    for r in range(1, L + 1):
        P = prod(0, r)
        Hr = np.zeros((V, K))
        for i in range(r):
            Hr += beta[i] * np.outer(v[i], k[i]) @ prod(i + 1, r)
        S = S0 @ P + Hr
        o[r - 1] = S @ (scale * q[r - 1])
    return o, S.T.copy()


def wy_ungated(k, v, beta):
    """WY factors of one ungated chunk: returns (W [n,K], U [n,V], P [K,K], H [V,K]).

    P and H are the explicit products; W and U come from the recursions."""
    k, v, beta = as_f64(k), as_f64(v), as_f64(beta)
    n, K = k.shape
    V = v.shape[1]
    W = np.zeros((n, K))
    U = np.zeros((n, V))
    for r in range(n):
        w = k[r].copy()
        u = v[r].copy()
        for i in range(r):
            kk = k[i] @ k[r]
            w -= W[i] * kk
            u -= U[i] * kk
        W[r] = beta[r] * w
        U[r] = beta[r] * u
    P = np.eye(K)
    H = np.zeros((V, K))
    for r in range(n):
        Ar = np.eye(K) - beta[r] * np.outer(k[r], k[r])
        P = P @ Ar
        H = H @ Ar + beta[r] * np.outer(v[r], k[r])
    return W, U, P, H
