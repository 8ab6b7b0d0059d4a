"""TEST INFRASTRUCTURE ONLY -- the input activations of the gated delta rule in
fp64, written from the definition.

"Gated Delta Network（GDN）" §3.1, eq. 5: the decay gate is
    log alpha_t = -e^{A_log} * softplus(W_alpha x_t + b_alpha)
with A_log = log A per head and b_alpha (dt_bias) added to the projection
before the softplus, and the write strength is beta_t = sigmoid(W_beta x_t).
§5 (gate fusion) lets beta range over (0, 2) for negative eigenvalues; the
plainest reading (taken here) is beta = 2 sigmoid(.).  For the per-key gate
the same formula is applied per key channel with dt_bias per (head, channel)
and A_log per head (the pages give the per-head form only; this is the
elementwise reading).

The inputs here are the raw logits a = W_alpha x_t and b = W_beta x_t.

q and k are L2-normalised per token and head ("TileLang 实战" §1.2: with
||k_t|| = 1 the write's eigenvalues are {1 - beta_t} and 1; "Gated Delta
Network（GDN）", implementation notes: q and k are L2-normalised).  The pages
give no epsilon; the reading taken here is x / sqrt(sum x^2 + 1e-6) over the
head dimension, which is x / ||x|| up to a relative 5e-7 for unit-scale rows
and stays finite for an all-zero row.
"""
from __future__ import annotations

import numpy as np


def softplus(z):
    """log(1 + e^z), evaluated without overflow: max(z, 0) + log(1 + e^{-|z|})."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z):
    """1 / (1 + e^{-z}), evaluated without overflow for either sign."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def log_gate(a, A_log, dt_bias):
    """log alpha from raw gate logits a.

    a: [..., H] (scalar gate) or [..., H, K] (per-key gate); A_log: [H];
    dt_bias: [H] or [H, K] (broadcast against a's trailing axes)."""
    a = np.asarray(a, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    scale = np.exp(A_log)
    if a.ndim >= 2 and dt_bias.ndim == 2:   # per-key gate: [..., H, K]
        scale = scale[:, None]
    return -scale * softplus(a + dt_bias)


def beta_from_logits(b, neg_eig=False):
    """beta = sigmoid(b), or 2 sigmoid(b) in (0, 2) with neg_eig."""
    s = sigmoid(b)
    return 2.0 * s if neg_eig else s


L2_EPS = 1e-6


def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis (the head dimension)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
