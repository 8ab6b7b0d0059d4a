"""TEST INFRASTRUCTURE ONLY: the chunked UT-form forward pass in fp64 (numpy).

This is the second, independent CPU reference.  It follows the chunkwise
algorithm of "TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.2.4 (UT
transform, eqs. 6-7), §2.2.6 (the gated substitutions) and §2.3 (eqs. 11-12),
in the orientation of its §3.0 (state stored as h = S^T, [K, V]), and the
five forward steps of "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记" (一、前向,
Steps 1-5) with the gates added.  Per chunk of n <= C tokens and entry state h:

  G      = inclusive cumulative sum of the log-gates inside the chunk
  Gamma  = exp(G_i - G_j) for j <= i, else 0   (masked before the exponent)
  A      = strictLower( diag(beta) (Gamma * K K^T) )          (Step 1)
  Ainv   = (I + A)^{-1}                                        (Step 2)
  W      = Ainv diag(beta) diag(gamma) K ,  U = Ainv diag(beta) V   (Step 3)
  V_new  = U - W h                                             (Step 4)
  O      = (scale Q * gamma) h + (scale Q K^T * Gamma) V_new   (Step 5)
  h     <- gamma_C h + (K * gamma_C / gamma)^T V_new           (Step 4)

with gamma_r = exp(G_r).  The pages' own UT matrix T equals Ainv diag(beta).
For the per-key-channel gate (Kimi Delta Attention, "DeltaNet 系列线性注意力
变体的推导之旅", chunkwise section) every Gamma-weighted inner product carries
exp(G_i[d] - G_j[d]) inside the sum over d, gamma becomes a K-vector applied
per key column of K and Q, and the state decays row-wise by exp(G_C).

The triangular inverse is numpy.linalg.inv (a library primitive); nothing is
blocked or fused beyond what is written above.
"""
from __future__ import annotations

import numpy as np

from .recurrence import as_f64


def _chunk(Qc, Kc, Vc, bc, gc, h, scale, per_key):
    n = Kc.shape[0]
    G = np.cumsum(gc, axis=0)
    incl = np.tril(np.ones((n, n), dtype=bool))
    if per_key:
        D = G[:, None, :] - G[None, :, :]
        E = np.where(incl[:, :, None], np.exp(np.where(incl[:, :, None], D, 0.0)), 0.0)
        KKg = np.einsum("id,jd,ijd->ij", Kc, Kc, E)
        QKg = np.einsum("id,jd,ijd->ij", Qc, Kc, E)
        gam = np.exp(G)                      # [n, K]
        Kw = (bc[:, None] * gam) * Kc
        Ks = np.exp(G[-1][None, :] - G) * Kc
        Qs = scale * gam * Qc
        end = np.exp(G[-1])[:, None]         # row-wise decay of h
    else:
        D = G[:, None] - G[None, :]
        Gam = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
        KKg = Gam * (Kc @ Kc.T)
        QKg = Gam * (Qc @ Kc.T)
        gam = np.exp(G)                      # [n]
        Kw = (bc * gam)[:, None] * Kc
        Ks = np.exp(G[-1] - G)[:, None] * Kc
        Qs = scale * gam[:, None] * Qc
        end = np.exp(G[-1])
    A = np.tril(bc[:, None] * KKg, -1)
    Ainv = np.linalg.inv(np.eye(n) + A)
    Aqk = scale * QKg
    W = Ainv @ Kw
    U = Ainv @ (bc[:, None] * Vc)
    Vnew = U - W @ h
    O = Qs @ h + Aqk @ Vnew
    h_next = end * h + Ks.T @ Vnew
    return dict(G=G, A=A, Ainv=Ainv, Aqk=Aqk, W=W, U=U, Vnew=Vnew, O=O, h_in=h,
                h_out=h_next)


def chunked_forward(q, k, v, beta, g, scale, h0=None, cu_seqlens=None,
                    gate="scalar", chunk=64, keep=False):
    """Chunked UT-form forward in fp64.

    Same arguments and layouts as oracle.recurrence.recurrent_forward, plus
    the chunk length.  Chunks restart at every sequence start, the last chunk
    of a sequence is ragged.  Returns (o, ht) or, with keep=True,
    (o, ht, inter) where inter holds token-indexed intermediates:
      G [B,T,H] or [B,T,H,K] (natural-log cumulative gate in its chunk),
      Ainv, A, Aqk [B,T,H,C] (row of the chunk matrix; columns >= n are 0),
      W [B,T,H,K], U, Vnew [B,T,H,V], and h_chunk: dict (seq, head, chunk)
      -> entry state [K, V].
    """
    q, k, v, beta, g = (as_f64(x) for x in (q, k, v, beta, g))
    h0 = as_f64(h0)
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = gate == "per_key"
    if cu_seqlens is None:
        seqs = [(b, b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens)
        seqs = [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(seqs)
    o = np.zeros((B, T, H, V))
    ht = np.zeros((N, H, K, V))
    if keep:
        C = chunk
        inter = dict(G=np.zeros(g.shape), A=np.zeros((B, T, H, C)),
                     Ainv=np.zeros((B, T, H, C)), Aqk=np.zeros((B, T, H, C)),
                     W=np.zeros((B, T, H, K)), U=np.zeros((B, T, H, V)),
                     Vnew=np.zeros((B, T, H, V)), h_chunk={})
    for n, b, s0, s1 in seqs:
        for hh in range(H):
            h = h0[n, hh].copy() if h0 is not None else np.zeros((K, V))
            for ci, c0 in enumerate(range(s0, s1, chunk)):
                c1 = min(c0 + chunk, s1)
                sl = slice(c0, c1)
                r = _chunk(q[b, sl, hh], k[b, sl, hh], v[b, sl, hh], beta[b, sl, hh],
                           g[b, sl, hh], h, scale, per_key)
                o[b, sl, hh] = r["O"]
                if keep:
                    m = c1 - c0
                    inter["G"][b, sl, hh] = r["G"]
                    inter["A"][b, sl, hh, :m] = r["A"]
                    inter["Ainv"][b, sl, hh, :m] = r["Ainv"]
                    inter["Aqk"][b, sl, hh, :m] = r["Aqk"]
                    inter["W"][b, sl, hh] = r["W"]
                    inter["U"][b, sl, hh] = r["U"]
                    inter["Vnew"][b, sl, hh] = r["Vnew"]
                    inter["h_chunk"][(n, hh, ci)] = h.copy()
                h = r["h_out"]
            ht[n, hh] = h
    if keep:
        return o, ht, inter
    return o, ht
