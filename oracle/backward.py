"""TEST INFRASTRUCTURE ONLY: gradients of the gated delta rule in fp64.

Two CPU references for the backward pass, described by "阅读笔记：DeltaNet 在
FLA 中的代码实现笔记" (二、反向传播): from the output gradient dO and the
final-state gradient dht, produce dq, dk, dv, dbeta, the gate gradient dg and
dh0.

recurrent_backward
    The definition.  The token recurrence (the same order as the fp64 C
    recurrence: decay, predict, residual, write, read) is written in plain
    PyTorch fp64 CPU ops and differentiated by torch.autograd, with the scalar
    loss L = <dO, O> + <dht, ht>.  Nothing chunked, nothing blocked.

chunked_backward
    The chunkwise backward in the order of the pages' six steps (recompute
    U, W; recompute the chunk entry states; the intra-chunk part of dU; the
    reverse state-gradient recurrence; dQ, dK part 1 and dW; the WY backward
    for dV, dK part 2 and dbeta), in numpy fp64.  The pages give the ungated
    DeltaNet form; the gate factors here are the chain rule through the gated
    forward of oracle.chunked (gamma, Gamma, the decayed keys K*gamma_C/gamma
    of the state update and gamma_C on the carried state), plus the gate
    gradient, which the pages do not give: dG per row of the chunk-local
    cumulative gate, then dg = reverse cumulative sum of dG inside the chunk.
    Every decay ratio is taken in the log domain (gamma_C / gamma_i as
    exp(G_C - G_i)), as the forward's Gamma is: with strong gates gamma
    itself underflows to 0.
    With the per-key-channel gate (KDA) every Gamma-weighted product becomes a
    per-channel decayed sum, (M o_E X)_id = sum_j M_ij X_jd exp(G_id - G_jd),
    the carried state gradient decays row by row, and dG is per channel.
    Both gates are pinned to recurrent_backward, which is in turn pinned by
    central finite differences of the independent C recurrence.
"""
from __future__ import annotations

import numpy as np

from .recurrence import as_f64


def _seqs(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, b, 0, T) for b in range(B)]
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    cu = np.asarray(cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                    dtype=np.int64)
    return [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def recurrent_backward(q, k, v, beta, g, scale, do, h0=None, dht=None, cu_seqlens=None,
                       gate="scalar"):
    """Gradients of L = <do, o> + <dht, ht> through the fp64 token recurrence.

    Shapes as oracle.recurrent_forward; do [B, T, H, V]; dht [N, H, K, V] or
    None (no final-state gradient).  Returns a dict with dq, dk [B,T,H,K],
    dv [B,T,H,V], dbeta [B,T,H], dg (shape of g) and dh0 [N,H,K,V] as fp64
    numpy arrays, plus o and ht of the same pass.  dh0 is the gradient with
    respect to the initial state (zeros when h0 is None: still defined).
    """
    import torch

    t64 = lambda x: torch.from_numpy(as_f64(x).copy())  # noqa: E731
    q, k, v, beta, g, do = (t64(x) for x in (q, k, v, beta, g, do))
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = gate == "per_key"
    seqs = _seqs(B, T, cu_seqlens)
    N = len(seqs)
    h0 = t64(h0) if h0 is not None else torch.zeros(N, H, K, V, dtype=torch.float64)
    dht = t64(dht) if dht is not None else None
    leaves = (q, k, v, beta, g, h0)
    for x in leaves:
        x.requires_grad_(True)
    o = torch.zeros(B, T, H, V, dtype=torch.float64)
    ht = torch.zeros(N, H, K, V, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    with torch.enable_grad():
        for n, b, s0, s1 in seqs:
            S = h0[n]                                          # [H, K, V]
            for t in range(s0, s1):
                a = torch.exp(g[b, t])                         # [H] or [H, K]
                S = S * (a[:, :, None] if per_key else a[:, None, None])    # decay
                p = torch.einsum("hkv,hk->hv", S, k[b, t])                  # predict
                r = beta[b, t][:, None] * (v[b, t] - p)                     # residual
                S = S + k[b, t][:, :, None] * r[:, None, :]                 # write
                ot = torch.einsum("hkv,hk->hv", S, scale * q[b, t])         # read
                loss = loss + (ot * do[b, t]).sum()
                o[b, t] = ot.detach()
            if dht is not None:
                loss = loss + (S * dht[n]).sum()
            ht[n] = S.detach()
        grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    out = {}
    for name, x, gr in zip(("dq", "dk", "dv", "dbeta", "dg", "dh0"), leaves, grads):
        out[name] = (gr if gr is not None else torch.zeros_like(x)).numpy()
    out["o"] = o.numpy()
    out["ht"] = ht.numpy()
    return out


def _chunk_fwd(Qc, Kc, Vc, bc, gc, h, scale):
    """Forward of one chunk (scalar gate), keeping what the backward needs."""
    n = Kc.shape[0]
    G = np.cumsum(gc)
    incl = np.tril(np.ones((n, n), dtype=bool))
    D = G[:, None] - G[None, :]
    Gam = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
    gam = np.exp(G)
    end = gam[-1]
    rest = np.exp(G[-1] - G)          # gamma_C / gamma_i in the log domain (no 0/0)
    KK = Kc @ Kc.T
    A = np.tril(bc[:, None] * Gam * KK, -1)
    Ainv = np.linalg.inv(np.eye(n) + A)
    Aqk = scale * Gam * (Qc @ Kc.T)
    W = Ainv @ ((bc * gam)[:, None] * Kc)
    U = Ainv @ (bc[:, None] * Vc)
    Vnew = U - W @ h
    Ks = rest[:, None] * Kc
    return dict(G=G, Gam=Gam, gam=gam, end=end, rest=rest, KK=KK, A=A, Ainv=Ainv, Aqk=Aqk, W=W, U=U,
                Vnew=Vnew, Ks=Ks, h_in=h, h_out=end * h + Ks.T @ Vnew)


def _chunk_bwd(Qc, Kc, Vc, bc, f, dOc, dH, scale):
    """Backward of one chunk.  dH is the gradient of the state leaving the
    chunk; returns (dq, dk, dv, dbeta, dg, dH entering, dVnew)."""
    G, Gam, gam, end = f["G"], f["Gam"], f["gam"], f["end"]
    h, Ainv, Aqk, W, Vnew, Ks, A = f["h_in"], f["Ainv"], f["Aqk"], f["W"], f["Vnew"], f["Ks"], f["A"]
    n = Kc.shape[0]
    incl = np.tril(np.ones((n, n), dtype=bool))
    # Step 3: the part of dU (= dV_new) that comes from this chunk's outputs.
    dVnew = Aqk.T @ dOc
    # Step 4: add the part through the state leaving the chunk, then carry the
    # state gradient to the chunk's entry.
    dVnew = dVnew + Ks @ dH
    Qs = scale * gam[:, None] * Qc
    dH_in = end * dH + Qs.T @ dOc - W.T @ dVnew
    # Step 5: dQ, dK part 1, dW.
    dAqk = np.where(incl, dOc @ Vnew.T, 0.0)
    dQ_inter = scale * gam[:, None] * (dOc @ h.T)
    dQ = dQ_inter + scale * (dAqk * Gam) @ Kc
    dKs = Vnew @ dH.T                                     # gradient of K*gamma_C/gamma
    dK = f["rest"][:, None] * dKs + scale * (dAqk * Gam).T @ Qc
    dW = -dVnew @ h.T
    # Step 6: WY backward.  W = Ainv diag(beta gamma) K, U = Ainv diag(beta) V.
    AtdW = Ainv.T @ dW
    AtdU = Ainv.T @ dVnew
    dV = bc[:, None] * AtdU
    dAinv = dVnew @ (bc[:, None] * Vc).T + dW @ ((bc * gam)[:, None] * Kc).T
    dA = np.tril(-Ainv.T @ dAinv @ Ainv.T, -1)
    dAG = dA * Gam
    dK = dK + (bc * gam)[:, None] * AtdW + dAG.T @ (bc[:, None] * Kc) + bc[:, None] * (dAG @ Kc)
    dbeta = (np.sum(AtdU * Vc, axis=1) + np.sum(AtdW * (gam[:, None] * Kc), axis=1)
             + np.sum(dAG * f["KK"], axis=1))
    # Gate: gradient of the chunk-local cumulative gate G, row by row.
    P = dAqk * Aqk
    R = dA * A
    s = np.sum(Ks * dKs, axis=1)
    dG = (np.sum(Qc * dQ_inter, axis=1)
          + P.sum(axis=1) - P.sum(axis=0)
          + R.sum(axis=1) - R.sum(axis=0)
          + np.sum(AtdW * ((bc * gam)[:, None] * Kc), axis=1)
          - s)
    dG[-1] += end * np.sum(dH * h) + s.sum()
    dg = np.cumsum(dG[::-1])[::-1]
    return dQ, dK, dV, dbeta, dg, dH_in, dVnew


def _chunk_fwd_pk(Qc, Kc, Vc, bc, gc, h, scale):
    """Forward of one chunk with the per-key-channel gate (gc [n, K]): every
    decay ratio E[i, j, d] = exp(G_id - G_jd) (j <= i) sits inside the sum over
    the key channel d ("DeltaNet 系列线性注意力变体的推导之旅", chunkwise KDA),
    taken in the log domain and masked before the exponential."""
    n = Kc.shape[0]
    G = np.cumsum(gc, axis=0)                                 # [n, K]
    incl = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
    D = G[:, None, :] - G[None, :, :]                          # [n, n, K]
    E = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
    gam = np.exp(G)
    end = gam[-1]                                             # [K]
    rest = np.exp(G[-1][None, :] - G)
    A = np.tril(bc[:, None] * np.einsum("id,jd,ijd->ij", Kc, Kc, E), -1)
    Ainv = np.linalg.inv(np.eye(n) + A)
    Aqk = scale * np.einsum("id,jd,ijd->ij", Qc, Kc, E)
    Kg = gam * Kc
    Y_of = lambda hh: Vc - Kg @ hh                            # noqa: E731
    Vnew = Ainv @ (bc[:, None] * Y_of(h))
    Ks = rest * Kc
    return dict(G=G, E=E, gam=gam, end=end, rest=rest, A=A, Ainv=Ainv, Aqk=Aqk, Kg=Kg,
                Y=Y_of(h), Vnew=Vnew, Ks=Ks, h_in=h, h_out=end[:, None] * h + Ks.T @ Vnew)


def _chunk_bwd_pk(Qc, Kc, Vc, bc, f, dOc, dH, scale):
    """Backward of one chunk with the per-key-channel gate; the same steps as
    _chunk_bwd with each Gamma-weighted product taken per channel:
    (M o_E X)_id = sum_j M_ij X_jd E_ijd.  Returns (dq, dk, dv, dbeta, dg,
    dH entering, dVnew)."""
    E, gam, end, rest = f["E"], f["gam"], f["end"], f["rest"]
    h, Ainv, Aqk, Kg, Y, Vnew, Ks = (f[x] for x in ("h_in", "Ainv", "Aqk", "Kg", "Y", "Vnew", "Ks"))
    n = Kc.shape[0]
    incl = np.tril(np.ones((n, n), dtype=bool))
    W = Ainv @ (bc[:, None] * Kg)
    # the reverse recurrence (Steps 3-4): the carried gradient decays by row
    dVnew = Aqk.T @ dOc + Ks @ dH
    Qs = scale * gam * Qc
    dH_in = end[:, None] * dH + Qs.T @ dOc - W.T @ dVnew
    # Step 5: the output's products and the state update's decayed keys
    dAqk = np.where(incl, dOc @ Vnew.T, 0.0)
    dQs = dOc @ h.T
    Pq = scale * np.einsum("ij,jd,ijd->id", dAqk, Kc, E)
    Pk = scale * np.einsum("ij,id,ijd->jd", dAqk, Qc, E)
    dKs = Vnew @ dH.T
    # Step 6: V_new = Ainv diag(beta) Y with Y = V - (K * gamma) h
    AtdU = Ainv.T @ dVnew
    dY = bc[:, None] * AtdU
    dKg = -dY @ h.T
    dA = np.tril(-Ainv.T @ (dVnew @ (bc[:, None] * Y).T) @ Ainv.T, -1)
    Pa1 = np.einsum("ij,jd,ijd->id", dA, Kc, E)
    Pa2 = np.einsum("ij,i,id,ijd->jd", dA, bc, Kc, E)
    dQ = scale * gam * dQs + Pq
    dK = rest * dKs + gam * dKg + Pk + bc[:, None] * Pa1 + Pa2
    dV = dY
    dbeta = np.sum(AtdU * Y, axis=1) + np.sum(Kc * Pa1, axis=1)
    # the gate: every place G_id enters, then the reverse cumulative sum
    dG = (Qs * dQs + Qc * Pq - Kc * Pk - Ks * dKs + Kg * dKg
          + bc[:, None] * Kc * Pa1 - Kc * Pa2)
    dG[-1] += end * np.sum(h * dH, axis=1) + np.sum(Ks * dKs, axis=0)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dQ, dK, dV, dbeta, dg, dH_in, dVnew


def chunked_backward(q, k, v, beta, g, scale, do, h0=None, dht=None, cu_seqlens=None,
                     chunk=64, keep=False, gate="scalar"):
    """Chunkwise backward, fp64.  Arguments as recurrent_backward plus the
    chunk length.  Returns the same dict (without o, ht); with keep=True also
    'dH_out' and 'h_in': dicts (seq, head, chunk) -> the state gradient
    leaving / the state entering that chunk, and 'dVnew' [B,T,H,V]."""
    fwd, bwd = (_chunk_fwd_pk, _chunk_bwd_pk) if gate == "per_key" else (_chunk_fwd, _chunk_bwd)
    q, k, v, beta, g, do = (as_f64(x) for x in (q, k, v, beta, g, do))
    B, T, H, K = q.shape
    V = v.shape[-1]
    seqs = _seqs(B, T, cu_seqlens)
    N = len(seqs)
    h0 = as_f64(h0) if h0 is not None else np.zeros((N, H, K, V))
    dht = as_f64(dht) if dht is not None else np.zeros((N, H, K, V))
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dbeta=np.zeros_like(beta), dg=np.zeros_like(g), dh0=np.zeros((N, H, K, V)))
    if keep:
        out.update(dH_out={}, h_in={}, dVnew=np.zeros_like(v))
    for n, b, s0, s1 in seqs:
        for hh in range(H):
            # Steps 1-2: recompute every chunk's forward and entry state.
            h = h0[n, hh].copy()
            fw = []
            for c0 in range(s0, s1, chunk):
                sl = slice(c0, min(c0 + chunk, s1))
                f = fwd(q[b, sl, hh], k[b, sl, hh], v[b, sl, hh], beta[b, sl, hh],
                        g[b, sl, hh], h, scale)
                fw.append((sl, f))
                h = f["h_out"]
            # Steps 3-6, last chunk first.
            dH = dht[n, hh].copy()
            for ci in range(len(fw) - 1, -1, -1):
                sl, f = fw[ci]
                if keep:
                    out["dH_out"][(n, hh, ci)] = dH.copy()
                    out["h_in"][(n, hh, ci)] = f["h_in"].copy()
                dQ, dK, dV, dbt, dg, dH, dVn = bwd(
                    q[b, sl, hh], k[b, sl, hh], v[b, sl, hh], beta[b, sl, hh], f,
                    do[b, sl, hh], dH, scale)
                out["dq"][b, sl, hh] = dQ
                out["dk"][b, sl, hh] = dK
                out["dv"][b, sl, hh] = dV
                out["dbeta"][b, sl, hh] = dbt
                out["dg"][b, sl, hh] = dg
                if keep:
                    out["dVnew"][b, sl, hh] = dVn
            out["dh0"][n, hh] = dH
    return out


def activation_backward(a, b, A_log, dt_bias, dg, dbeta, neg_eig=False):
    """Chain rule through the input activation, fp64.

    a, b [B, T, H]: the raw gate and beta logits (a [B, T, H, K] for the
    per-key gate); A_log [H]; dt_bias [H] ([H, K] per-key); dg (the shape of
    a), dbeta [B, T, H]: the gradients with respect to log alpha and beta (as
    the backward produces them).  With log alpha = -e^{A_log} softplus(a +
    dt_bias) and beta = sigmoid(b) (2 sigmoid(b) with neg_eig)
    ("Gated Delta Network（GDN）" §3.1 eq. 5, §5; per channel for the
    per-key gate):
      d/da       = dg * (-e^{A_log} sigmoid(a + dt_bias))   (softplus' = sigmoid)
      d/db       = dbeta * s (1 - s) (times 2 with neg_eig),  s = sigmoid(b)
      d/dA_log   = sum over tokens (and channels) of dg * log alpha
                   (d log alpha / d A_log = log alpha)
      d/ddt_bias = sum over tokens of d/da
    Returns (da, db, dA_log [H], ddt_bias (the shape of dt_bias))."""
    from .activation import log_gate, sigmoid
    a, b, A_log, dt_bias, dg, dbeta = (as_f64(x) for x in (a, b, A_log, dt_bias, dg, dbeta))
    per_key = dt_bias.ndim == 2
    el = np.exp(A_log)[:, None] if per_key else np.exp(A_log)
    da = dg * (-el * sigmoid(a + dt_bias))
    s = sigmoid(b)
    db = dbeta * s * (1.0 - s) * (2.0 if neg_eig else 1.0)
    lg = log_gate(a, A_log, dt_bias)
    tok = tuple(range(dg.ndim - (2 if per_key else 1)))
    dA_log = np.sum(dg * lg, axis=tok)
    if per_key:
        dA_log = np.sum(dA_log, axis=-1)
    ddt_bias = np.sum(da, axis=tok)
    return da, db, dA_log, ddt_bias


def l2_normalize_backward(x, dy, eps=None):
    """Gradient with respect to x of <dy, l2_normalize(x)>: with n2 = sum x^2
    + eps over the head dimension, y = x / sqrt(n2) has the symmetric Jacobian
    (I - x x^T / n2) / sqrt(n2), so dx = (dy - x (x . dy) / n2) / sqrt(n2)."""
    from .activation import L2_EPS
    eps = L2_EPS if eps is None else eps
    x, dy = as_f64(x), as_f64(dy)
    n2 = np.sum(x * x, axis=-1, keepdims=True) + eps
    return (dy - x * (np.sum(x * dy, axis=-1, keepdims=True) / n2)) / np.sqrt(n2)
