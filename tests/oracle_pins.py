"""Checks that pin the fp64 oracle to facts the pages and the mathematics fix.

Each pin takes a forward function with the signature of
oracle.recurrent_forward and returns the worst relative error it sees, so
the same pin can be run on the real oracle (must be tiny) and on oracles with
a planted mistake (must be large).  Inputs are drawn here with a local numpy
generator; they are tiny.
"""
from __future__ import annotations

import numpy as np

import oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def draw(seed, B=1, T=9, H=2, K=5, V=3, per_key=False, h0=True, A=(0.2, 3.0)):
    rng = np.random.default_rng(seed)
    q = _unit(rng.standard_normal((B, T, H, K)))
    k = _unit(rng.standard_normal((B, T, H, K)))
    v = rng.standard_normal((B, T, H, V))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    a = rng.uniform(*A, size=H)
    if per_key:
        g = -a[None, None, :, None] * np.logaddexp(0, rng.standard_normal((B, T, H, K)) + 0.5)
    else:
        g = -a[None, None, :] * np.logaddexp(0, rng.standard_normal((B, T, H)) + 0.5)
    hz = rng.standard_normal((B, H, K, V)) * 0.5 if h0 else None
    return dict(q=q, k=k, v=v, beta=beta, g=g, h0=hz, gate="per_key" if per_key else "scalar")


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _call(fwd, d, scale, **kw):
    args = dict(h0=d["h0"], gate=d["gate"])
    args.update(kw)
    return fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], scale, **args)


def pin_beta1_readback(fwd, per_key=False, seed=1):
    """beta = 1 and a unit key, then a read with q = k and scale 1 returns v
    exactly, whatever the gate and the prior state ("DeltaNet 系列线性注意力
    变体的推导之旅", DeltaNet section: with beta_t = 1 the same-key query
    gives back v_t)."""
    d = draw(seed, per_key=per_key)
    d["beta"][:] = 1.0
    d["q"] = d["k"].copy()
    o, _ = _call(fwd, d, 1.0)
    return _rel(o, d["v"])


def pin_orthogonal_untouched(fwd, per_key=False, seed=2):
    """A query orthogonal to k_t sees only the forgotten old state:
    S_t q = (S_{t-1} D_t) q ("DeltaNet 系列…", locality of the rank-1 write;
    "TileLang 实战…" §1.1: memory orthogonal to k_t is left as it is)."""
    d = draw(seed, per_key=per_key, T=7)
    t = 5
    kt = d["k"][0, t]
    q = d["q"][0, t] - np.sum(d["q"][0, t] * kt, -1, keepdims=True) * kt
    d["q"][0, t] = q / np.linalg.norm(q, axis=-1, keepdims=True)
    scale = 0.7
    o, _ = _call(fwd, d, scale)
    pre = {k_: (v_[:, :t] if k_ in ("q", "k", "v", "beta", "g") else v_) for k_, v_ in d.items()}
    _, h_prev = _call(fwd, pre, scale)
    H = d["q"].shape[2]
    errs = []
    for hh in range(H):
        gt = d["g"][0, t, hh]
        dec = np.exp(gt)[:, None] if per_key else np.exp(gt)
        want = (dec * h_prev[0, hh]).T @ (scale * d["q"][0, t, hh])
        errs.append(_rel(o[0, t, hh], want))
    return max(errs)


def pin_householder_spectrum(seed=3, K=6):
    """I - beta k k^T has eigenvalue 1 - beta along a unit k and 1 on the
    K-1 orthogonal directions ("TileLang 实战…" §1.2)."""
    rng = np.random.default_rng(seed)
    k = _unit(rng.standard_normal(K))
    beta = 0.37
    ev = np.sort(np.linalg.eigvals(oracle.transition(k, beta, 0.0, False)).real)
    want = np.sort(np.array([1 - beta] + [1.0] * (K - 1)))
    return float(np.max(np.abs(ev - want)))


def pin_pure_decay(fwd, per_key=False, seed=4):
    """beta = 0 removes the delta part: h_t = exp(sum_{i<=t} g_i) h0 and
    o_t = scale h_t^T q_t ("TileLang 实战…" §2.3, the beta -> 0 limit;
    "Gated Delta Network（GDN）" §6)."""
    d = draw(seed, per_key=per_key, T=8)
    d["beta"][:] = 0.0
    scale = 0.3
    o, ht = _call(fwd, d, scale)
    G = np.cumsum(d["g"], axis=1)            # [B, T, H(, K)]
    B, T, H, K = d["q"].shape
    errs = []
    for hh in range(H):
        for t in range(T):
            dec = np.exp(G[0, t, hh])
            h = (dec[:, None] if per_key else dec) * d["h0"][0, hh]
            errs.append(_rel(o[0, t, hh], h.T @ (scale * d["q"][0, t, hh])))
        errs.append(_rel(ht[0, hh], h))
    return max(errs)


def pin_brute_force(fwd, per_key=False, seed=5, K=4, V=3, T=12):
    """The recurrence equals the explicit transition products S_r = S_0 P_r + H_r
    ("Gated Delta Network（GDN）" §4.1(a), eq. 8)."""
    d = draw(seed, per_key=per_key, T=T, K=K, V=V, H=2)
    scale = 0.8
    o, ht = _call(fwd, d, scale)
    errs = []
    for hh in range(2):
        ob, hb = oracle.brute_force_forward(d["q"][0, :, hh], d["k"][0, :, hh], d["v"][0, :, hh],
                                            d["beta"][0, :, hh], d["g"][0, :, hh], scale,
                                            h0=d["h0"][0, hh], gate=d["gate"])
        errs += [_rel(o[0, :, hh], ob), _rel(ht[0, hh], hb)]
    return max(errs)


def pin_linearity(fwd, per_key=False, seed=6):
    """For fixed (q, k, beta, g) the map (v, h0) -> (o, ht) is linear (the
    recurrence is affine in S and linear in v)."""
    d1 = draw(seed, per_key=per_key)
    d2 = draw(seed + 100, per_key=per_key)
    d2.update(q=d1["q"], k=d1["k"], beta=d1["beta"], g=d1["g"])
    a, b = 1.7, -0.6
    d3 = dict(d1)
    d3["v"] = a * d1["v"] + b * d2["v"]
    d3["h0"] = a * d1["h0"] + b * d2["h0"]
    o1, h1 = _call(fwd, d1, 0.5)
    o2, h2 = _call(fwd, d2, 0.5)
    o3, h3 = _call(fwd, d3, 0.5)
    return max(_rel(o3, a * o1 + b * o2), _rel(h3, a * h1 + b * h2))


def pin_split_resume(fwd, per_key=False, seed=7):
    """Running T1 tokens, then T2 tokens from the returned state, equals one
    run over T1 + T2 tokens (the state is the whole carry)."""
    d = draw(seed, per_key=per_key, T=11)
    o, ht = _call(fwd, d, 0.4)
    t1 = 4
    a = {k_: (v_[:, :t1] if k_ in ("q", "k", "v", "beta", "g") else v_) for k_, v_ in d.items()}
    oa, ha = _call(fwd, a, 0.4)
    b = {k_: (v_[:, t1:] if k_ in ("q", "k", "v", "beta", "g") else v_) for k_, v_ in d.items()}
    b["h0"] = ha
    ob, hb = _call(fwd, b, 0.4)
    return max(_rel(np.concatenate([oa, ob], 1), o), _rel(hb, ht))


def pin_packing(fwd, per_key=False, seed=8):
    """Packed sequences with cu_seqlens equal separate runs: the state resets
    at each sequence start ("Gated Delta Network（GDN）", terminology note:
    a chunk boundary is not a sequence boundary)."""
    lens = [5, 1, 0, 8]
    ds = [draw(seed + i, per_key=per_key, T=L, B=1) for i, L in enumerate(lens)]
    cat = {k_: np.concatenate([d[k_] for d in ds], 1) for k_ in ("q", "k", "v", "beta", "g")}
    cat["h0"] = np.concatenate([d["h0"] for d in ds], 0)
    cat["gate"] = ds[0]["gate"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o, ht = _call(fwd, cat, 0.6, cu_seqlens=cu)
    errs = []
    for i, d in enumerate(ds):
        oi, hi = _call(fwd, d, 0.6)
        errs.append(_rel(o[:, cu[i]:cu[i + 1]], oi) if lens[i] else 0.0)
        errs.append(_rel(ht[i], hi[0]))
    return max(errs)


def pin_equal_channel_gates(fwd, seed=9):
    """The per-key gate with all channels equal is the scalar gate."""
    d = draw(seed, per_key=False)
    o, ht = _call(fwd, d, 0.5)
    e = dict(d)
    e["g"] = np.repeat(d["g"][..., None], d["q"].shape[-1], axis=-1)
    e["gate"] = "per_key"
    o2, h2 = _call(fwd, e, 0.5)
    return max(_rel(o2, o), _rel(h2, ht))


def pin_value_split(fwd, per_key=False, seed=10):
    """Value columns evolve independently: running on a slice of the value
    columns (with the matching slice of h0) gives that slice of o and ht
    ("TileLang 实战…" §3.3, the kernel mirror that tiles d_v)."""
    d = draw(seed, per_key=per_key, V=6)
    o, ht = _call(fwd, d, 0.5)
    errs = []
    for sl in (slice(0, 2), slice(2, 6)):
        e = dict(d)
        e["v"] = d["v"][..., sl]
        e["h0"] = d["h0"][..., sl]
        oe, he = _call(fwd, e, 0.5)
        errs += [_rel(oe, o[..., sl]), _rel(he, ht[..., sl])]
    return max(errs)


ALL_FWD_PINS = [pin_beta1_readback, pin_orthogonal_untouched, pin_pure_decay,
                pin_brute_force, pin_linearity, pin_split_resume, pin_packing,
                pin_value_split]
