"""Pins of the fp64 backward oracle (CPU only).

The autograd oracle (oracle.backward.recurrent_backward) is pinned to
things outside itself:
  * central finite differences of the loss L = <dO, O> + <dht, ht> computed
    with the C token recurrence (oracle.recurrent_forward, separate code), for
    every input element of tiny problems: both gate kinds, packed sequences
    with an empty one, beta in (0, 2);
  * closed forms at beta = 0, where the recurrence is pure decay and the
    gradients of k and v vanish; dbeta at beta = 0 is the first-order effect
    of one write, derived by hand below.
The chunked backward (the pages' six steps with the gate terms) is then
pinned to the autograd oracle to 1e-10 at several chunk lengths, for the
scalar gate and for the per-key-channel gate (whose chunked form decays
every product channel by channel).
"""
import numpy as np
import pytest

import oracle
from oracle.backward import chunked_backward, recurrent_backward
from oracle_pins import draw

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def _extras(seed, d, N):
    rng = np.random.default_rng(seed + 1000)
    B, T, H, _ = d["q"].shape
    V = d["v"].shape[-1]
    K = d["q"].shape[-1]
    return rng.standard_normal((B, T, H, V)), rng.standard_normal((N, H, K, V))


def _loss(d, do, dht, scale, cu=None):
    o, ht = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], scale,
                                     h0=d["h0"], gate=d["gate"], cu_seqlens=cu)
    return float(np.sum(o * do) + np.sum(ht * dht))


def _fd_check(d, do, dht, scale, cu=None, eps=1e-6):
    """Worst relative error of every gradient element against central
    differences of the C recurrence."""
    got = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], scale, do,
                             h0=d["h0"], dht=dht, cu_seqlens=cu, gate=d["gate"])
    worst = 0.0
    for name, key in zip(NAMES, ("q", "k", "v", "beta", "g", "h0")):
        x = d[key]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(d, do, dht, scale, cu)
            x[idx] = keep - eps
            lm = _loss(d, do, dht, scale, cu)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        scale_ref = max(np.max(np.abs(fd)), 1e-12)
        worst = max(worst, float(np.max(np.abs(got[name] - fd)) / scale_ref))
    return worst


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_autograd_matches_finite_differences(per_key):
    d = draw(21, B=2, T=5, H=2, K=4, V=3, per_key=per_key)
    do, dht = _extras(21, d, 2)
    assert _fd_check(d, do, dht, 0.7) < 1e-7


def test_finite_differences_packed_and_wide_beta():
    """Packed sequences (one empty), beta in (0, 2) (negative eigenvalues of
    the transition), no final-state gradient on one call."""
    d = draw(22, B=1, T=9, H=2, K=3, V=2)
    rng = np.random.default_rng(5)
    d["beta"] = rng.uniform(0.05, 1.95, size=d["beta"].shape)
    cu = np.array([0, 4, 4, 9])
    d["h0"] = rng.standard_normal((3, 2, 3, 2)) * 0.5
    do, dht = _extras(22, d, 3)
    assert _fd_check(d, do, dht, 0.5, cu=cu) < 1e-7
    assert _fd_check(d, do, np.zeros_like(dht), 0.5, cu=cu) < 1e-7


def test_zero_beta_closed_forms():
    """beta = 0: S_t = exp(G_t) h0 with G the running sum of g.  Then
    dk = dv = 0, dq_t = scale exp(G_t) h0 do_t, dh0 = sum_t scale exp(G_t)
    q_t do_t^T + exp(G_T) dht, dg_s = sum_{t>=s} scale exp(G_t) q_t^T h0 do_t
    + exp(G_T) <dht, h0>, and dbeta_t (the first-order effect of the write
    k_t (v_t - exp(G_t) h0^T k_t)^T made at t, decayed by exp(G_u - G_t) to
    each later read and to the final state)."""
    d = draw(23, B=1, T=7, H=1, K=4, V=3)
    d["beta"][:] = 0.0
    do, dht = _extras(23, d, 1)
    scale = 0.9
    got = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], scale, do,
                             h0=d["h0"], dht=dht)
    q, k, v, g = d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0], d["g"][0, :, 0]
    h0, dO, dH = d["h0"][0, 0], do[0, :, 0], dht[0, 0]
    T = q.shape[0]
    G = np.cumsum(g)
    dq = np.stack([scale * np.exp(G[t]) * h0 @ dO[t] for t in range(T)])
    dh0 = sum(scale * np.exp(G[t]) * np.outer(q[t], dO[t]) for t in range(T)) + np.exp(G[-1]) * dH
    contrib = np.array([scale * np.exp(G[t]) * q[t] @ h0 @ dO[t] for t in range(T)])
    dg = np.array([contrib[s:].sum() for s in range(T)]) + np.exp(G[-1]) * np.sum(dH * h0)
    dbeta = np.zeros(T)
    for t in range(T):
        r = v[t] - np.exp(G[t]) * h0.T @ k[t]
        dbeta[t] = sum(scale * np.exp(G[u] - G[t]) * (q[u] @ k[t]) * (r @ dO[u])
                       for u in range(t, T)) + np.exp(G[-1] - G[t]) * (k[t] @ dH @ r)
    assert np.max(np.abs(got["dk"])) == 0.0
    assert np.max(np.abs(got["dv"])) == 0.0
    for name, ref in (("dq", dq), ("dh0", dh0), ("dg", dg), ("dbeta", dbeta)):
        x = got[name].reshape(ref.shape)
        assert np.max(np.abs(x - ref)) <= 1e-13 * np.max(np.abs(ref)), name


def test_forward_values_match_c_recurrence():
    """The autograd pass computes the same o and ht as the C recurrence."""
    d = draw(24, B=2, T=11, H=2, K=5, V=4)
    do, dht = _extras(24, d, 2)
    got = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.6, do,
                             h0=d["h0"], dht=dht)
    o, ht = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.6,
                                     h0=d["h0"])
    assert np.max(np.abs(got["o"] - o)) < 1e-13
    assert np.max(np.abs(got["ht"] - ht)) < 1e-13


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 150])
def test_chunked_backward_matches_autograd(chunk, T, per_key):
    d = draw(30 + T, B=2, T=T, H=2, K=8, V=6, A=(0.5, 8.0), per_key=per_key)
    do, dht = _extras(30 + T, d, 2)
    ref = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.35, do,
                             h0=d["h0"], dht=dht, gate=d["gate"])
    got = chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.35, do,
                           h0=d["h0"], dht=dht, chunk=chunk, gate=d["gate"])
    for name in NAMES:
        assert _rel(got[name], ref[name]) < 1e-10, name


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_chunked_backward_strong_decay(per_key):
    """The pages' strongest gates (A up to 16): gamma underflows to 0 inside
    a 64-token chunk, and the chunked backward still matches (no 0/0)."""
    d = draw(45, B=1, T=150, H=2, K=8, V=6, A=(8.0, 16.0), per_key=per_key)
    do, dht = _extras(45, d, 1)
    ref = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.35, do,
                             h0=d["h0"], dht=dht, gate=d["gate"])
    with np.errstate(divide="raise", invalid="raise", under="ignore"):
        got = chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.35, do,
                               h0=d["h0"], dht=dht, chunk=64, gate=d["gate"])
    # the case is the underflowing one
    assert np.any(np.exp(np.cumsum(d["g"][0, :64, 0], axis=0))[-1] == 0.0)
    for name in NAMES:
        assert _rel(got[name], ref[name]) < 1e-10, name


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_chunked_backward_packed_wide_beta(per_key):
    d = draw(40, B=1, T=90, H=2, K=6, V=5, per_key=per_key)
    rng = np.random.default_rng(40)
    d["beta"] = rng.uniform(0.05, 1.95, size=d["beta"].shape)
    cu = np.array([0, 17, 17, 70, 90])
    d["h0"] = rng.standard_normal((4, 2, 6, 5)) * 0.3
    do, dht = _extras(40, d, 4)
    ref = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.4, do,
                             h0=d["h0"], dht=dht, cu_seqlens=cu, gate=d["gate"])
    got = chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.4, do,
                           h0=d["h0"], dht=dht, cu_seqlens=cu, chunk=16, gate=d["gate"])
    for name in NAMES:
        assert _rel(got[name], ref[name]) < 1e-10, name


@pytest.mark.parametrize("drop", ["wy_a_term", "gate_state_term", "state_carry"])
def test_chunked_backward_mutations_fail(drop, monkeypatch):
    """A plausible slip in the chunked backward (a dropped WY term, the
    gamma_C factor on the carried state gradient, the last-row gate term)
    breaks the match with the autograd oracle."""
    import oracle.backward as ob
    real = ob._chunk_bwd

    def planted(Qc, Kc, Vc, bc, f, dOc, dH, scale):
        dQ, dK, dV, dbt, dg, dH_in, dVn = real(Qc, Kc, Vc, bc, f, dOc, dH, scale)
        if drop == "wy_a_term":
            dAinv = dVn @ (bc[:, None] * Vc).T - (dVn @ f["h_in"].T) @ ((bc * f["gam"])[:, None] * Kc).T
            dA = np.tril(-f["Ainv"].T @ dAinv @ f["Ainv"].T, -1)
            dK = dK - bc[:, None] * ((dA * f["Gam"]) @ Kc)
        elif drop == "gate_state_term":
            dg = dg - f["end"] * np.sum(dH * f["h_in"])
        else:
            dH_in = dH_in - f["end"] * dH + dH
        return dQ, dK, dV, dbt, dg, dH_in, dVn

    monkeypatch.setattr(ob, "_chunk_bwd", planted)
    d = draw(50, B=1, T=40, H=1, K=6, V=5, A=(0.02, 0.1))
    do, dht = _extras(50, d, 1)
    ref = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.5, do,
                             h0=d["h0"], dht=dht)
    got = ob.chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.5, do,
                              h0=d["h0"], dht=dht, chunk=8)
    assert max(_rel(got[n], ref[n]) for n in NAMES) > 1e-4


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("neg_eig", [False, True])
def test_activation_backward_matches_finite_differences(neg_eig, per_key):
    """The activation's chain rule against central differences of
    L = <dg, log_gate(a, A_log, dt_bias)> + <dbeta, beta_from_logits(b)>
    through oracle.activation (every element of a, b, A_log, dt_bias); the
    per-key gate has a and dt_bias per channel and A_log per head."""
    from oracle import activation as act
    from oracle.backward import activation_backward
    rng = np.random.default_rng(90)
    B, T, H, K = 2, 5, 3, 4
    ga = (B, T, H, K) if per_key else (B, T, H)
    a, b = rng.standard_normal(ga) * 2, rng.standard_normal((B, T, H)) * 2
    A_log = np.log(rng.uniform(0.5, 16, H))
    dt_bias = rng.standard_normal((H, K) if per_key else H)
    dg, dbeta = rng.standard_normal(ga), rng.standard_normal((B, T, H))

    def loss(a_, b_, A_, d_):
        return float(np.sum(dg * act.log_gate(a_, A_, d_)) +
                     np.sum(dbeta * act.beta_from_logits(b_, neg_eig)))
    got = activation_backward(a, b, A_log, dt_bias, dg, dbeta, neg_eig)
    args = [a, b, A_log, dt_bias]
    eps = 1e-6
    for which in range(4):
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss(*args)
            x[idx] = keep - eps
            lm = loss(*args)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(got[which] - fd)) <= 1e-7 * max(np.max(np.abs(fd)), 1.0), which


def test_l2_normalize_backward_matches_finite_differences():
    """The L2 normalisation's chain rule against central differences of
    <dy, l2_normalize(x)> (every element), and for eps = 0 the gradient is
    orthogonal to x (the normalised output does not change along x)."""
    from oracle import activation as act
    from oracle.backward import l2_normalize_backward
    rng = np.random.default_rng(96)
    x = rng.standard_normal((2, 3, 2, 8)) * 0.7
    x[0, 0, 0] *= 1e-2    # a short row, where the epsilon matters more
    dy = rng.standard_normal(x.shape)
    got = l2_normalize_backward(x, dy)
    fd = np.zeros_like(x)
    h = 1e-7
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + h
        lp = float(np.sum(dy * act.l2_normalize(x)))
        x[idx] = keep - h
        lm = float(np.sum(dy * act.l2_normalize(x)))
        x[idx] = keep
        fd[idx] = (lp - lm) / (2 * h)
    assert np.max(np.abs(got - fd)) <= 1e-6 * max(np.max(np.abs(fd)), 1.0)
    g0 = l2_normalize_backward(x, dy, eps=0.0)
    assert np.max(np.abs(np.sum(g0 * x, axis=-1))) <= 1e-12


@pytest.mark.parametrize("drop", ["row_decay", "gate_state_term"])
def test_chunked_backward_per_key_mutations_fail(drop, monkeypatch):
    """With the per-key gate, carrying the state gradient back with one mean
    decay instead of row by row, or dropping the per-channel state term of
    the last row's gate gradient, breaks the match with the autograd oracle."""
    import oracle.backward as ob
    real = ob._chunk_bwd_pk

    def planted(Qc, Kc, Vc, bc, f, dOc, dH, scale):
        dQ, dK, dV, dbt, dg, dH_in, dVn = real(Qc, Kc, Vc, bc, f, dOc, dH, scale)
        if drop == "row_decay":
            dH_in = dH_in - f["end"][:, None] * dH + np.mean(f["end"]) * dH
        else:
            dg = dg - (f["end"] * np.sum(f["h_in"] * dH, axis=1))[None, :]
        return dQ, dK, dV, dbt, dg, dH_in, dVn

    monkeypatch.setattr(ob, "_chunk_bwd_pk", planted)
    d = draw(51, B=1, T=40, H=1, K=6, V=5, A=(0.02, 0.3), per_key=True)
    do, dht = _extras(51, d, 1)
    ref = recurrent_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.5, do,
                             h0=d["h0"], dht=dht, gate="per_key")
    got = ob.chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.5, do,
                              h0=d["h0"], dht=dht, chunk=8, gate="per_key")
    assert max(_rel(got[n], ref[n]) for n in NAMES) > 1e-4
