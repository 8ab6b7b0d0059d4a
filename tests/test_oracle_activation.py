"""Pins of the input activations ("Gated Delta Network（GDN）" §3.1 eq. 5: the
gate log alpha = -e^{A_log} softplus(a + dt_bias), beta = sigmoid(b)) and of
the recurrence with beta in (0, 2) (§5: negative eigenvalues), on the fp64
oracle.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import activation as act
from oracle_pins import _unit, draw

TOL = 1e-12


def test_activation_closed_forms():
    # softplus(0) = ln 2, sigmoid(0) = 1/2
    assert abs(act.softplus(0.0) - np.log(2.0)) < 1e-16
    assert act.sigmoid(0.0) == 0.5
    # far right: log(1 + e^z) = z + log(1 + e^{-z}), and log(1 + x) = x - x^2/2 + ...
    z = np.array([40.0, 200.0, 700.0])
    np.testing.assert_allclose(act.softplus(z), z + np.exp(-z), rtol=1e-15, atol=0)
    # far left: log(1 + e^z) = e^z (1 - e^z / 2 + ...)
    z = np.array([-40.0, -200.0, -700.0])
    np.testing.assert_allclose(act.softplus(z), np.exp(z), rtol=1e-15, atol=0)
    np.testing.assert_allclose(act.sigmoid(np.array([-800.0, 800.0])), [0.0, 1.0], atol=1e-300)


def test_activation_identities():
    x = np.random.default_rng(0).uniform(-30, 30, size=1000)
    # softplus(x) - softplus(-x) = x; sigmoid(x) + sigmoid(-x) = 1
    np.testing.assert_allclose(act.softplus(x) - act.softplus(-x), x, rtol=0, atol=1e-13)
    np.testing.assert_allclose(act.sigmoid(x) + act.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    # sigmoid is the derivative of softplus (central differences)
    h = 1e-5
    d = (act.softplus(x + h) - act.softplus(x - h)) / (2 * h)
    np.testing.assert_allclose(d, act.sigmoid(x), rtol=0, atol=1e-9)
    # e^{softplus(x)} = 1 + e^x on a range where neither side overflows
    y = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(np.exp(act.softplus(y)), 1.0 + np.exp(y), rtol=1e-14)


def test_log_gate_values():
    A = 3.0
    # a + dt_bias = 0: log alpha = -A ln 2
    assert abs(act.log_gate(0.25, np.log(A), -0.25) + A * np.log(2.0)) < 1e-15
    # a -> -inf: no decay; a large: log alpha -> -A (a + dt_bias)
    assert act.log_gate(-800.0, np.log(A), 0.0) == 0.0
    assert abs(act.log_gate(60.0, np.log(A), 1.0) / (-A * 61.0) - 1.0) < 1e-15
    # always <= 0 (alpha in (0, 1])
    a = np.random.default_rng(1).standard_normal((50, 4)) * 10
    assert np.all(act.log_gate(a, np.log([0.5, 1, 4, 16]), np.array([0.5, -1, 0, 2])) <= 0)


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_log_gate_broadcast_matches_elementwise(per_key):
    """The tensor form equals the formula applied element by element (the
    head index selects A_log, the head (and key channel) index dt_bias)."""
    rng = np.random.default_rng(2)
    T, H, K = 7, 3, 5
    a = rng.standard_normal((T, H, K) if per_key else (T, H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt = rng.standard_normal((H, K) if per_key else (H,))
    got = act.log_gate(a, A_log, dt)
    for t in range(T):
        for h in range(H):
            for c in (range(K) if per_key else [None]):
                ai = a[t, h, c] if per_key else a[t, h]
                di = dt[h, c] if per_key else dt[h]
                want = -np.exp(A_log[h]) * np.log1p(np.exp(ai + di))
                gi = got[t, h, c] if per_key else got[t, h]
                assert abs(gi - want) <= 1e-14 * max(1.0, abs(want))


def test_beta_ranges():
    b = np.random.default_rng(3).standard_normal(1000) * 6
    s = act.beta_from_logits(b)
    n = act.beta_from_logits(b, neg_eig=True)
    assert np.all((s > 0) & (s < 1)) and np.all((n > 0) & (n < 2))
    np.testing.assert_array_equal(n, 2 * s)
    assert act.beta_from_logits(0.0) == 0.5 and act.beta_from_logits(0.0, neg_eig=True) == 1.0


# ------------------------------------------------------ beta in (0, 2)
@pytest.mark.parametrize("beta", [1.3, 1.9, 2.0])
def test_householder_spectrum_negative(beta):
    """I - beta k k^T along a unit k has eigenvalue 1 - beta < 0 for beta > 1
    ("TileLang 实战…" §1.2); beta = 2 is a reflection (orthogonal)."""
    k = _unit(np.random.default_rng(4).standard_normal(6))
    P = oracle.transition(k, beta, 0.0, False)
    ev = np.sort(np.linalg.eigvals(P).real)
    assert np.max(np.abs(ev - np.sort([1 - beta] + [1.0] * 5))) < TOL
    if beta == 2.0:
        assert np.max(np.abs(P @ P.T - np.eye(6))) < TOL


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_same_key_readback_any_beta(per_key):
    """Reading with q = k_t and scale 1 right after the write returns
    beta v_t + (1 - beta) (D_t S_{t-1}^T) k_t (the rank-1 write, "DeltaNet 系列
    线性注意力变体的推导之旅", DeltaNet section), for beta in (0, 2)."""
    d = draw(5, T=6, H=2, K=5, V=3, per_key=per_key)
    rng = np.random.default_rng(6)
    d["beta"] = act.beta_from_logits(rng.standard_normal(d["beta"].shape) * 2, neg_eig=True)
    d["q"] = d["k"].copy()
    o, _ = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0, h0=d["h0"],
                                    gate=d["gate"])
    for t in range(6):
        pre = {n: x[:, :t] for n, x in d.items() if n in ("q", "k", "v", "beta", "g")}
        if t == 0:
            S = d["h0"][0]
        else:
            _, S = oracle.recurrent_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"],
                                            1.0, h0=d["h0"], gate=d["gate"])
            S = S[0]
        for h in range(2):
            dec = np.exp(d["g"][0, t, h])
            Sd = (dec[:, None] if per_key else dec) * S[h]   # decayed state [K, V]
            k, v, b = d["k"][0, t, h], d["v"][0, t, h], d["beta"][0, t, h]
            want = b * v + (1 - b) * (Sd.T @ k)
            assert np.max(np.abs(o[0, t, h] - want)) < 1e-12 * max(1, np.max(np.abs(want)))


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_brute_force_and_chunked_negative_eigenvalues(per_key):
    """beta in (0, 2): the recurrence equals the explicit transition products
    ("Gated Delta Network（GDN）" §4.1(a), eq. 8), and the chunked UT form equals
    the recurrence to 1e-10 (the unit-lower system stays invertible: det 1)."""
    d = draw(7, T=12, H=2, K=4, V=3, per_key=per_key)
    d["beta"] = act.beta_from_logits(np.random.default_rng(8).standard_normal(d["beta"].shape) * 2,
                                     neg_eig=True)
    o, ht = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 0.8, h0=d["h0"],
                                     gate=d["gate"])
    for h in range(2):
        ob, hb = oracle.brute_force_forward(d["q"][0, :, h], d["k"][0, :, h], d["v"][0, :, h],
                                            d["beta"][0, :, h], d["g"][0, :, h], 0.8,
                                            h0=d["h0"][0, h], gate=d["gate"])
        assert np.max(np.abs(o[0, :, h] - ob)) < 1e-12 * np.max(np.abs(ob))
        assert np.max(np.abs(ht[0, h] - hb)) < 1e-12 * np.max(np.abs(hb))
    e = draw(9, B=2, T=150, H=2, K=16, V=8, per_key=per_key, A=(1.0, 16.0))
    e["beta"] = act.beta_from_logits(np.random.default_rng(10).standard_normal(e["beta"].shape) * 2,
                                     neg_eig=True)
    a = oracle.recurrent_forward(e["q"], e["k"], e["v"], e["beta"], e["g"], 0.25, h0=e["h0"],
                                 gate=e["gate"])
    for chunk in (16, 64):
        b = oracle.chunked_forward(e["q"], e["k"], e["v"], e["beta"], e["g"], 0.25, h0=e["h0"],
                                   gate=e["gate"], chunk=chunk)
        for x, y in zip(b[:2], a):
            assert np.max(np.abs(x - y)) < 1e-10 * np.max(np.abs(y))


def test_l2_normalize_pins():
    """l2_normalize: unit norm and the same direction (up to the epsilon's
    relative 5e-7 at unit scale), exactly unit norm with eps = 0, scale
    invariance, per-row independence, and a zero row stays zero."""
    rng = np.random.default_rng(95)
    x = rng.standard_normal((3, 5, 2, 16)) * rng.uniform(0.5, 3.0, (3, 5, 2, 1))
    y = act.l2_normalize(x)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-6)
    assert np.allclose(y, x / n, rtol=0, atol=1e-6)
    y0 = act.l2_normalize(x, eps=0.0)
    assert np.allclose(np.linalg.norm(y0, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(act.l2_normalize(7.5 * x, eps=0.0), y0, rtol=0, atol=1e-14)
    # each (token, head) row on its own: normalising a slice gives the same
    assert np.array_equal(act.l2_normalize(x[1:2, 3:4, 1:2]), y[1:2, 3:4, 1:2])
    z = act.l2_normalize(np.zeros((2, 16)))
    assert np.all(z == 0.0)
    # the eps reading: x / sqrt(|x|^2 + 1e-6), checked on a row of norm 1e-3
    small = np.full(4, 5e-4)
    assert np.allclose(act.l2_normalize(small), small / np.sqrt(1e-6 + 1e-6), rtol=1e-14)
