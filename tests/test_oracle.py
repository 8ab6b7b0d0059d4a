"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import gdn_synth
from oracle_pins import (ALL_FWD_PINS, draw, pin_equal_channel_gates,
                         pin_householder_spectrum)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-13


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("pin", ALL_FWD_PINS, ids=lambda p: p.__name__)
def test_recurrence_pins(pin, per_key):
    assert pin(oracle.recurrent_forward, per_key=per_key) < TOL


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("pin", ALL_FWD_PINS, ids=lambda p: p.__name__)
def test_chunked_pins(pin, per_key):
    """The chunked UT reference satisfies the same pins (chunk 4: several
    chunks and a ragged tail in every case)."""
    def fwd(*a, **kw):
        kw.pop("threads", None)
        kw.pop("want_state", None)
        return oracle.chunked_forward(*a, chunk=4, **kw)
    assert pin(fwd, per_key=per_key) < 1e-12


def test_equal_channel_gates():
    assert pin_equal_channel_gates(oracle.recurrent_forward) < TOL


def test_householder_spectrum():
    assert pin_householder_spectrum() < TOL


def _fwd_both(d, scale, chunk, **kw):
    a = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], scale,
                                 h0=d["h0"], gate=d["gate"], **kw)
    b = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], scale,
                               h0=d["h0"], gate=d["gate"], chunk=chunk, **kw)
    return a, b


def _rel(x, y):
    return np.max(np.abs(x - y)) / np.max(np.abs(y))


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 150])
def test_chunked_matches_recurrence(per_key, chunk, T):
    """Chunked UT form vs token recurrence to 1e-10 relative (the chunked and
    recurrent forms are the same map in exact arithmetic: "TileLang 实战…"
    §2.3 and its §3.4 check)."""
    d = draw(11 + T, B=2, T=T, H=2, K=16, V=8, per_key=per_key, A=(1.0, 16.0))
    (o1, h1), (o2, h2) = _fwd_both(d, 0.25, chunk)
    assert _rel(o2, o1) < 1e-10
    assert _rel(h2, h1) < 1e-10


def test_chunked_matches_recurrence_packed():
    d = gdn_synth.make_prefill(gdn_synth.prefill_spec(2, H=2, K=16, V=12,
                               rand_lengths=None, lengths=(70, 1, 0, 129, 64)), 5)
    a = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                                 cu_seqlens=d["cu_seqlens"])
    b = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                               cu_seqlens=d["cu_seqlens"], chunk=64)
    assert _rel(b[0], a[0]) < 1e-10 and _rel(b[1], a[1]) < 1e-10


def test_golden_tilelang_consistency_table():
    """Reproduce the page's §3.4 setting (B=2, H=2, N=12, d=4, C=4, fp64,
    scale 1, zero state): chunk+UT vs token recurrence, the d_v-tiled mirror,
    alpha == 1 and beta -> 1e-12.  The page's inputs are not printed, so our
    draws differ; the errors must sit at the same rounding level."""
    gold = json.load(open(os.path.join(GOLDEN, "tilelang_gdn_sec3_4.json")))
    c = gold["config"]
    d = draw(2024, B=c["B"], T=c["N"], H=c["H"], K=c["d_k"], V=c["d_v"], h0=False)
    (o1, h1), (o2, h2) = _fwd_both(d, 1.0, c["C"])
    slack = 16.0
    assert np.max(np.abs(o2 - o1)) <= slack * gold["max_abs"]["chunk_vs_token"]
    # d_v-tiled mirror: each block of block_DV value columns run alone
    bd = c["block_DV"]
    for j in range(0, c["d_v"], bd):
        e = dict(d)
        e["v"] = d["v"][..., j:j + bd]
        oe, _ = oracle.chunked_forward(e["q"], e["k"], e["v"], e["beta"], e["g"], 1.0,
                                       chunk=c["C"])
        assert np.max(np.abs(oe - o1[..., j:j + bd])) <= slack * gold["max_abs"]["mirror_vs_token"]
    a1 = dict(d)
    a1["g"] = np.zeros_like(d["g"])
    (o1, _), (o2, _) = _fwd_both(a1, 1.0, c["C"])
    assert np.max(np.abs(o2 - o1)) <= slack * gold["max_abs"]["alpha1_chunk_vs_token"]
    b0 = dict(d)
    b0["beta"] = np.full_like(d["beta"], 1e-12)
    (o1, _), (o2, _) = _fwd_both(b0, 1.0, c["C"])
    assert np.max(np.abs(o2 - o1)) <= slack * gold["max_abs"]["beta_1e-12_chunk_vs_token"]


def test_ungated_wy_identities():
    """P = I - W^T K and H = U^T K, with w_r, u_r from the WY recursions
    ("TileLang 实战…" §2.2.2-2.2.3, eqs. 4-5), and the chunked reference's
    W, U at alpha == 1 equal those recursions (its UT route, eqs. 6-7)."""
    d = draw(21, T=8, H=1, K=6, V=5)
    k, v, b = d["k"][0, :, 0], d["v"][0, :, 0], d["beta"][0, :, 0]
    W, U, P, Hm = oracle.wy_ungated(k, v, b)
    assert np.max(np.abs(P - (np.eye(6) - W.T @ k))) < TOL
    assert np.max(np.abs(Hm - U.T @ k)) < TOL
    g0 = np.zeros_like(d["g"])
    _, _, inter = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], g0, 1.0,
                                         chunk=8, keep=True)
    assert np.max(np.abs(inter["W"][0, :, 0] - W)) < TOL
    assert np.max(np.abs(inter["U"][0, :, 0] - U)) < TOL


@pytest.mark.parametrize("per_key", [False, True], ids=["gdn", "kda"])
def test_gated_chunk_transition(per_key):
    """With gates, one chunk maps S_in to S_in F + G_w with
    F = Diag(gamma_C) - W^T K~ and G_w = U^T K~, K~ = K scaled to the chunk end;
    F and G_w must equal the explicit products of the per-token transitions
    ("TileLang 实战…" §2.1; "Gated Delta Network（GDN）" eq. 8)."""
    d = draw(22, T=6, H=1, K=5, V=4, per_key=per_key)
    _, _, inter = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0,
                                         gate=d["gate"], chunk=6, keep=True)
    k, v, b, g = d["k"][0, :, 0], d["v"][0, :, 0], d["beta"][0, :, 0], d["g"][0, :, 0]
    W, U = inter["W"][0, :, 0], inter["U"][0, :, 0]
    G = np.cumsum(g, axis=0)
    if per_key:
        Kt = np.exp(G[-1][None, :] - G) * k
        F = np.diag(np.exp(G[-1])) - W.T @ Kt
    else:
        Kt = np.exp(G[-1] - G)[:, None] * k
        F = np.exp(G[-1]) * np.eye(5) - W.T @ Kt
    Gw = U.T @ Kt
    Fx = np.eye(5)
    Hx = np.zeros((4, 5))
    for i in range(6):
        Ai = oracle.transition(k[i], b[i], g[i], per_key)
        Fx = Fx @ Ai
        Hx = Hx @ Ai + b[i] * np.outer(v[i], k[i])
    assert np.max(np.abs(F - Fx)) < TOL
    assert np.max(np.abs(Gw - Hx)) < TOL


def test_triangular_inverse_and_two_constructions():
    """Ainv = (I + A)^{-1} with A strictly lower and unit diagonal system
    ("TileLang 实战…" §2.3: determinant 1, no pivoting), checked against a
    triangular solve; A built as diag(beta)(Gamma * K K^T) equals
    ((K * beta) K^T) * Gamma (the §3.4 remark)."""
    d = draw(23, T=64, H=1, K=32, V=4, A=(1.0, 16.0))
    _, _, inter = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], 1.0,
                                         chunk=64, keep=True)
    A = inter["A"][0, :, 0]
    Ai = inter["Ainv"][0, :, 0]
    n = A.shape[0]
    assert np.allclose(np.triu(A), 0.0)
    assert np.max(np.abs((np.eye(n) + A) @ Ai - np.eye(n))) < 1e-12
    ref = scipy.linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True,
                                        unit_diagonal=True)
    assert np.max(np.abs(Ai - ref)) < 1e-12
    k, b, g = d["k"][0, :, 0], d["beta"][0, :, 0], d["g"][0, :, 0]
    G = np.cumsum(g)
    idx = np.arange(n)
    low = idx[:, None] >= idx[None, :]
    Gam = np.where(low, np.exp(np.where(low, G[:, None] - G[None, :], 0.0)), 0.0)
    A2 = np.tril(((k * b[:, None]) @ k.T) * Gam, -1)
    assert np.max(np.abs(A - A2)) < 1e-15


def test_decode_step_is_one_token_of_the_recurrence():
    d = gdn_synth.make_decode(gdn_synth.DecodeSpec("t", "bf16", N=3, H=2, K=8, V=6, steps=3))
    st = oracle.as_f64(d["state"])
    seq_o = []
    for s in range(3):
        o, st = oracle.recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s],
                                      d["g"][s], d["scale"], st)
        seq_o.append(o)
    # the same tokens as 3 sequences of length 3 run as prefill
    q = d["q"].permute(1, 0, 2, 3)
    o2, h2 = oracle.recurrent_forward(q, d["k"].permute(1, 0, 2, 3), d["v"].permute(1, 0, 2, 3),
                                      d["beta"].permute(1, 0, 2), d["g"].permute(1, 0, 2),
                                      d["scale"], h0=d["state"])
    assert np.max(np.abs(np.stack(seq_o, 1) - o2)) < TOL
    assert np.max(np.abs(st - h2)) < TOL


def test_generator_is_deterministic_and_normalised():
    a = gdn_synth.make_prefill(gdn_synth.prefill_spec(1, B=1, T=70, H=2), 3)
    b = gdn_synth.make_prefill(gdn_synth.prefill_spec(1, B=1, T=70, H=2), 3)
    for key in ("q", "k", "v", "beta", "g", "h0"):
        assert (a[key] == b[key]).all()
    n = a["k"].double().norm(dim=-1)
    assert (n - 1).abs().max() < 1e-2          # bf16 rounding of unit rows
    assert (a["g"] <= 0).all() and (a["beta"] > 0).all() and (a["beta"] < 1).all()
    L = gdn_synth.draw_lengths(2, 2)
    assert len(L) == 16 and L[-1] == 65536 and all(128 <= x <= 8192 for x in L[:-1])
    small = gdn_synth.prefill_spec(2, H=2, K=16, V=16, rand_lengths=(3, 5, 9, 40))
    p = gdn_synth.make_prefill(small, 2)
    assert int(p["cu_seqlens"][-1]) == sum(p["lengths"]) == p["q"].shape[1]
    assert p["lengths"][-1] == 40 and all(5 <= x <= 9 for x in p["lengths"][:3])
