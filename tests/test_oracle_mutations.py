"""Planted mistakes in a copy of the recurrence must each fail some pin.

The copy below is a small numpy twin of the oracle's token recurrence with
switches that introduce the mistakes the pages warn about (reading before
the write, dropping alpha from the erase term, decaying after the write,
losing the scale, ...).  Every mistake must be caught by at least one of the
pins that the real oracle passes, which shows the pins are strong enough.
"""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_FWD_PINS, pin_equal_channel_gates


def twin(mistake=None):
    def fwd(q, k, v, beta, g, scale, h0=None, cu_seqlens=None, gate="scalar",
            threads=0, want_state=True):
        q, k, v, beta, g = (oracle.as_f64(x) for x in (q, k, v, beta, g))
        B, T, H, K = q.shape
        V = v.shape[-1]
        per_key = gate == "per_key"
        if cu_seqlens is None:
            seqs = [(b, b, 0, T) for b in range(B)]
        else:
            cu = np.asarray(cu_seqlens)
            seqs = [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
        o = np.zeros((B, T, H, V))
        ht = np.zeros((len(seqs), H, K, V))
        for n, b, s0, s1 in seqs:
            for hh in range(H):
                h = np.array(h0[n, hh], dtype=float) if h0 is not None else np.zeros((K, V))
                if mistake == "h0_ignored":
                    h = np.zeros((K, V))
                for t in range(s0, s1):
                    gt = g[b, t - 1 if (mistake == "gate_lag" and t > s0) else t, hh]
                    if mistake == "gate_sign":
                        gt = -gt
                    dec = np.exp(gt)
                    D = dec[:, None] if per_key else dec
                    if mistake == "kda_columns" and per_key:
                        D = dec[None, :V] if V <= K else dec[None, :]
                    kt, vt, qt, bt = k[b, t, hh], v[b, t, hh], q[b, t, hh], beta[b, t, hh]
                    sq = qt if mistake == "no_scale" else scale * qt
                    if mistake == "decay_after_write":
                        p = h.T @ kt
                        h = D * (h + np.outer(kt, bt * (vt - p)))
                    elif mistake == "no_alpha_in_erase":
                        p = h.T @ kt
                        h = D * h + np.outer(kt, bt * (vt - p))
                    elif mistake == "beta_on_v_only":
                        h = D * h
                        p = h.T @ kt
                        h = h + np.outer(kt, bt * vt - p)
                    elif mistake == "read_before_write":
                        h = D * h
                        o[b, t, hh] = h.T @ sq
                        p = h.T @ kt
                        h = h + np.outer(kt, bt * (vt - p))
                        continue
                    else:
                        h = D * h
                        p = h.T @ kt
                        h = h + np.outer(kt, bt * (vt - p))
                    o[b, t, hh] = (h @ sq[:V] if mistake == "transposed_read" and K == V
                                   else h.T @ sq)
                ht[n, hh] = h
        return o, ht
    return fwd


MISTAKES = ["read_before_write", "decay_after_write", "no_alpha_in_erase",
            "beta_on_v_only", "no_scale", "gate_sign", "gate_lag", "h0_ignored",
            "kda_columns"]


def _caught(fwd, per_key):
    worst = 0.0
    for pin in ALL_FWD_PINS:
        try:
            worst = max(worst, pin(fwd, per_key=per_key))
        except Exception:
            return True
    return worst > 1e-6


def test_twin_without_mistake_passes():
    for per_key in (False, True):
        for pin in ALL_FWD_PINS:
            assert pin(twin(None), per_key=per_key) < 1e-12


@pytest.mark.parametrize("mistake", MISTAKES)
def test_mistake_is_caught(mistake):
    per_key = mistake == "kda_columns"
    assert _caught(twin(mistake), per_key)


def test_transposed_read_is_caught():
    # only expressible with K == V; the brute-force pin runs at K=4, V=3, so
    # use the equal-gate pin's shapes through a square draw instead
    from oracle_pins import pin_brute_force
    assert pin_brute_force(twin("transposed_read"), K=4, V=4) > 1e-6
