"""Shared helpers for the GPU parity tests: run the HIP path and the oracle
on the same seeded inputs and compare to the bar the method fixes."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(d):
    out = dict(d)
    for key in ("q", "k", "v", "beta", "g", "h0", "cu_seqlens", "state"):
        if d.get(key) is not None:
            out[key] = d[key].cuda()
    return out


def run_gpu(d, **kw):
    import gated_delta_rule_14_amd as gdn
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], scale=d["scale"],
                          h0=x.get("h0"), cu_seqlens=x.get("cu_seqlens"), chunk=d["chunk"],
                          gate=d["gate"], **kw)
    torch.cuda.synchronize()
    return o, ht


def run_oracle(d, heads=None):
    """The fp64 token recurrence; with `heads`, only those heads (the others
    stay zero)."""
    q, k, v, beta, g, h0 = d["q"], d["k"], d["v"], d["beta"], d["g"], d.get("h0")
    if heads is not None:
        sel = list(heads)
        q, k, v, beta, g = (x[:, :, sel] for x in (q, k, v, beta, g))
        h0 = h0[:, sel] if h0 is not None else None
    return oracle.recurrent_forward(q, k, v, beta, g, d["scale"], h0=h0,
                                    cu_seqlens=d.get("cu_seqlens"), gate=d["gate"])


def rel_err(got, want):
    got = got.detach().float().cpu().double().numpy() if hasattr(got, "detach") else got
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def check(d, o, ht, o_ref, ht_ref, heads=None, tol=None):
    tol = TOL[d["spec"].dtype] if tol is None else tol
    if heads is not None:
        o = o[:, :, list(heads)]
        ht = ht[:, list(heads)] if ht is not None else None
    eo = rel_err(o, o_ref)
    eh = rel_err(ht, ht_ref) if ht is not None else 0.0
    assert np.isfinite(eo) and eo <= tol, "o: max|o-o_ref| / max|o_ref| = %.3g > %.1g" % (eo, tol)
    assert np.isfinite(eh) and eh <= tol, "ht: relative error %.3g > %.1g" % (eh, tol)
    return eo, eh
