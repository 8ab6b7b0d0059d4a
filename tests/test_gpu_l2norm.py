"""GPU parity of the in-kernel q/k L2 normalisation (GDN_ACT_QK_L2NORM) against
the fp64 oracle: the oracle normalises the same q, k (oracle.activation.
l2_normalize) and runs the recurrence or the chunked backward on them; the
backward's dq, dk then go through oracle.backward.l2_normalize_backward.

The generator's q and k are already unit-norm, so every case first scales
each (token, head) row by a seeded factor in [0.25, 4] and rounds to the
input dtype; both sides read those rounded values.  Bar as in the other
parity tests (max |x - x_ref| <= tol max |x_ref|)."""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from oracle import activation as act
from oracle.backward import chunked_backward, l2_normalize_backward
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _rescale(d, seed):
    """q, k rows times seeded factors, rounded to the input dtype."""
    rng = np.random.default_rng(seed)
    for name in ("q", "k"):
        x = d[name]
        f = torch.from_numpy(rng.uniform(0.25, 4.0, tuple(x.shape[:-1]) + (1,)))
        d[name] = (x.double() * f).to(x.dtype)
    return d


def _normalised(d):
    return act.l2_normalize(oracle.as_f64(d["q"])), act.l2_normalize(oracle.as_f64(d["k"]))


@pytest.mark.parametrize("cid,dt,gate,K,V,logits", [
    (1, "bf16", "scalar", 128, 128, False),    # the fused kernel's shape
    (1, "bf16", "scalar", 128, 128, True),     # with the gate and beta activations too
    (0, "f32", "per_key", 64, 64, False),
    (1, "bf16", "per_key", 128, 64, True),
])
def test_prefill_l2norm(gpu_lib, cid, dt, gate, K, V, logits):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(cid, dtype=dt, B=2, T=200, H=3, K=K, V=V, gate=gate, h0_std=0.05)
    print("case: l2norm prefill", spec, "logits", logits, flush=True)
    d = _rescale(gdn_synth.make_prefill(spec, 101, logits=logits), 201)
    x = to_dev(d)
    a = gdn.activation(gate_logits=logits, beta_sigmoid=logits, qk_l2norm=True,
                       A_log=d["A_log"].cuda() if logits else None,
                       dt_bias=d["dt_bias"].cuda() if logits else None)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          gate=gate, act=a)
    torch.cuda.synchronize()
    g, b = oracle.as_f64(d["g"]), oracle.as_f64(d["beta"])
    if logits:
        g = act.log_gate(g, oracle.as_f64(d["A_log"]), oracle.as_f64(d["dt_bias"]))
        b = act.beta_from_logits(b)
    qn, kn = _normalised(d)
    o_ref, ht_ref = oracle.recurrent_forward(qn, kn, d["v"], b, g, d["scale"], h0=d["h0"], gate=gate)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print("relative errors: o %.2e ht %.2e" % (eo, eh), flush=True)
    assert eo <= TOL[dt] and eh <= TOL[dt]


def test_prefill_l2norm_packed_gva(gpu_lib):
    """Packed sequences (one empty) with two value heads per q/k head."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(1, H=4, K=64, V=128, rand_lengths=None, lengths=(70, 0, 129, 1),
                                  h0_std=0.02)
    print("case: l2norm packed gva", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 102)
    m = 2
    d["q"], d["k"] = d["q"][:, :, ::m].contiguous(), d["k"][:, :, ::m].contiguous()
    d = _rescale(d, 202)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          cu_seqlens=x["cu_seqlens"], act=gdn.activation(qk_l2norm=True))
    torch.cuda.synchronize()
    qn, kn = _normalised(d)
    qn, kn = np.repeat(qn, m, axis=2), np.repeat(kn, m, axis=2)
    o_ref, ht_ref = oracle.recurrent_forward(qn, kn, d["v"], d["beta"], d["g"], d["scale"],
                                             h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print("relative errors: o %.2e ht %.2e" % (eo, eh), flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("dt,gate,K,V", [("bf16", "scalar", 128, 128), ("f32", "per_key", 64, 64)])
def test_decode_l2norm(gpu_lib, dt, gate, K, V):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.DecodeSpec("l2-decode", dt, N=6, H=2, K=K, V=V, steps=3, gate=gate)
    print("case: l2norm decode", spec, flush=True)
    d = gdn_synth.make_decode(spec, 103)
    st = d["state"].cuda()
    ref_st = oracle.as_f64(d["state"])
    rng = np.random.default_rng(203)
    a = gdn.activation(qk_l2norm=True)
    for t in range(spec.steps):
        q = (d["q"][t].double() * torch.from_numpy(rng.uniform(0.25, 4.0, (6, 2, 1)))).to(d["q"].dtype)
        k = (d["k"][t].double() * torch.from_numpy(rng.uniform(0.25, 4.0, (6, 2, 1)))).to(d["k"].dtype)
        o = gdn.recurrent_step(q.cuda(), k.cuda(), d["v"][t].cuda(), d["beta"][t].cuda(),
                               d["g"][t].cuda(), st, d["scale"], gate=gate, act=a)
        torch.cuda.synchronize()
        o_ref, ref_st = oracle.recurrent_step(act.l2_normalize(oracle.as_f64(q)),
                                              act.l2_normalize(oracle.as_f64(k)), d["v"][t],
                                              d["beta"][t], d["g"][t], d["scale"], ref_st, gate=gate)
        eo = rel_err(o, o_ref)
        print("step %d o rel err %.2e" % (t, eo), flush=True)
        assert eo <= TOL[dt]
    es = rel_err(st, ref_st)
    print("state rel err %.2e" % es, flush=True)
    assert es <= TOL[dt]


@pytest.mark.parametrize("cid,dt,K,V,m,logits", [(1, "bf16", 128, 128, 1, True),
                                                (0, "f32", 64, 64, 1, False),
                                                (1, "bf16", 64, 128, 2, False)])
def test_backward_l2norm(gpu_lib, cid, dt, K, V, m, logits):
    """dq, dk of the raw rows: the oracle's chunked backward on the
    normalised q, k (q, k repeated over each group of m value heads, their
    gradients summed per group), then the normalisation's chain rule."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(cid, dtype=dt, B=2, T=150, H=2 * m, K=K, V=V, h0_std=0.05)
    print("case: l2norm backward", spec, "m", m, "logits", logits, flush=True)
    d = gdn_synth.make_prefill(spec, 104, logits=logits)
    if m > 1:
        d["q"], d["k"] = d["q"][:, :, ::m].contiguous(), d["k"][:, :, ::m].contiguous()
    d = _rescale(d, 204)
    gr = gdn_synth.make_grads(d, 104)
    x = to_dev(d)
    a = gdn.activation(gate_logits=logits, beta_sigmoid=logits, qk_l2norm=True,
                       A_log=d["A_log"].cuda() if logits else None,
                       dt_bias=d["dt_bias"].cuda() if logits else None)
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                        h0=x["h0"], dht=gr["dht"].cuda(), act=a)
    torch.cuda.synchronize()
    g, b = oracle.as_f64(d["g"]), oracle.as_f64(d["beta"])
    if logits:
        g = act.log_gate(g, oracle.as_f64(d["A_log"]), oracle.as_f64(d["dt_bias"]))
        b = act.beta_from_logits(b)
    qn, kn = _normalised(d)
    ref = chunked_backward(np.repeat(qn, m, axis=2), np.repeat(kn, m, axis=2), d["v"], b, g,
                           d["scale"], gr["do"], h0=d["h0"], dht=gr["dht"], chunk=d["chunk"])
    B, T, Hv = d["v"].shape[:3]
    names = ["dq", "dk", "dv", "dh0"]
    for name, raw in (("dq", d["q"]), ("dk", d["k"])):
        dn = ref[name].reshape(B, T, Hv // m, m, K).sum(axis=3)
        ref[name] = l2_normalize_backward(raw, dn)
    if not logits:   # (with logits dbeta, dg are the logits' gradients: covered elsewhere)
        names += ["dbeta", "dg"]
    errs = {n: rel_err(got[n], ref[n]) for n in names}
    print("relative errors:", {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= TOL[dt], "%s: %.3g" % (n, e)
