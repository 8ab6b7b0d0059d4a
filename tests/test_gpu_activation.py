"""GPU parity of the in-kernel input activation (gdn_chunk_fwd_act,
gdn_recurrent_step_act: "Gated Delta Network（GDN）" §3.1 eq. 5 and §5 gate
fusion) and of beta in (0, 2) (§5, negative eigenvalues), against the fp64
oracle applied to the same raw logits.  Bar as in the other parity tests."""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from oracle import activation as act
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _activated(d, neg):
    g = act.log_gate(oracle.as_f64(d["g"]), oracle.as_f64(d["A_log"]), oracle.as_f64(d["dt_bias"]))
    b = act.beta_from_logits(oracle.as_f64(d["beta"]), neg_eig=neg)
    return g, b


def _prefill(spec, seed, gate_logits, beta_sigmoid, neg=False, heads=None):
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(spec, seed, logits=True)
    print("case:", spec, "seed", seed, "gate", gate_logits, "beta", beta_sigmoid, "neg", neg,
          flush=True)
    x = to_dev(d)
    g_ref, b_ref = _activated(d, neg)
    # inputs the kernel activates stay raw; the others are passed activated
    g_in = x["g"] if gate_logits else torch.from_numpy(g_ref.astype(np.float32)).cuda()
    b_in = x["beta"] if beta_sigmoid else torch.from_numpy(b_ref.astype(np.float32)).cuda()
    a = gdn.activation(gate_logits=gate_logits, beta_sigmoid=beta_sigmoid, neg_eig=neg,
                       A_log=d["A_log"].cuda(), dt_bias=d["dt_bias"].cuda())
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], b_in, g_in, d["scale"], h0=x.get("h0"),
                          cu_seqlens=x.get("cu_seqlens"), gate=d["gate"], act=a)
    torch.cuda.synchronize()
    q, k, v, h0 = d["q"], d["k"], d["v"], d.get("h0")
    if heads is not None:
        sel = list(heads)
        q, k, v, g_ref, b_ref = q[:, :, sel], k[:, :, sel], v[:, :, sel], g_ref[:, :, sel], \
            b_ref[:, :, sel]
        h0 = h0[:, sel] if h0 is not None else None
        o, ht = o[:, :, sel], ht[:, sel]
    o_ref, ht_ref = oracle.recurrent_forward(q, k, v, b_ref, g_ref, d["scale"], h0=h0,
                                             cu_seqlens=d.get("cu_seqlens"), gate=d["gate"])
    tol = TOL[spec.dtype]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    assert eo <= tol and eh <= tol, (eo, eh)
    return eo, eh


def _spec(cid, **kw):
    return gdn_synth.prefill_spec(cid, **kw)


# bf16, scalar gate, K = V = 128: the fused kernel; ragged last chunk
@pytest.mark.parametrize("gate_logits,beta_sigmoid,neg", [(True, True, False), (True, True, True),
                                                          (True, False, False),
                                                          (False, True, True)])
def test_fused_activation(gpu_lib, gate_logits, beta_sigmoid, neg):
    _prefill(_spec(1, B=2, T=200, H=3), 31, gate_logits, beta_sigmoid, neg)


def test_fused_activation_packed(gpu_lib):
    spec = _spec(2, H=3, rand_lengths=None, lengths=(70, 1, 0, 129, 64), h0_std=0.02)
    _prefill(spec, 32, True, True, True)


# the two-stage route: fp32, and the per-key gate (dt_bias per head and channel)
@pytest.mark.parametrize("dt,gate,K,V", [("f32", "scalar", 64, 64), ("bf16", "per_key", 64, 128),
                                         ("f32", "per_key", 64, 64)])
def test_two_stage_activation(gpu_lib, dt, gate, K, V):
    cid = 3 if gate == "per_key" else 1
    _prefill(_spec(cid, dtype=dt, B=2, T=150, H=2, K=K, V=V, h0_std=0.02), 33, True, True, True)


def test_negative_eigenvalues_bench_shape(gpu_lib):
    """beta = 2 sigmoid(b) in (0, 2) on the bench shape's sequence length and
    head size (B=4, T=4096, d=128, bf16, nonzero initial state), 4 heads, every
    output against the oracle."""
    _prefill(_spec(1, H=4), 34, True, True, True)


@pytest.mark.parametrize("dt,gate,K,V", [("bf16", "scalar", 128, 128), ("f32", "per_key", 64, 128)])
def test_decode_activation(gpu_lib, dt, gate, K, V):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.DecodeSpec("t", dt, N=5, H=3, K=K, V=V, steps=8, gate=gate)
    d = gdn_synth.make_decode(spec, 35, logits=True)
    print("case:", spec, flush=True)
    x = to_dev(d)
    a = gdn.activation(gate_logits=True, beta_sigmoid=True, neg_eig=True, A_log=d["A_log"].cuda(),
                       dt_bias=d["dt_bias"].cuda())
    state = x["state"].clone()
    outs = [gdn.recurrent_step(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s], state,
                               scale=d["scale"], gate=gate, act=a) for s in range(spec.steps)]
    torch.cuda.synchronize()
    g_ref, b_ref = _activated(d, True)
    ref = oracle.as_f64(d["state"])
    for s in range(spec.steps):
        o_ref, ref = oracle.recurrent_step(d["q"][s], d["k"][s], d["v"][s], b_ref[s], g_ref[s],
                                           d["scale"], ref, gate=gate)
        assert rel_err(outs[s], o_ref) <= TOL[dt], ("step", s)
    assert rel_err(state, ref) <= TOL[dt]
