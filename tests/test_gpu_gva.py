"""GPU parity of grouped value heads (GVA, "Gated Delta Network（GDN）" §5):
q, k with H heads, v with H_V = m H heads, one state per value head, value
head hv reading q/k head hv // m.  Reference: the fp64 recurrence per value
head on q, k repeated m times along the head axis."""
import pytest
import torch

import gdn_synth
import oracle
from oracle import activation as act
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _gva_prefill(spec, m, seed, with_act=False):
    """spec.H is the value-head count; q and k keep every m-th head."""
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(spec, seed, logits=with_act)
    print("case:", spec, "m", m, "seed", seed, "act", with_act, flush=True)
    q, k = d["q"][:, :, ::m].contiguous(), d["k"][:, :, ::m].contiguous()
    x = to_dev(d)
    kw = {}
    beta, g = d["beta"], d["g"]
    if with_act:
        kw["act"] = gdn.activation(gate_logits=True, beta_sigmoid=True, neg_eig=True,
                                   A_log=d["A_log"].cuda(), dt_bias=d["dt_bias"].cuda())
        g = act.log_gate(oracle.as_f64(d["g"]), oracle.as_f64(d["A_log"]), oracle.as_f64(d["dt_bias"]))
        beta = act.beta_from_logits(oracle.as_f64(d["beta"]), neg_eig=True)
    o, ht = gdn.chunk_fwd(q.cuda(), k.cuda(), x["v"], x["beta"], x["g"], d["scale"], h0=x.get("h0"),
                          cu_seqlens=x.get("cu_seqlens"), gate=d["gate"], **kw)
    torch.cuda.synchronize()
    qe, ke = q.repeat_interleave(m, dim=2), k.repeat_interleave(m, dim=2)
    o_ref, ht_ref = oracle.recurrent_forward(qe, ke, d["v"], beta, g, d["scale"], h0=d.get("h0"),
                                             cu_seqlens=d.get("cu_seqlens"), gate=d["gate"])
    tol = TOL[spec.dtype]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    assert eo <= tol and eh <= tol, (eo, eh)


def test_gva_fused(gpu_lib):
    """bf16, scalar gate, K = V = 128 (the fused kernel), m = 2, ragged."""
    _gva_prefill(gdn_synth.prefill_spec(1, B=2, T=200, H=4), 2, 41)


def test_gva_fused_packed_with_activation(gpu_lib):
    spec = gdn_synth.prefill_spec(2, H=6, rand_lengths=None, lengths=(70, 1, 129), h0_std=0.02)
    _gva_prefill(spec, 3, 42, with_act=True)


@pytest.mark.parametrize("dt,cid,K,V,m", [("f32", 1, 64, 64, 2), ("bf16", 3, 64, 128, 2),
                                          ("bf16", 3, 128, 64, 4)])
def test_gva_two_stage(gpu_lib, dt, cid, K, V, m):
    _gva_prefill(gdn_synth.prefill_spec(cid, dtype=dt, B=2, T=150, H=4, K=K, V=V, h0_std=0.02),
                 m, 43)


@pytest.mark.parametrize("dt,gate,K,V,m", [("bf16", "scalar", 128, 128, 2),
                                           ("f32", "per_key", 64, 128, 4)])
def test_gva_decode(gpu_lib, dt, gate, K, V, m):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.DecodeSpec("t", dt, N=5, H=4, K=K, V=V, steps=6, gate=gate)
    d = gdn_synth.make_decode(spec, 44)
    print("case:", spec, "m", m, flush=True)
    x = to_dev(d)
    q, k = x["q"][:, :, ::m].contiguous(), x["k"][:, :, ::m].contiguous()
    state = x["state"].clone()
    outs = [gdn.recurrent_step(q[s], k[s], x["v"][s], x["beta"][s], x["g"][s], state,
                               scale=d["scale"], gate=gate) for s in range(spec.steps)]
    torch.cuda.synchronize()
    qe = d["q"][:, :, ::m].repeat_interleave(m, dim=2)
    ke = d["k"][:, :, ::m].repeat_interleave(m, dim=2)
    ref = oracle.as_f64(d["state"])
    for s in range(spec.steps):
        o_ref, ref = oracle.recurrent_step(qe[s], ke[s], d["v"][s], d["beta"][s], d["g"][s],
                                           d["scale"], ref, gate=gate)
        assert rel_err(outs[s], o_ref) <= TOL[dt], ("step", s)
    assert rel_err(state, ref) <= TOL[dt]
