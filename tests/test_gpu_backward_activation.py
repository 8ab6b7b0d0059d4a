"""GPU parity of the backward with the in-kernel input activation
(gdn_chunk_bwd_act: "Gated Delta Network（GDN）" §3.1 eq. 5, §5 gate fusion
and beta in (0, 2)) against the fp64 oracle: chunked_backward on the
activated inputs, then activation_backward's chain rule to the raw logits
and the per-head sums dA_log, ddt_bias.  Bar as in the other backward
tests (max |x - x_ref| <= tol max |x_ref| per gradient)."""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from oracle import activation as act
from oracle.backward import activation_backward, chunked_backward
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _run(spec, seed, gate_logits, beta_sigmoid, neg=False, m=1, dht_std=0.1):
    """m > 1: q, k with H / m heads shared by groups of m value heads."""
    import gated_delta_rule_14_amd as gdn
    print("case:", spec, "seed", seed, "gate", gate_logits, "beta", beta_sigmoid, "neg", neg,
          "m", m, flush=True)
    d = gdn_synth.make_prefill(spec, seed, logits=True)
    H = d["v"].shape[2]
    # a different dt_bias per head, so that a head mix-up shows
    d["dt_bias"] = d["dt_bias"] + torch.linspace(-0.5, 0.5, H, dtype=torch.float32)
    gr = gdn_synth.make_grads(d, seed, dht_std=dht_std)
    f64 = oracle.as_f64
    g_act = act.log_gate(f64(d["g"]), f64(d["A_log"]), f64(d["dt_bias"]))
    b_act = act.beta_from_logits(f64(d["beta"]), neg_eig=neg)
    x = to_dev(d)
    # inputs the kernels activate stay raw; the others are passed activated
    g_in = x["g"] if gate_logits else torch.from_numpy(g_act.astype(np.float32)).cuda()
    b_in = x["beta"] if beta_sigmoid else torch.from_numpy(b_act.astype(np.float32)).cuda()
    q, k = d["q"], d["k"]
    if m > 1:
        q, k = q[:, :, ::m].contiguous(), k[:, :, ::m].contiguous()
    a = gdn.activation(gate_logits=gate_logits, beta_sigmoid=beta_sigmoid, neg_eig=neg,
                       A_log=d["A_log"].cuda(), dt_bias=d["dt_bias"].cuda())
    got = gdn.chunk_bwd(q.cuda(), k.cuda(), x["v"], b_in, g_in, gr["do"].cuda(), d["scale"],
                        h0=x.get("h0"), dht=gr["dht"].cuda() if gr["dht"] is not None else None,
                        cu_seqlens=x.get("cu_seqlens"), act=a)
    torch.cuda.synchronize()
    qe, ke = (q.repeat_interleave(m, dim=2), k.repeat_interleave(m, dim=2)) if m > 1 else (q, k)
    ref = chunked_backward(qe, ke, d["v"], b_act, g_act, d["scale"], gr["do"], h0=d.get("h0"),
                           dht=gr["dht"], cu_seqlens=d.get("cu_seqlens"), chunk=d["chunk"])
    if m > 1:
        B, T = d["v"].shape[:2]
        for name in ("dq", "dk"):
            ref[name] = ref[name].reshape(B, T, H // m, m, -1).sum(axis=3)
    da, db, dA_log, ddt = activation_backward(d["g"], d["beta"], d["A_log"], d["dt_bias"],
                                              ref["dg"], ref["dbeta"], neg_eig=neg)
    names = ["dq", "dk", "dv", "dbeta", "dg", "dh0"]
    if gate_logits:
        ref["dg"], ref["dA_log"], ref["ddt_bias"] = da, dA_log, ddt
        names += ["dA_log", "ddt_bias"]
    else:
        assert "dA_log" not in got
    if beta_sigmoid:
        ref["dbeta"] = db
    tol = TOL[spec.dtype]
    errs = {n: rel_err(got[n], ref[n]) for n in names}
    print("relative errors:", {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= tol, "%s: %.3g > %.1g" % (n, e, tol)


def test_bwd_act_f32_all(gpu_lib):
    """fp32, K = V = 64, ragged tail: gate and beta logits, beta in (0, 2)."""
    spec = gdn_synth.prefill_spec(0, B=2, T=200, H=3, h0_std=0.1)
    _run(spec, 91, True, True, neg=True)


@pytest.mark.parametrize("gate_logits,beta_sigmoid,neg", [(True, True, False), (True, False, False),
                                                          (False, True, True)])
def test_bwd_act_bf16(gpu_lib, gate_logits, beta_sigmoid, neg):
    spec = gdn_synth.prefill_spec(1, B=2, T=300, H=3)
    _run(spec, 92, gate_logits, beta_sigmoid, neg)


def test_bwd_act_bf16_packed_with_empty_sequence(gpu_lib):
    """Unused chunk slots of the packed table must not enter dA_log, ddt_bias."""
    spec = gdn_synth.prefill_spec(1, H=2, rand_lengths=None, lengths=(70, 0, 129, 64, 1),
                                  h0_std=0.02)
    _run(spec, 93, True, True, neg=True)


def test_bwd_act_bf16_gva(gpu_lib):
    """Grouped value heads (two value heads per q/k head) with the activation."""
    spec = gdn_synth.prefill_spec(1, B=2, T=150, H=4, K=64, V=128, h0_std=0.05)
    _run(spec, 94, True, True, neg=False, m=2)


@pytest.mark.slow
def test_bwd_act_full_size_head_sums(gpu_lib):
    """The 4 x 4096-token, 16-head, d = 128 bf16 workload with gate and beta
    logits: dA_log and ddt_bias (sums over 16384 tokens) against the oracle
    for every head; the per-token gradients of two (sequence, head) pairs."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.PREFILL[1]
    print("case: full size, activation", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 1, logits=True)
    gr = gdn_synth.make_grads(d, 1)
    x = to_dev(d)
    a = gdn.activation(gate_logits=True, beta_sigmoid=True, A_log=d["A_log"].cuda(),
                       dt_bias=d["dt_bias"].cuda())
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                        h0=x.get("h0"), dht=gr["dht"].cuda(), act=a)
    torch.cuda.synchronize()
    f64 = oracle.as_f64
    g_act = act.log_gate(f64(d["g"]), f64(d["A_log"]), f64(d["dt_bias"]))
    b_act = act.beta_from_logits(f64(d["beta"]))
    B, T, H = d["v"].shape[:3]
    dA = np.zeros(H)
    ddt = np.zeros(H)
    h0 = d.get("h0")
    for h in range(H):
        sl = slice(h, h + 1)
        ref = chunked_backward(d["q"][:, :, sl], d["k"][:, :, sl], d["v"][:, :, sl],
                               b_act[:, :, sl], g_act[:, :, sl], d["scale"], gr["do"][:, :, sl],
                               h0=h0[:, sl] if h0 is not None else None, dht=gr["dht"][:, sl],
                               chunk=d["chunk"])
        da, db, dA_h, ddt_h = activation_backward(d["g"][:, :, sl], d["beta"][:, :, sl],
                                                  d["A_log"][sl], d["dt_bias"][sl], ref["dg"],
                                                  ref["dbeta"])
        dA[h], ddt[h] = dA_h[0], ddt_h[0]
        if h in (0, 11):
            for name, r in (("dg", da), ("dbeta", db), ("dq", ref["dq"]), ("dk", ref["dk"])):
                e = rel_err(got[name][:, :, sl], r)
                print("head", h, name, "%.2e" % e, flush=True)
                assert e <= TOL["bf16"], (h, name, e)
    e1, e2 = rel_err(got["dA_log"], dA), rel_err(got["ddt_bias"], ddt)
    print("dA_log %.2e ddt_bias %.2e" % (e1, e2), flush=True)
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]
