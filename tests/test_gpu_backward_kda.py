"""GPU parity of the chunked backward with the per-key-channel gate (Kimi
Delta Attention) against the fp64 oracle on the same seeded inputs.

Reference: oracle.backward.chunked_backward(gate="per_key") (numpy fp64,
pinned to the autograd backward of the token recurrence to 1e-10, itself
pinned by central differences of the C recurrence); the strong-decay case
compares with the autograd oracle directly.  The activation cases follow
with oracle.backward.activation_backward (per-channel dt_bias) and
l2_normalize_backward.  Every gradient must satisfy
max|x - x_ref| <= 2e-2 * max|x_ref| (bf16 inputs, fp32 accumulation), the
bar of the other backward tests.
"""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from oracle import activation as act
from oracle.backward import (activation_backward, chunked_backward, l2_normalize_backward,
                             recurrent_backward)
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def _spec(**kw):
    base = dict(B=2, T=300, H=3, gate="per_key", h0_std=0.05)
    base.update(kw)
    return gdn_synth.prefill_spec(3, **base)


def _gpu(d, gr, want_dh0=True):
    import gated_delta_rule_14_amd as gdn
    x = to_dev(d)
    out = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(),
                        scale=d["scale"], h0=x.get("h0"),
                        dht=gr["dht"].cuda() if gr["dht"] is not None else None,
                        cu_seqlens=x.get("cu_seqlens"), want_dh0=want_dh0, gate="per_key")
    torch.cuda.synchronize()
    return out


def _ref(d, gr, heads=None, batch=None, fn=chunked_backward):
    q, k, v, beta, g, h0, do, dht = (d["q"], d["k"], d["v"], d["beta"], d["g"], d.get("h0"),
                                     gr["do"], gr["dht"])
    if batch is not None:
        q, k, v, beta, g, do = (x[batch:batch + 1] for x in (q, k, v, beta, g, do))
        h0 = h0[batch:batch + 1] if h0 is not None else None
        dht = dht[batch:batch + 1] if dht is not None else None
    if heads is not None:
        sel = list(heads)
        q, k, v, beta, g, do = (x[:, :, sel] for x in (q, k, v, beta, g, do))
        h0 = h0[:, sel] if h0 is not None else None
        dht = dht[:, sel] if dht is not None else None
    kw = dict(h0=h0, dht=dht, cu_seqlens=d.get("cu_seqlens"), gate="per_key")
    if fn is chunked_backward:
        kw["chunk"] = d["chunk"]
    return fn(q, k, v, beta, g, d["scale"], do, **kw)


def _check(got, ref, heads=None, batch=None, names=NAMES):
    errs = {}
    for name in names:
        x = got[name]
        if batch is not None:
            x = x[batch:batch + 1]
        if heads is not None:
            x = x[:, list(heads)] if name == "dh0" else x[:, :, list(heads)]
        errs[name] = rel_err(x, ref[name])
    print("relative errors:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= TOL["bf16"], "%s: %.3g > %.1g" % (name, e, TOL["bf16"])


def _case(spec, seed, dht_std=0.1, want_dh0=True):
    print("case: kda backward", spec, "seed", seed, flush=True)
    d = gdn_synth.make_prefill(spec, seed)
    gr = gdn_synth.make_grads(d, seed, dht_std=dht_std)
    return d, gr, _gpu(d, gr, want_dh0)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_kda_bwd(gpu_lib, K, V):
    """Several chunks and a ragged tail, h0 and dht."""
    d, gr, got = _case(_spec(K=K, V=V), 153 + K + V)
    _check(got, _ref(d, gr))


@pytest.mark.parametrize("T", [1, 16, 64, 65])
def test_kda_bwd_chunk_edges(gpu_lib, T):
    """One token, one 16-token block, exactly one chunk, one chunk and one token."""
    d, gr, got = _case(_spec(T=T, H=2), 160 + T)
    _check(got, _ref(d, gr))


def test_kda_bwd_strong_decay_against_autograd(gpu_lib):
    """The pages' strongest gates (A up to 16, so per-channel decays
    underflow inside a 16-token block), against the autograd oracle."""
    d, gr, got = _case(_spec(B=1, T=130, H=2, A_range=(4.0, 16.0)), 152)
    _check(got, _ref(d, gr, fn=recurrent_backward))


def test_kda_bwd_packed_with_empty_sequence(gpu_lib):
    spec = _spec(H=3, rand_lengths=None, lengths=(70, 0, 129, 64, 1), h0_std=0.02)
    d, gr, got = _case(spec, 154)
    _check(got, _ref(d, gr))


def test_kda_bwd_no_state_gradients(gpu_lib):
    """No h0, no dht, dh0 not requested."""
    d, gr, got = _case(_spec(B=1, T=190, H=2, h0_std=None), 155, dht_std=None, want_dh0=False)
    assert got["dh0"] is None
    _check(got, _ref(d, gr), names=NAMES[:-1])


def test_kda_bwd_wide_beta(gpu_lib):
    """beta in (0, 2): the negative-eigenvalue range of the write."""
    spec = _spec(B=1, T=200, H=2)
    print("case: kda wide beta", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 156)
    d["beta"] = 2.0 * d["beta"]
    gr = gdn_synth.make_grads(d, 156)
    _check(_gpu(d, gr), _ref(d, gr))


@pytest.mark.parametrize("m,l2", [(1, False), (1, True), (2, False)])
def test_kda_bwd_activation(gpu_lib, m, l2):
    """Gate and beta logits (beta in (0, 2)), per-channel dt_bias: the
    logit gradients and dA_log [H], ddt_bias [H, K]; with l2 the q/k
    normalisation too; m = 2: two value heads per q/k head."""
    import gated_delta_rule_14_amd as gdn
    spec = _spec(B=2, T=150, H=4, K=64 if m > 1 else 128, V=128, h0_std=0.05)
    seed = 170 + 10 * m + l2
    print("case: kda backward activation", spec, "m", m, "l2", l2, flush=True)
    d = gdn_synth.make_prefill(spec, seed, logits=True)
    H, K = d["v"].shape[2], d["q"].shape[3]
    d["dt_bias"] = d["dt_bias"] + torch.linspace(-0.5, 0.5, H * K, dtype=torch.float32).reshape(H, K)
    gr = gdn_synth.make_grads(d, seed)
    q, k = d["q"], d["k"]
    if l2:   # rows of norm other than 1, rounded to bf16 (both sides read these)
        rng = np.random.default_rng(seed)
        q, k = ((x.double() * torch.from_numpy(rng.uniform(0.25, 4.0, tuple(x.shape[:-1]) + (1,))))
                .to(x.dtype) for x in (q, k))
    if m > 1:
        q, k = q[:, :, ::m].contiguous(), k[:, :, ::m].contiguous()
    x = to_dev(d)
    a = gdn.activation(gate_logits=True, beta_sigmoid=True, neg_eig=True, qk_l2norm=l2,
                       A_log=d["A_log"].cuda(), dt_bias=d["dt_bias"].cuda())
    got = gdn.chunk_bwd(q.cuda(), k.cuda(), x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                        h0=x["h0"], dht=gr["dht"].cuda(), act=a, gate="per_key")
    torch.cuda.synchronize()
    f64 = oracle.as_f64
    g_act = act.log_gate(f64(d["g"]), f64(d["A_log"]), f64(d["dt_bias"]))
    b_act = act.beta_from_logits(f64(d["beta"]), neg_eig=True)
    qe, ke = (q.repeat_interleave(m, dim=2), k.repeat_interleave(m, dim=2)) if m > 1 else (q, k)
    qn, kn = (act.l2_normalize(f64(qe)), act.l2_normalize(f64(ke))) if l2 else (qe, ke)
    ref = chunked_backward(qn, kn, d["v"], b_act, g_act, d["scale"], gr["do"], h0=d["h0"],
                           dht=gr["dht"], chunk=d["chunk"], gate="per_key")
    if l2:
        ref["dq"] = l2_normalize_backward(qe, ref["dq"])
        ref["dk"] = l2_normalize_backward(ke, ref["dk"])
    if m > 1:
        B, T = d["v"].shape[:2]
        for name in ("dq", "dk"):
            ref[name] = ref[name].reshape(B, T, H // m, m, -1).sum(axis=3)
    ref["dg"], ref["dbeta"], ref["dA_log"], ref["ddt_bias"] = activation_backward(
        d["g"], d["beta"], d["A_log"], d["dt_bias"], ref["dg"], ref["dbeta"], neg_eig=True)
    _check(got, ref, names=NAMES + ("dA_log", "ddt_bias"))


@pytest.mark.slow
def test_kda_bwd_full_size_sampled(gpu_lib):
    """The 2 x 8192-token, 16-head, d = 128 bf16 KDA prefill: the whole
    backward on the GPU, two (sequence, head) pairs checked against the oracle."""
    spec = gdn_synth.PREFILL[3]
    d, gr, got = _case(spec, 3)
    for b, h in ((0, 0), (1, 13)):
        _check(got, _ref(d, gr, heads=[h], batch=b), heads=[h], batch=b)


def test_kda_bwd_activation_packed_with_empty_sequences(gpu_lib):
    """Gate and beta logits on packed input with empty sequences: the unused
    chunk slots of the packed table must not enter dA_log or ddt_bias."""
    import gated_delta_rule_14_amd as gdn
    spec = _spec(H=2, K=64, V=64, rand_lengths=None, lengths=(0, 70, 0, 129, 64, 1), h0_std=0.05)
    print("case: kda backward activation, packed", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 181, logits=True)
    H, K = d["v"].shape[2], d["q"].shape[3]
    d["dt_bias"] = d["dt_bias"] + torch.linspace(-0.5, 0.5, H * K, dtype=torch.float32).reshape(H, K)
    gr = gdn_synth.make_grads(d, 181)
    x = to_dev(d)
    a = gdn.activation(gate_logits=True, beta_sigmoid=True, A_log=d["A_log"].cuda(),
                       dt_bias=d["dt_bias"].cuda())
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                        h0=x["h0"], dht=gr["dht"].cuda(), cu_seqlens=x["cu_seqlens"], act=a,
                        gate="per_key")
    torch.cuda.synchronize()
    f64 = oracle.as_f64
    g_act = act.log_gate(f64(d["g"]), f64(d["A_log"]), f64(d["dt_bias"]))
    b_act = act.beta_from_logits(f64(d["beta"]))
    ref = chunked_backward(d["q"], d["k"], d["v"], b_act, g_act, d["scale"], gr["do"], h0=d["h0"],
                           dht=gr["dht"], cu_seqlens=d["cu_seqlens"], chunk=d["chunk"],
                           gate="per_key")
    ref["dg"], ref["dbeta"], ref["dA_log"], ref["ddt_bias"] = activation_backward(
        d["g"], d["beta"], d["A_log"], d["dt_bias"], ref["dg"], ref["dbeta"])
    _check(got, ref, names=NAMES + ("dA_log", "ddt_bias"))
