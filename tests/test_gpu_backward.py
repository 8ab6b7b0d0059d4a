"""GPU parity of the chunked backward (gdn_chunk_bwd) against the fp64
oracle on the same seeded inputs.

Reference: oracle.backward.chunked_backward (numpy fp64, pinned to autograd
through the token recurrence to 1e-10, which is pinned by central
differences of the C recurrence); one case also compares with the autograd
oracle directly.  Every gradient must satisfy
max|x - x_ref| <= tol * max|x_ref| with the forward's bar: 1e-4 for fp32
inputs, 2e-2 for bf16 inputs (fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import gdn_synth
from oracle.backward import chunked_backward, recurrent_backward
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def _gpu(d, gr, want_dh0=True):
    import gated_delta_rule_14_amd as gdn
    x = to_dev(d)
    out = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(),
                        scale=d["scale"], h0=x.get("h0"),
                        dht=gr["dht"].cuda() if gr["dht"] is not None else None,
                        cu_seqlens=x.get("cu_seqlens"), want_dh0=want_dh0)
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
    kw = dict(h0=h0, dht=dht, cu_seqlens=d.get("cu_seqlens"))
    if fn is chunked_backward:
        kw["chunk"] = d["chunk"]
    return fn(q, k, v, beta, g, d["scale"], do, **kw)


def _check(d, got, ref, tol=None, heads=None, batch=None, names=NAMES):
    tol = TOL[d["spec"].dtype] if tol is None else tol
    errs = {}
    for name in names:
        x = got[name]
        if x is None:
            continue
        if batch is not None:
            x = x[batch:batch + 1]
        if heads is not None:
            x = x[:, list(heads)] if name == "dh0" else x[:, :, list(heads)]
        errs[name] = rel_err(x, ref[name])
    print("relative errors:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= tol, "%s: %.3g > %.1g" % (name, e, tol)
    return errs


def _case(spec, seed, dht_std=0.1, want_dh0=True):
    print("case:", spec, "seed", seed, flush=True)
    d = gdn_synth.make_prefill(spec, seed)
    gr = gdn_synth.make_grads(d, seed, dht_std=dht_std)
    return d, gr, _gpu(d, gr, want_dh0)


def test_bwd_f32_d64_ragged(gpu_lib):
    """fp32, K = V = 64, several chunks and a ragged tail, h0 and dht."""
    spec = gdn_synth.prefill_spec(0, B=2, T=200, H=2, h0_std=0.1)
    d, gr, got = _case(spec, 51)
    _check(d, got, _ref(d, gr))


def test_bwd_f32_strong_decay_against_autograd(gpu_lib):
    """fp32 with the pages' strong gates (A up to 16), compared with the
    autograd oracle itself."""
    spec = gdn_synth.prefill_spec(0, B=1, T=130, H=2, A_range=(1.0, 16.0), h0_std=0.1)
    d, gr, got = _case(spec, 52)
    _check(d, got, _ref(d, gr, fn=recurrent_backward))


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_bwd_bf16(gpu_lib, K, V):
    spec = gdn_synth.prefill_spec(1, B=2, T=300, H=3, K=K, V=V)
    d, gr, got = _case(spec, 53 + K + V)
    _check(d, got, _ref(d, gr))


def test_bwd_bf16_packed_with_empty_sequence(gpu_lib):
    spec = gdn_synth.prefill_spec(2, H=3, rand_lengths=None, lengths=(70, 0, 129, 64, 1),
                                  h0_std=0.02)
    d, gr, got = _case(spec, 54)
    _check(d, got, _ref(d, gr))


def test_bwd_no_state_gradients(gpu_lib):
    """No h0, no dht, dh0 not requested."""
    spec = gdn_synth.prefill_spec(1, B=1, T=190, H=2, h0_std=None)
    d, gr, got = _case(spec, 55, dht_std=None, want_dh0=False)
    assert got["dh0"] is None
    _check(d, got, _ref(d, gr), names=NAMES[:-1])


def test_bwd_wide_beta(gpu_lib):
    """beta in (0, 2): the negative-eigenvalue range of the write."""
    spec = gdn_synth.prefill_spec(1, B=1, T=200, H=2)
    print("case: wide beta", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 56)
    d["beta"] = 2.0 * d["beta"]
    gr = gdn_synth.make_grads(d, 56)
    _check(d, _gpu(d, gr), _ref(d, gr))


@pytest.mark.slow
def test_bwd_full_size_sampled(gpu_lib):
    """The 4 x 4096-token, 16-head, d = 128 bf16 prefill: the whole backward
    on the GPU, two (sequence, head) pairs checked against the oracle."""
    spec = gdn_synth.PREFILL[1]
    d, gr, got = _case(spec, 1)
    for b, h in ((0, 0), (3, 11)):
        _check(d, got, _ref(d, gr, heads=[h], batch=b), heads=[h], batch=b)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_bwd_chunk_edges(gpu_lib, T):
    """One token, exactly one chunk, one chunk and one token (bf16, K = V = 128)."""
    spec = gdn_synth.prefill_spec(1, B=2, T=T, H=2)
    d, gr, got = _case(spec, 60 + T)
    _check(d, got, _ref(d, gr))


def test_bwd_f32_single_head_strong_gates(gpu_lib):
    """fp32, one head, the strongest gates of the bench workload (A up to 16)
    over several chunks: gamma underflows inside chunks."""
    spec = gdn_synth.prefill_spec(0, B=1, T=320, H=1, A_range=(8.0, 16.0), h0_std=0.1)
    d, gr, got = _case(spec, 70)
    _check(d, got, _ref(d, gr))


@pytest.mark.parametrize("dt,cid,K,V,m", [("bf16", 1, 128, 128, 2), ("bf16", 1, 64, 128, 4),
                                          ("f32", 0, 64, 64, 2)])
def test_bwd_gva(gpu_lib, dt, cid, K, V, m):
    """Grouped value heads: q, k with H heads, everything of a state with
    H_V = m H.  Reference: the oracle on q, k repeated m times along the head
    axis, its dq, dk summed over each group of m value heads (the chain rule
    of the repetition)."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(cid, dtype=dt, B=2, T=150, H=4, K=K, V=V, h0_std=0.05)
    print("case: gva", spec, "m", m, flush=True)
    d = gdn_synth.make_prefill(spec, 80 + m)
    gr = gdn_synth.make_grads(d, 80 + m)
    q, k = d["q"][:, :, ::m].contiguous(), d["k"][:, :, ::m].contiguous()
    x = to_dev(d)
    got = gdn.chunk_bwd(q.cuda(), k.cuda(), x["v"], x["beta"], x["g"], gr["do"].cuda(),
                        scale=d["scale"], h0=x["h0"], dht=gr["dht"].cuda())
    torch.cuda.synchronize()
    qe, ke = q.repeat_interleave(m, dim=2), k.repeat_interleave(m, dim=2)
    ref = chunked_backward(qe, ke, d["v"], d["beta"], d["g"], d["scale"], gr["do"], h0=d["h0"],
                           dht=gr["dht"], chunk=d["chunk"])
    B, T, Hv = d["v"].shape[:3]
    for name in ("dq", "dk"):
        ref[name] = ref[name].reshape(B, T, Hv // m, m, K).sum(axis=3)
    assert tuple(got["dq"].shape) == tuple(q.shape)
    _check(d, got, ref)
