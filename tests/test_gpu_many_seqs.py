"""Packed input with more sequences than the chunk table ranks by length
(1100 > 1024: the sequences are then taken in index order), many of them
empty or one token long, on the fused route (bf16, K = V = 128), the
two-stage route (fp32, K = V = 64) and the backward.  Reference: the fp64
oracle on the same inputs; bar as in the other parity tests."""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from oracle.backward import chunked_backward
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

N_SEQ = 1100


def _lengths(seed):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, 41, N_SEQ)       # 0 .. 40 tokens
    n[rng.choice(N_SEQ, 40, replace=False)] = 0
    n[:3] = (130, 64, 1)                 # a few that span chunks
    return tuple(int(x) for x in n)


@pytest.mark.parametrize("cid,dt,K,V", [(1, "bf16", 128, 128), (0, "f32", 64, 64)])
def test_forward_many_sequences(gpu_lib, cid, dt, K, V):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(cid, dtype=dt, H=2, K=K, V=V, rand_lengths=None,
                                  lengths=_lengths(110 + cid), h0_std=0.05)
    print("case: %d packed sequences" % N_SEQ, spec.dtype, K, V, flush=True)
    d = gdn_synth.make_prefill(spec, 111)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                                             h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print("relative errors: o %.2e ht %.2e" % (eo, eh), flush=True)
    assert eo <= TOL[dt] and eh <= TOL[dt]
    # an empty sequence hands its initial state through unchanged
    lens = np.diff(d["cu_seqlens"].numpy())
    empty = np.nonzero(lens == 0)[0]
    assert len(empty) > 0
    assert torch.equal(ht[empty].cpu(), d["h0"][empty])


def test_backward_many_sequences(gpu_lib):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(1, H=2, K=64, V=64, rand_lengths=None, lengths=_lengths(112),
                                  h0_std=0.05)
    print("case: backward, %d packed sequences" % N_SEQ, flush=True)
    d = gdn_synth.make_prefill(spec, 113)
    gr = gdn_synth.make_grads(d, 113)
    x = to_dev(d)
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                        h0=x["h0"], dht=gr["dht"].cuda(), cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = chunked_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"], gr["do"],
                           h0=d["h0"], dht=gr["dht"], cu_seqlens=d["cu_seqlens"], chunk=d["chunk"])
    errs = {n: rel_err(got[n], ref[n]) for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0")}
    print("relative errors:", {n: "%.2e" % e for n, e in errs.items()}, flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= TOL["bf16"], "%s: %.3g" % (n, e)
