"""gdn_chunk_fwd_noalloc (the forward without a workspace, for callers that
cannot allocate) against gdn_chunk_fwd on the same inputs: two calls in a
row on one GPU, the second with fewer packed sequences and tokens than the
first (the library's scratch keeps the first call's records), then a call
without packed offsets.  The two entry points run the same kernels on the
same inputs, so o and ht must agree bit for bit; the first call is also
checked against the fp64 oracle at the bf16 bar."""
import ctypes

import pytest
import torch

import gdn_synth
import oracle
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(d, x, o, ht):
    import gated_delta_rule_14_amd as gdn
    from gated_delta_rule_14_amd import _binding as B
    lib = gdn.load()
    cu = x.get("cu_seqlens")
    N = cu.numel() - 1 if cu is not None else x["q"].shape[0]
    desc = gdn.fwd_desc(x["q"], x["v"], "scalar", 64, d["scale"], N if cu is not None else 0)
    B._check(lib.gdn_chunk_fwd_noalloc(ctypes.byref(desc), None, B._ptr(x["q"]), B._ptr(x["k"]),
                                       B._ptr(x["v"]), B._ptr(x["beta"]), B._ptr(x["g"]),
                                       B._ptr(x.get("h0")), B._ptr(cu), B._ptr(o), B._ptr(ht),
                                       B._stream(None)))


def _case(spec, seed, want_oracle=False):
    import gated_delta_rule_14_amd as gdn
    print("case: no-alloc", spec.name, getattr(spec, "lengths", None), "seed", seed, flush=True)
    d = gdn_synth.make_prefill(spec, seed)
    x = to_dev(d)
    o_ref, ht_ref = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"],
                                  h0=x.get("h0"), cu_seqlens=x.get("cu_seqlens"))
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    _noalloc(d, x, o, ht)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
    if want_oracle:
        o64, ht64 = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                                             h0=d.get("h0"), cu_seqlens=d.get("cu_seqlens"))
        assert rel_err(o, o64) <= TOL["bf16"] and rel_err(ht, ht64) <= TOL["bf16"]


def test_noalloc_matches_chunk_fwd(gpu_lib):
    big = gdn_synth.prefill_spec(2, H=4, rand_lengths=None, lengths=(300, 0, 129, 64, 1, 700, 65),
                                 h0_std=0.05)
    small = gdn_synth.prefill_spec(2, H=2, rand_lengths=None, lengths=(70, 3), h0_std=0.05)
    _case(big, 150, want_oracle=True)
    _case(small, 151)
    _case(gdn_synth.prefill_spec(1, B=2, T=200, H=2), 152)
    # the other head sizes run the same entry point (K = V = 64 here)
    _case(gdn_synth.prefill_spec(2, H=2, K=64, V=64, rand_lengths=None, lengths=(130, 5)), 153)


def test_noalloc_refuses_other_shapes(gpu_lib):
    import gated_delta_rule_14_amd as gdn
    from gated_delta_rule_14_amd import _binding as B
    lib = gdn.load()
    fake = ctypes.c_void_p(1 << 20)
    for kw in (dict(qkv_dtype=0), dict(gate=1), dict(key_dim=96), dict(chunk=32)):
        a = dict(batch=1, seq_len=64, num_heads=2, key_dim=128, value_dim=128, num_seqs=0, chunk=64,
                 qkv_dtype=1, gate=0, scale=0.088)
        a.update(kw)
        desc = gdn.FwdDesc(**a)
        assert lib.gdn_chunk_fwd_noalloc(ctypes.byref(desc), None, fake, fake, fake, fake, fake, None,
                                         None, fake, None, None) == 4
    desc = gdn.FwdDesc(1, 64, 2, 128, 128, 5000, 64, 1, 0, 0.088, 0)
    assert lib.gdn_chunk_fwd_noalloc(ctypes.byref(desc), None, fake, fake, fake, fake, fake, None,
                                     fake, fake, None, None) == 4
    assert "4096" in lib.gdn_last_error().decode()
