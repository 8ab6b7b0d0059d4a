"""The single-pass kernel at the head sizes other than K = V = 128 (bf16,
scalar gate): (K, V) in {(64, 64), (128, 64), (64, 128)}.  The kernel is
compiled once per (K, V); what K changes is the K/Q row length in local
memory (and its bank permutation), the number of 32-channel MFMA steps of
the K h, Q h and K K^T products and the number of 16-row state tiles per
state wave; V changes the number of 32-wide value slices per head.  Cases:
packed sequences with empty ones, grouped value heads with the activation,
L2-normalised q/k, strong gates at the workloads' full shape with the
state carried through weak gates, and the two-stage route against this
one.  Reference: the fp64 recurrence; bar max|x - x_ref| <= 2e-2 max|x_ref|."""
import pytest
import torch

import gdn_synth
import oracle
from parity_util import TOL, check, rel_err, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu

HEADS = [(64, 64), (128, 64), (64, 128)]


@pytest.mark.parametrize("K,V", HEADS)
def test_packed_with_empty(gpu_lib, K, V):
    import gated_delta_rule_14_amd as gdn
    lengths = (0, 70, 1, 0, 129, 64)
    spec = gdn_synth.prefill_spec(2, H=3, K=K, V=V, rand_lengths=None, lengths=lengths, h0_std=0.05)
    print("case: packed", spec, flush=True)
    d = gdn_synth.make_prefill(spec, 150)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(d)
    print("relative errors: o %.2e ht %.2e" % check(d, o, ht, o_ref, ht_ref), flush=True)
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(ht[n].cpu(), d["h0"][n]), n


@pytest.mark.parametrize("K,V", HEADS)
def test_gva_with_activation(gpu_lib, K, V):
    from test_gpu_gva import _gva_prefill
    _gva_prefill(gdn_synth.prefill_spec(1, B=2, T=300, H=4, K=K, V=V, h0_std=0.02), 2, 151,
                 with_act=True)


@pytest.mark.parametrize("K,V", HEADS)
def test_l2norm(gpu_lib, K, V):
    import gated_delta_rule_14_amd as gdn
    from oracle import activation as act
    from test_gpu_l2norm import _normalised, _rescale
    spec = gdn_synth.prefill_spec(1, B=2, T=200, H=3, K=K, V=V, h0_std=0.05)
    print("case: l2norm", spec, flush=True)
    d = _rescale(gdn_synth.make_prefill(spec, 152, logits=True), 153)
    x = to_dev(d)
    a = gdn.activation(gate_logits=True, beta_sigmoid=True, qk_l2norm=True, A_log=d["A_log"].cuda(),
                       dt_bias=d["dt_bias"].cuda())
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"], act=a)
    torch.cuda.synchronize()
    g = act.log_gate(oracle.as_f64(d["g"]), oracle.as_f64(d["A_log"]), oracle.as_f64(d["dt_bias"]))
    b = act.beta_from_logits(oracle.as_f64(d["beta"]))
    qn, kn = _normalised(d)
    o_ref, ht_ref = oracle.recurrent_forward(qn, kn, d["v"], b, g, d["scale"], h0=d["h0"])
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print("relative errors: o %.2e ht %.2e" % (eo, eh), flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("K,V", HEADS)
@pytest.mark.parametrize("A_range", [None, (0.001, 0.05)])
def test_full_shape(gpu_lib, K, V, A_range):
    """B=4, T=4096, H=16: 64 chained chunks per sequence, every output of
    every head; the workloads' gates, then weak ones."""
    kw = {} if A_range is None else {"A_range": A_range}
    spec = gdn_synth.prefill_spec(1, K=K, V=V, **kw)
    d = gdn_synth.make_prefill(spec, 154)
    print("case:", spec, flush=True)
    o, ht = run_gpu(d)
    o_ref, ht_ref = run_oracle(d)
    print("relative errors: o %.2e ht %.2e" % check(d, o, ht, o_ref, ht_ref), flush=True)


@pytest.mark.parametrize("K,V", HEADS + [(128, 128)])
def test_routes_agree(gpu_lib, K, V):
    """gdn_chunk_intra + gdn_chunk_scan (the two-stage route, which
    gdn_chunk_fwd no longer takes for these bf16 shapes) against the oracle
    and against gdn_chunk_fwd, weak gates so the carried state matters."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(1, B=2, T=330, H=2, K=K, V=V, A_range=(0.001, 0.05))
    d = gdn_synth.make_prefill(spec, 155)
    print("case: routes", spec, flush=True)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"])
    r = gdn.chunk_intra(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], store_ainv=False)
    o2, ht2 = torch.empty_like(o), torch.empty_like(ht)
    gdn.chunk_scan(r["desc"], r["workspace"], o2, h0=x["h0"], ht=ht2)
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(d)
    check(d, o, ht, o_ref, ht_ref)
    check(d, o2, ht2, o_ref, ht_ref)
    check(d, o2, ht2, o.double().cpu().numpy(), ht.double().cpu().numpy())


@pytest.mark.parametrize("K,V", HEADS)
def test_no_state_in_or_out(gpu_lib, K, V):
    """No initial state (zeros) and no final state requested: o alone, ragged."""
    spec = gdn_synth.prefill_spec(1, B=2, T=150, H=2, K=K, V=V, h0_std=None)
    d = gdn_synth.make_prefill(spec, 156)
    print("case: no h0, no ht", spec, flush=True)
    o, ht = run_gpu(d, output_final_state=False)
    assert ht is None
    o_ref, ht_ref = run_oracle(d)
    print("relative error: o %.2e" % check(d, o, None, o_ref, None)[0], flush=True)
