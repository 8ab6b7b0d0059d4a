"""GPU parity with weak gates, where the state carries across many chunks.

With the workloads' default gate magnitudes (A ~ U(1, 16), per-token
log-decay -A softplus(N(0,1) + 0.5)) a chunk's state has decayed by at least
e^-60 before the next chunk ends, so it reaches the next chunk's outputs only
through that chunk's first tokens and never reaches the final state.  With
A ~ U(0.001, 0.05) the decay over a chunk is e^-0.06 .. e^-3: the state
decay gamma_C h, the K h correction of the chunk's values and the rounding
of the carried state all reach o and ht over every chunk of the sequence.
Same bar as every parity test: max|x - x_ref| <= tol * max|x_ref|, 1e-4 for
fp32 inputs, 2e-2 for bf16 (fp32 accumulation).
"""
import pytest

import gdn_synth
from parity_util import check, run_gpu, run_oracle
from test_gpu_backward import _case, _check, _ref

pytestmark = pytest.mark.gpu

WEAK = (0.001, 0.05)


def _fwd(spec, seed):
    d = gdn_synth.make_prefill(spec, seed)
    print("case:", spec, "seed", seed, flush=True)
    o, ht = run_gpu(d)
    o_ref, ht_ref = run_oracle(d)
    print("relative errors: o %.2e ht %.2e" % check(d, o, ht, o_ref, ht_ref), flush=True)


@pytest.mark.parametrize("dt,K,V", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64),
                                    ("f32", 128, 128), ("f32", 64, 64)])
def test_weak_gates_routes(gpu_lib, dt, K, V):
    """bf16 runs the single-pass kernel at each of these head sizes, fp32 the
    two-stage route.  600 tokens: ten chunks, the last one ragged."""
    _fwd(gdn_synth.prefill_spec(1, dtype=dt, B=2, T=600, H=2, K=K, V=V, A_range=WEAK), 21)


@pytest.mark.parametrize("dt,K", [("bf16", 128), ("f32", 64)])
def test_weak_gates_per_key(gpu_lib, dt, K):
    _fwd(gdn_synth.prefill_spec(3, dtype=dt, B=2, T=600, H=2, K=K, A_range=WEAK, h0_std=0.02), 22)


def test_weak_gates_packed(gpu_lib):
    """Packed sequences, one of them empty: each restarts from its own h0."""
    _fwd(gdn_synth.prefill_spec(2, H=3, rand_lengths=None, lengths=(700, 0, 129, 1000), A_range=WEAK,
                                h0_std=0.02), 23)


def test_weak_gates_bench_shape(gpu_lib):
    """The bench workload's shape (B=4, T=4096, H=16, d=128, bf16, h0) with
    weak gates: 64 chained chunks per sequence, every output of every head."""
    _fwd(gdn_synth.prefill_spec(1, A_range=WEAK), 24)


@pytest.mark.parametrize("dt,K,V", [("bf16", 128, 128), ("f32", 64, 64)])
def test_weak_gates_backward(gpu_lib, dt, K, V):
    """The reverse recurrence carries dH across every chunk."""
    spec = gdn_synth.prefill_spec(1, dtype=dt, B=2, T=600, H=2, K=K, V=V, A_range=WEAK)
    d, gr, got = _case(spec, 25)
    _check(d, got, _ref(d, gr))


def test_weak_gates_backward_per_key(gpu_lib):
    import test_gpu_backward_kda as kda
    spec = kda._spec(B=1, T=600, H=2, A_range=WEAK, h0_std=0.02)
    print("case:", spec, "seed", 26, flush=True)
    d = gdn_synth.make_prefill(spec, 26)
    gr = gdn_synth.make_grads(d, 26)
    _check(d, kda._gpu(d, gr), kda._ref(d, gr))


@pytest.mark.parametrize("cid,dt,K,V", [(1, "bf16", 128, 128), (3, "bf16", 64, 128)])
def test_weak_gates_activation(gpu_lib, cid, dt, K, V):
    """Raw gate and beta logits activated in the kernels (A_log = log A),
    beta in (0, 2): the single-pass kernel and the per-key two-stage route."""
    from test_gpu_activation import _prefill
    spec = gdn_synth.prefill_spec(cid, dtype=dt, B=2, T=600, H=2, K=K, V=V, A_range=WEAK, h0_std=0.02)
    print("relative errors: o %.2e ht %.2e" % _prefill(spec, 27, True, True, True), flush=True)


def test_weak_gates_gva(gpu_lib):
    """Two value heads per q/k head on the single-pass kernel, with the
    activation."""
    from test_gpu_gva import _gva_prefill
    _gva_prefill(gdn_synth.prefill_spec(1, B=2, T=600, H=4, A_range=WEAK), 2, 28, with_act=True)


def test_weak_gates_l2norm(gpu_lib):
    """q/k normalised in the single-pass kernel (rows first rescaled by seeded
    factors in [0.25, 4]), with the gate and beta activations."""
    import torch
    import gated_delta_rule_14_amd as gdn
    import oracle
    from oracle import activation as act
    from parity_util import TOL, rel_err, to_dev
    from test_gpu_l2norm import _normalised, _rescale
    spec = gdn_synth.prefill_spec(1, B=2, T=600, H=3, A_range=WEAK, h0_std=0.05)
    print("case: l2norm", spec, flush=True)
    d = _rescale(gdn_synth.make_prefill(spec, 29, logits=True), 30)
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
