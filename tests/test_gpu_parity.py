"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on
seeded inputs, element by element.  Bar: max|o - o_ref| <= tol * max|o_ref|
(tol 1e-4 for fp32 q/k/v, 2e-2 for bf16 with fp32 accumulation); the final
state to the same relative bound."""
import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from parity_util import TOL, check, rel_err, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _spec(cid, **kw):
    return gdn_synth.prefill_spec(cid, **kw)


def _roundtrip(spec, seed, heads=None, **kw):
    d = gdn_synth.make_prefill(spec, seed)
    print("case:", spec, "seed", seed, flush=True)
    o, ht = run_gpu(d, **kw)
    o_ref, ht_ref = run_oracle(d, heads)
    return d, check(d, o, ht, o_ref, ht_ref, heads)


# ---------------------------------------------------------------- prefill
def test_tiny_fp32_workload(gpu_lib):
    """B=1, H=1, T=256, d=64, fp32, zero state (the small fp32 workload)."""
    _roundtrip(gdn_synth.PREFILL[0], 0)
    _roundtrip(gdn_synth.PREFILL[0], 100)


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_lengths(gpu_lib, T, dt):
    _roundtrip(_spec(1, dtype=dt, B=2, T=T, H=3, K=64, V=64), 7 + T)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64)])
def test_head_dims_with_state(gpu_lib, K, V):
    _roundtrip(_spec(1, B=2, T=300, H=2, K=K, V=V), 11)


def test_fp32_d128(gpu_lib):
    _roundtrip(_spec(1, dtype="f32", B=1, T=257, H=2, K=128, V=128), 12)


@pytest.mark.parametrize("dt,K", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_per_key_gate(gpu_lib, dt, K):
    _roundtrip(_spec(3, dtype=dt, B=2, T=333, H=2, K=K, V=128, h0_std=0.02), 13)


def test_packed_sequences(gpu_lib):
    spec = _spec(2, H=3, rand_lengths=None, lengths=(70, 1, 0, 129, 64, 300))
    _roundtrip(spec, 14)
    _roundtrip(_spec(2, H=3, rand_lengths=None, lengths=(65, 0, 200), h0_std=0.02), 15)


def test_packed_per_key(gpu_lib):
    _roundtrip(_spec(3, B=1, H=2, lengths=(100, 64, 3), rand_lengths=None), 16)


def test_no_final_state_and_in_place_carry(gpu_lib):
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(_spec(1, B=2, T=150, H=2), 17)
    x = to_dev(d)
    o1, ht1 = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"])
    o2, none = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                             output_final_state=False)
    assert none is None and torch.equal(o1, o2)
    carry = x["h0"].clone()
    o3, ht3 = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=carry,
                            ht=carry)
    torch.cuda.synchronize()
    assert ht3.data_ptr() == carry.data_ptr()
    assert torch.equal(o3, o1) and torch.equal(ht3, ht1)


def test_split_resume_and_determinism(gpu_lib):
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(_spec(1, B=1, T=320, H=2), 18)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"])
    o_b, ht_b = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"])
    assert torch.equal(o, o_b) and torch.equal(ht, ht_b)        # bitwise deterministic
    s = 128                                                     # split on a chunk boundary
    sl = lambda t, a, b: t[:, a:b].contiguous()
    o1, h1 = gdn.chunk_fwd(*(sl(x[n], 0, s) for n in ("q", "k", "v", "beta", "g")), d["scale"],
                           h0=x["h0"])
    o2, h2 = gdn.chunk_fwd(*(sl(x[n], s, 320) for n in ("q", "k", "v", "beta", "g")), d["scale"],
                           h0=h1)
    assert torch.equal(torch.cat([o1, o2], 1), o) and torch.equal(h2, ht)


# ------------------------------------------------------ intra-chunk stage
def _intra_case(spec, seed):
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(spec, seed)
    x = to_dev(d)
    r = gdn.chunk_intra(x["q"], x["k"], x["v"], x["beta"], x["g"], scale=d["scale"],
                        cu_seqlens=x.get("cu_seqlens"), gate=d["gate"])
    torch.cuda.synchronize()
    _, _, ref = oracle.chunked_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                                       h0=d.get("h0"), cu_seqlens=d.get("cu_seqlens"),
                                       gate=d["gate"], chunk=64, keep=True)
    return d, r, ref


@pytest.mark.parametrize("dt,gate", [("f32", "scalar"), ("bf16", "scalar"), ("bf16", "per_key")])
def test_intra_stage_matches_chunked_reference(gpu_lib, dt, gate):
    """k1-k3 against the chunked UT reference's per-chunk products."""
    spec = _spec(1, dtype=dt, B=2, T=150, H=2, K=64, V=128, gate=gate)
    d, r, ref = _intra_case(spec, 19)
    B, T, H = 2, 150, 2
    nt = 3
    tol = 1e-4 if dt == "f32" else 2e-2
    for b in range(B):
        for hh in range(H):
            for j in range(nt):
                c = b * nt + j
                n = min(64, T - 64 * j)
                sl = slice(64 * j, 64 * j + n)
                ai = r["ainv"][hh, c, :n, :n].double().cpu().numpy()
                ai_ref = ref["Ainv"][b, sl, hh, :n]
                assert rel_err(ai, ai_ref) < (1e-5 if dt == "f32" else 1e-4)
                for key, name in (("w", "W"), ("u", "U"), ("aqk", "Aqk")):
                    got = r[key][hh, c, :n].float().cpu().double().numpy()
                    want = ref[name][b, sl, hh]
                    if key == "aqk":
                        want = want[:, :64]
                        got = got[:, :64]
                    assert rel_err(got, want) < tol, (key, b, hh, j)
                # padded rows are zero
                assert float(r["w"][hh, c, n:].abs().max() if n < 64 else 0) == 0.0
                G = r["gcum"][hh, c, :n].double().cpu().numpy() / np.log2(np.e)
                G_ref = ref["G"][b, sl, hh]
                if gate == "per_key":
                    # only the last row is written: G at the chunk's last
                    # token (padded rows of a ragged chunk add nothing)
                    G = r["gcum"][hh, c, 63].double().cpu().numpy() / np.log2(np.e)
                    G_ref = G_ref[n - 1]
                assert np.max(np.abs(G - G_ref)) < 1e-4 * max(1, np.abs(G).max())


# ------------------------------------------------------- full-size workloads
def test_gdn_prefill_full_size(gpu_lib):
    """B=4, T=4096, H=16, d=128, bf16, nonzero initial state: every output."""
    _roundtrip(gdn_synth.PREFILL[1], 1)


def test_kda_prefill_full_size(gpu_lib):
    """B=2, T=8192, H=16, d=128, per-key gate, bf16: every output."""
    _roundtrip(gdn_synth.PREFILL[3], 3)


def test_varlen_prefill_full_size(gpu_lib):
    """16 packed sequences (one of 65536 tokens), H=32: every output of every
    head and every sequence.  The oracle runs on groups of 8 heads at a time
    (to bound host memory); the bar is taken over the whole output."""
    d = gdn_synth.make_prefill(gdn_synth.PREFILL[2], 2)
    print("case: packed full size, all heads", flush=True)
    o, ht = run_gpu(d)
    o = o.float().cpu()
    ht = ht.cpu()
    H = d["q"].shape[2]
    num = {"o": 0.0, "ht": 0.0}
    den = {"o": 0.0, "ht": 0.0}
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(h0 + 8, H)))
        o_ref, ht_ref = run_oracle(d, heads)
        for name, got, want in (("o", o[:, :, heads], o_ref), ("ht", ht[:, heads], ht_ref)):
            num[name] = max(num[name], float(np.abs(got.double().numpy() - want).max()))
            den[name] = max(den[name], float(np.abs(want).max()))
        print("  heads %d-%d done" % (heads[0], heads[-1]), flush=True)
    for name in ("o", "ht"):
        err = num[name] / den[name]
        print("  %s relative error %.2e" % (name, err), flush=True)
        assert np.isfinite(err) and err <= TOL["bf16"], (name, err)


# ------------------------------------------------------------------ decode
def _decode_case(spec, seed):
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_decode(spec, seed)
    print("case:", spec, "seed", seed, flush=True)
    x = to_dev(d)
    state = x["state"].clone()
    outs = []
    for s in range(spec.steps):
        outs.append(gdn.recurrent_step(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s],
                                       state, scale=d["scale"], gate=d["gate"]))
    torch.cuda.synchronize()
    o = torch.stack(outs).float().cpu()
    ref_state = oracle.as_f64(d["state"])
    tol = TOL[spec.dtype]
    for s in range(spec.steps):
        q, k, v, beta, g = (d[n][s] for n in ("q", "k", "v", "beta", "g"))
        o_ref, ref_state = oracle.recurrent_step(q, k, v, beta, g, d["scale"], ref_state,
                                                 gate=d["gate"])
        assert rel_err(o[s], o_ref) <= tol, ("step", s)
    assert rel_err(state.cpu(), ref_state) <= tol


@pytest.mark.parametrize("dt,gate,K,V", [("bf16", "scalar", 128, 128), ("f32", "scalar", 64, 64),
                                         ("bf16", "per_key", 128, 64), ("f32", "per_key", 64, 128)])
def test_decode_steps(gpu_lib, dt, gate, K, V):
    spec = gdn_synth.DecodeSpec("t", dt, N=5, H=3, K=K, V=V, steps=8, gate=gate)
    _decode_case(spec, 21)


def test_decode_full_size(gpu_lib):
    """256 sequences x 32 heads, 64 steps in place: the output of every
    sequence and head at every step, and the final state, against the oracle.
    The 64 steps of one sequence are its token recurrence over 64 tokens, so
    the oracle runs them as one 64-token sequence per (sequence, head) (the
    same function the single-step oracle calls, on all steps at once)."""
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.DECODE[4]
    d = gdn_synth.make_decode(spec, 4)
    print("case: decode full size, every sequence and step", flush=True)
    x = to_dev(d)
    state = x["state"].clone()
    outs = []
    for s in range(spec.steps):
        outs.append(gdn.recurrent_step(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s],
                                       state, scale=d["scale"], gate=d["gate"]))
    torch.cuda.synchronize()
    o = torch.stack(outs, 1).float().cpu()          # [N, steps, H, V]
    seq = [d[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "beta", "g")]
    o_ref, st_ref = oracle.recurrent_forward(*seq, d["scale"], h0=d["state"], gate=d["gate"])
    eo, es = rel_err(o, o_ref), rel_err(state, st_ref)
    print("  o relative error %.2e, state %.2e" % (eo, es), flush=True)
    assert eo <= TOL[spec.dtype] and es <= TOL[spec.dtype]
    # every step separately meets the bar too
    for s in range(spec.steps):
        assert rel_err(o[:, s], o_ref[:, s]) <= TOL[spec.dtype], ("step", s)


def test_stages_compose_to_forward(gpu_lib):
    """gdn_chunk_intra followed by gdn_chunk_scan (the two-stage path) meets
    the parity bar, like gdn_chunk_fwd (which runs the fused kernel for this
    shape), and the two agree with each other to the same bar."""
    import gated_delta_rule_14_amd as gdn
    d = gdn_synth.make_prefill(_spec(1, B=2, T=200, H=2), 22)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"])
    r = gdn.chunk_intra(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], store_ainv=False)
    o2 = torch.empty_like(o)
    ht2 = torch.empty_like(ht)
    gdn.chunk_scan(r["desc"], r["workspace"], o2, h0=x["h0"], ht=ht2)
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(d)
    check(d, o, ht, o_ref, ht_ref)
    check(d, o2, ht2, o_ref, ht_ref)
    check(d, o2, ht2, o.double().cpu().numpy(), ht.double().cpu().numpy())
