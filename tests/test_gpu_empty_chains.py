"""Empty sequences on the single-pass route (bf16, scalar gate, K = V = 128):
a packed sequence of length 0 starting inside the first chunk of the packed
tokens, packs that start or end with empty sequences, a pack of empty
sequences only, and seq_len = 0 through the C ABI.  An empty sequence hands
its initial state through unchanged (ht = h0 bit for bit); the others meet
the parity bar against the fp64 oracle.  Every buffer load of an empty
sequence has a zero byte range, so nothing outside the inputs is read."""
import ctypes

import numpy as np
import pytest
import torch

import gdn_synth
import oracle
from parity_util import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths", [(0, 70, 0, 129), (0, 0, 5), (63, 0), (0, 1, 0, 64, 0)])
def test_packed_with_empty_sequences(gpu_lib, lengths):
    import gated_delta_rule_14_amd as gdn
    spec = gdn_synth.prefill_spec(2, H=3, rand_lengths=None, lengths=lengths, h0_std=0.05)
    print("case: empty chains, lengths", lengths, flush=True)
    d = gdn_synth.make_prefill(spec, 140)
    x = to_dev(d)
    o, ht = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.recurrent_forward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["scale"],
                                             h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    assert rel_err(o, o_ref) <= TOL["bf16"] and rel_err(ht, ht_ref) <= TOL["bf16"]
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(ht[n].cpu(), d["h0"][n]), n


def _abi_call(desc, q, k, v, beta, g, h0, cu, o, ht, ws):
    import gated_delta_rule_14_amd as gdn
    from gated_delta_rule_14_amd import _binding as B
    lib = gdn.load()
    B._check(lib.gdn_chunk_fwd(ctypes.byref(desc), B._ptr(q), B._ptr(k), B._ptr(v), B._ptr(beta),
                               B._ptr(g), B._ptr(h0), B._ptr(cu), B._ptr(o), B._ptr(ht),
                               B._ptr(ws), ws.numel(), B._stream(None)))


@pytest.mark.parametrize("packed", [False, True])
def test_zero_tokens_through_the_abi(gpu_lib, packed):
    """seq_len = 0: every sequence is empty.  The tensors of zero tokens are
    stood in for by small allocated buffers (a zero-sized tensor has no
    address); the kernel reads none of them."""
    import gated_delta_rule_14_amd as gdn
    H, K, V = 4, 128, 128
    N = 3 if packed else 2
    print("case: seq_len 0, packed" if packed else "case: seq_len 0", flush=True)
    dev = "cuda"
    dummy = lambda dt: torch.zeros(64, dtype=dt, device=dev)  # noqa: E731
    q, k, v, o = (dummy(torch.bfloat16) for _ in range(4))
    beta, g = dummy(torch.float32), dummy(torch.float32)
    gen = torch.Generator().manual_seed(141)
    h0 = (0.05 * torch.randn(N, H, K, V, generator=gen)).to(dev)
    ht = torch.full_like(h0, float("nan"))
    cu = torch.zeros(N + 1, dtype=torch.int64, device=dev) if packed else None
    desc = gdn.FwdDesc(1 if packed else N, 0, H, K, V, N if packed else 0, 64, 1, 0, K ** -0.5, 0)
    ws = torch.zeros(gdn.workspace_bytes(desc), dtype=torch.uint8, device=dev)
    _abi_call(desc, q, k, v, beta, g, h0, cu, o, ht, ws)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0)
    assert gdn.sync_status(desc, ws) == 0
    if packed:
        gdn.seqlens_status(desc, ws)      # [0, 0, 0, 0] is valid
    assert torch.count_nonzero(o).item() == 0   # nothing written to the stand-in output
