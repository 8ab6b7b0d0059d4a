"""The device-side check of packed offsets (GDN_ERR_BAD_SEQLENS through the
workspace word of gdn_seqlens_status_offset, read by the binding when
GDN_DEBUG is set).  Invalid offsets are clamped by the chunk-table kernel,
so every access stays in bounds; only the flag is checked here."""
import pytest
import torch

import gdn_synth
from parity_util import to_dev

pytestmark = pytest.mark.gpu

# three sequences over T = 100 tokens, as the valid offsets [0, 40, 70, 100]
BAD = {"decreasing": [0, 100, 50, 100], "not_from_0": [10, 40, 70, 100],
       "not_to_T": [0, 40, 70, 90]}


def _data(cid, dt, K, V):
    spec = gdn_synth.prefill_spec(cid, dtype=dt, H=2, K=K, V=V, rand_lengths=None,
                                  lengths=(40, 30, 30), h0_std=0.02)
    d = gdn_synth.make_prefill(spec, 130)
    return d, to_dev(d)


@pytest.mark.parametrize("cid,dt,K,V", [(1, "bf16", 128, 128), (0, "f32", 64, 64)])
def test_forward_offsets_check(gpu_lib, monkeypatch, cid, dt, K, V):
    import gated_delta_rule_14_amd as gdn
    monkeypatch.setenv("GDN_DEBUG", "1")
    d, x = _data(cid, dt, K, V)
    print("case: offsets check", dt, K, V, flush=True)
    gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                  cu_seqlens=x["cu_seqlens"])          # valid: no error
    for name, cu in BAD.items():
        print("  bad offsets:", name, flush=True)
        with pytest.raises(gdn.GdnError) as err:
            gdn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], d["scale"], h0=x["h0"],
                          cu_seqlens=torch.tensor(cu, dtype=torch.int64, device="cuda"))
        assert err.value.status == 8
    torch.cuda.synchronize()


def test_backward_offsets_check(gpu_lib, monkeypatch):
    import gated_delta_rule_14_amd as gdn
    monkeypatch.setenv("GDN_DEBUG", "1")
    d, x = _data(1, "bf16", 64, 64)
    gr = gdn_synth.make_grads(d, 130)
    print("case: backward offsets check", flush=True)
    kw = dict(h0=x["h0"], dht=gr["dht"].cuda())
    gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                  cu_seqlens=x["cu_seqlens"], **kw)
    with pytest.raises(gdn.GdnError) as err:
        gdn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], gr["do"].cuda(), d["scale"],
                      cu_seqlens=torch.tensor(BAD["decreasing"], dtype=torch.int64, device="cuda"),
                      **kw)
    assert err.value.status == 8
    torch.cuda.synchronize()
