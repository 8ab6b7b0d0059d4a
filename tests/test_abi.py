"""The C ABI on the CPU: the library loads, exports what include/gdn.h
declares, and rejects bad arguments before launching anything (every call
below fails validation, so no GPU is touched)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_14_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return gdn.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gdn.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == gdn.ABI_VERSION
    for code, name in gdn._binding.STATUS.items():
        assert lib.gdn_status_str(code).decode() == name
    assert lib.gdn_status_str(99).decode() == "GDN_ERR_UNKNOWN"


def _desc(**kw):
    d = dict(batch=2, seq_len=256, num_heads=4, key_dim=128, value_dim=128, num_seqs=0, chunk=64,
             qkv_dtype=1, gate=0, scale=0.088)
    d.update(kw)
    return gdn.FwdDesc(**d)


def _status(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(chunk=48), 4), (dict(chunk=128), 4), (dict(chunk=8), 4), (dict(key_dim=96), 4), (dict(value_dim=256), 4),
    (dict(qkv_dtype=7), 3), (dict(gate=5), 3), (dict(batch=0), 2), (dict(num_heads=0), 2),
    (dict(seq_len=-1), 2), (dict(qkv_dtype=0, gate=1, key_dim=128), 4),
    (dict(batch=2, num_seqs=3), 2), (dict(num_heads=4, num_v_heads=6), 2),
    (dict(num_v_heads=-1), 2),
])
def test_descriptor_errors(lib, kw, code):
    n = ctypes.c_size_t()
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(_desc(**kw)), ctypes.byref(n)) == code
    assert lib.gdn_last_error().decode() != ""


def test_workspace_size_and_layout(lib):
    d = _desc()
    L = gdn.workspace_layout(d)
    assert L.max_chunks == 2 * 4
    blocks = 4 * L.max_chunks
    assert L.w - L.gcum >= blocks * 64 * 4
    assert L.u - L.w >= blocks * 64 * 128 * 2
    assert L.total >= L.chunks
    offs = [L.gcum, L.w, L.u, L.qs, L.ks, L.aqk, L.ainv, L.chunks, L.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    # the two-stage path (here fp32) needs the whole layout; the fused path
    # (bf16, scalar gate, K and V each 64 or 128) only the per-sequence records
    assert gdn.workspace_bytes(_desc(qkv_dtype=0)) == gdn.workspace_layout(_desc(qkv_dtype=0)).total
    assert gdn.workspace_bytes(_desc(gate=1)) == gdn.workspace_layout(_desc(gate=1)).total
    # (then 256 bytes for the synchronisation status word)
    assert gdn.workspace_bytes(d) == 256 + 256
    assert gdn.workspace_bytes(_desc(batch=1, seq_len=300, num_seqs=40)) == 768 + 256
    # packed: one extra chunk slot per sequence
    P = gdn.workspace_layout(_desc(batch=1, seq_len=300, num_seqs=3))
    assert P.max_chunks == 5 + 3


FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 4)


def _fwd(lib, d, q=FAKE, o=FAKE, ws=FAKE, wsb=1 << 40, cu=None, h0=None):
    return lib.gdn_chunk_fwd(ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, h0, cu, o, None, ws,
                             wsb, None)


def test_chunk_fwd_rejects_before_launch(lib):
    d = _desc()
    assert _fwd(lib, d, q=None) == 1
    assert _fwd(lib, d, o=None) == 1
    assert _fwd(lib, d, ws=None) == 1
    assert _fwd(lib, d, q=MIS) == 6
    assert _fwd(lib, d, h0=ctypes.c_void_p((1 << 20) + 2)) == 6
    assert _fwd(lib, d, ws=ctypes.c_void_p((1 << 20) + 64)) == 6
    assert _fwd(lib, d, wsb=128) == 5
    assert _fwd(lib, d, wsb=256) == 5                               # no room for the status word
    assert _fwd(lib, _desc(qkv_dtype=0), wsb=1024) == 5
    assert _fwd(lib, _desc(batch=2, num_seqs=2), cu=FAKE) == 2      # packed needs B == 1
    assert _fwd(lib, _desc(batch=1), cu=FAKE) == 2                  # packed needs num_seqs
    assert lib.gdn_chunk_intra(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               1 << 40, 0, None) == 1
    assert lib.gdn_chunk_scan(ctypes.byref(d), None, None, None, None, FAKE, 1 << 40, None) == 1
    assert lib.gdn_chunk_scan(ctypes.byref(d), None, None, FAKE, None, FAKE, 1024, None) == 5


def test_step_rejects_before_launch(lib):
    d = gdn.StepDesc(4, 2, 128, 128, 1, 0, 0.1)
    args = [FAKE] * 7
    assert lib.gdn_recurrent_step(ctypes.byref(d), None, *args[1:], None) == 1
    assert lib.gdn_recurrent_step(ctypes.byref(d), ctypes.c_void_p(3), *args[1:], None) == 6
    assert lib.gdn_recurrent_step(ctypes.byref(d), *args[:5], MIS, args[6], None) == 6
    bad = gdn.StepDesc(4, 2, 96, 128, 1, 0, 0.1)
    assert lib.gdn_recurrent_step(ctypes.byref(bad), *args, None) == 4
    bad = gdn.StepDesc(4, 2, 128, 128, 9, 0, 0.1)
    assert lib.gdn_recurrent_step(ctypes.byref(bad), *args, None) == 3


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        gdn.chunk_fwd(q, q, q, torch.zeros(1, 64, 1), torch.zeros(1, 64, 1))


def test_activation_rejects_before_launch(lib):
    """gdn_chunk_fwd_act / gdn_recurrent_step_act check the activation
    arguments before anything else is launched."""
    d = _desc()
    odd = ctypes.c_void_p((1 << 20) + 2)

    def fwd(flags, A_log, dt_bias):
        a = gdn.Activation(flags, A_log, dt_bias)
        return lib.gdn_chunk_fwd_act(ctypes.byref(d), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None, None, FAKE, None, FAKE, 1 << 40, None)

    def step(flags, A_log, dt_bias):
        s = gdn.StepDesc(4, 2, 128, 128, 1, 0, 0.1)
        a = gdn.Activation(flags, A_log, dt_bias)
        return lib.gdn_recurrent_step_act(ctypes.byref(s), ctypes.byref(a), *([FAKE] * 7), None)

    for fn in (fwd, step):
        assert fn(16, None, None) == 4           # unknown bit
        assert fn(4, None, None) == 4            # NEG_EIG without BETA_SIGMOID
        assert fn(1, None, FAKE) == 1            # GATE needs A_log
        assert fn(1 | 2, FAKE, None) == 1        # ... and dt_bias
        assert fn(1, odd, FAKE) == 6             # 4-byte alignment
        assert lib.gdn_last_error().decode() != ""


def test_chunk_bwd_rejects_before_launch(lib):
    """The backward's shape limits and argument checks fail before any launch."""
    n = ctypes.c_size_t()
    ws = lambda d: lib.gdn_chunk_bwd_workspace(ctypes.byref(d), ctypes.byref(n))  # noqa: E731
    assert ws(_desc()) == 0 and n.value > 0
    base = n.value
    assert ws(_desc(gate=1)) == 0                       # the per-key gate, bf16
    assert n.value > base                               # (its gate is per channel)
    assert ws(_desc(gate=1, qkv_dtype=0, key_dim=64, value_dim=64)) == 4   # ... bf16 only
    assert ws(_desc(num_v_heads=4)) == 0                # H_V == H
    base = n.value
    assert ws(_desc(num_v_heads=8)) == 0                # grouped value heads
    assert n.value > base                               # (room for the per-head dq, dk terms)
    assert ws(_desc(num_v_heads=6)) == 2                # not a multiple of H
    assert ws(_desc(qkv_dtype=0)) == 4                  # fp32 needs K = V = 64
    assert ws(_desc(qkv_dtype=0, key_dim=64, value_dim=64)) == 0
    assert ws(_desc(chunk=48)) == 4
    assert ws(_desc(chunk=32)) == 4 and ws(_desc(chunk=16)) == 4  # only the 64-token tiling
    # the workspace grows with the per-chunk states: above the forward layout
    assert n.value > gdn.workspace_layout(_desc(qkv_dtype=0, key_dim=64, value_dim=64)).total
    d = _desc()

    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, h0=None, cu=None, do=FAKE, dht=None,
                 dq=FAKE, dk=FAKE, dv=FAKE, dbeta=FAKE, dg=FAKE, dh0=None, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.gdn_chunk_bwd(ctypes.byref(kw.pop("desc", d)), a["q"], a["k"], a["v"], a["beta"],
                                 a["g"], a["h0"], a["cu"], a["do"], a["dht"], a["dq"], a["dk"],
                                 a["dv"], a["dbeta"], a["dg"], a["dh0"], a["ws"], a["wsb"], None)
    for name in ("q", "do", "dq", "dk", "dv", "dbeta", "dg", "ws"):
        assert bwd(**{name: None}) == 1, name
    for name in ("q", "do", "dq", "dv"):
        assert bwd(**{name: MIS}) == 6, name
    assert bwd(dht=ctypes.c_void_p((1 << 20) + 2)) == 6
    assert bwd(ws=ctypes.c_void_p((1 << 20) + 64)) == 6
    assert bwd(wsb=1024) == 5
    assert bwd(desc=_desc(gate=1, qkv_dtype=0, key_dim=64, value_dim=64)) == 4   # per-key: bf16
    assert bwd(desc=_desc(batch=1), cu=FAKE) == 2
    assert lib.gdn_last_error().decode() != ""


def test_chunk_bwd_act_rejects_before_launch(lib):
    """gdn_chunk_bwd_act checks the activation and its extra outputs before
    any launch."""
    d = _desc()
    odd = ctypes.c_void_p((1 << 20) + 2)

    def bwd(flags, A_log=FAKE, dt_bias=FAKE, dA_log=FAKE, ddt_bias=FAKE, desc=d):
        a = gdn.Activation(flags, A_log, dt_bias)
        return lib.gdn_chunk_bwd_act(ctypes.byref(desc), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     None, dA_log, ddt_bias, FAKE, 1 << 40, None)
    assert bwd(16) == 4                          # unknown bit
    assert bwd(4) == 4                           # NEG_EIG without BETA_SIGMOID
    assert bwd(1, A_log=None) == 1               # GATE needs A_log, dt_bias
    assert bwd(1, dA_log=None) == 1              # ... and the dA_log, ddt_bias outputs
    assert bwd(1 | 2, ddt_bias=None) == 1
    assert bwd(1, dA_log=odd) == 6
    assert bwd(1, desc=_desc(gate=1, qkv_dtype=0, key_dim=64, value_dim=64)) == 4   # per-key: bf16
    assert lib.gdn_last_error().decode() != ""


def test_l2norm_flag_and_workspace(lib):
    """GDN_ACT_QK_L2NORM is a known bit and runs on either route, so the
    workspace does not depend on it; an unknown bit is refused before
    anything else."""
    d = _desc()
    n = ctypes.c_size_t()

    def ws(flags, desc=d):
        a = gdn.Activation(flags, None, None)
        return lib.gdn_chunk_fwd_workspace_act(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(n))
    assert ws(0) == 0 and n.value == gdn.workspace_bytes(d) == 512
    assert ws(8) == 0 and n.value == 512
    f32 = _desc(qkv_dtype=0)
    assert ws(8, f32) == 0 and n.value == gdn.workspace_layout(f32).total
    assert ws(16) == 4
    assert lib.gdn_chunk_fwd_workspace_act(ctypes.byref(d), None, ctypes.byref(n)) == 0
    assert n.value == 512
    # the two-stage route with the flag still checks its workspace
    a = gdn.Activation(8, None, None)
    assert lib.gdn_chunk_fwd_act(ctypes.byref(f32), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None, None, FAKE, None, FAKE, 256, None) == 5


def test_chunk_sizes(lib):
    """Only the 64-token tiling is built: chunk 16 and 32 are refused with
    GDN_ERR_UNSUPPORTED by every entry point, before any launch."""
    n = ctypes.c_size_t()
    L = gdn.WorkspaceLayout()
    a = gdn.Activation(0, None, None)
    for c in (16, 32):
        for kw in (dict(), dict(qkv_dtype=0), dict(gate=1)):
            d = _desc(chunk=c, **kw)
            assert lib.gdn_chunk_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 4
            assert lib.gdn_chunk_fwd_workspace_act(ctypes.byref(d), ctypes.byref(a), ctypes.byref(n)) == 4
            assert lib.gdn_workspace_layout_of(ctypes.byref(d), ctypes.byref(L)) == 4
            assert _fwd(lib, d) == 4
            assert lib.gdn_chunk_fwd_act(ctypes.byref(d), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE,
                                         FAKE, None, None, FAKE, None, FAKE, 1 << 40, None) == 4
            assert lib.gdn_chunk_intra(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                       FAKE, 1 << 40, 0, None) == 4
            assert lib.gdn_chunk_scan(ctypes.byref(d), None, None, FAKE, None, FAKE, 1 << 40,
                                      None) == 4
            assert "64-token" in lib.gdn_last_error().decode()
        d = _desc(chunk=c)
        assert lib.gdn_chunk_bwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 4
        assert lib.gdn_chunk_bwd(ctypes.byref(d), *([FAKE] * 5), None, None, FAKE, None,
                                 *([FAKE] * 5), None, FAKE, 1 << 40, None) == 4
        assert lib.gdn_sync_status_offset(ctypes.byref(d), None, ctypes.byref(n)) == 4


def test_sync_status_offset(lib):
    """The single-pass kernel's synchronisation status word: inside the
    workspace it is sized for, after the packed-input records and their
    check word; shapes that run the two-stage route have none."""
    off = ctypes.c_size_t()

    def where(d, act=None):
        return lib.gdn_sync_status_offset(ctypes.byref(d), ctypes.byref(act) if act else None,
                                          ctypes.byref(off))
    d = _desc()
    assert where(d) == 0 and off.value == 256 and off.value + 4 <= gdn.workspace_bytes(d)
    p = _desc(batch=1, seq_len=300, num_seqs=40)
    assert where(p) == 0 and off.value == 768 and off.value + 4 <= gdn.workspace_bytes(p)
    so = ctypes.c_size_t()
    assert lib.gdn_seqlens_status_offset(ctypes.byref(p), None, 0, ctypes.byref(so)) == 0
    assert so.value + 4 <= off.value                            # the two words do not overlap
    assert where(d, gdn.Activation(8, None, None)) == 0 and off.value == 256
    assert where(_desc(qkv_dtype=0)) == 4                       # two stages: no waits
    assert where(_desc(gate=1)) == 4
    assert where(_desc(key_dim=64)) == 0 and off.value == 256    # the single-pass kernel at K = 64 too
    assert lib.gdn_sync_status_offset(ctypes.byref(d), None, None) == 1
    assert gdn.sync_status_offset(d) == 256 and gdn.sync_status_offset(_desc(gate=1)) is None


def test_seqlens_status_offset(lib):
    """Where a packed call leaves its check of cu_seqlens: after the
    per-sequence records, inside the workspace the call is sized for."""
    off = ctypes.c_size_t()

    def where(d, act=None, backward=0):
        return lib.gdn_seqlens_status_offset(ctypes.byref(d), ctypes.byref(act) if act else None,
                                             backward, ctypes.byref(off))
    d = _desc(batch=1, seq_len=300, num_seqs=5)                 # the single-pass kernel's shape
    assert where(d) == 0 and off.value == 5 * 16
    assert off.value + 4 <= gdn.workspace_bytes(d)
    d2 = _desc(batch=1, seq_len=300, num_seqs=5, qkv_dtype=0)   # two stages
    assert where(d2) == 0 and off.value == gdn.workspace_layout(d2).seqs + 5 * 16
    assert off.value + 4 <= gdn.workspace_bytes(d2)
    a8 = gdn.Activation(8, None, None)                          # L2 flag: the same route
    assert where(d, a8) == 0 and off.value == 5 * 16
    assert where(d, backward=1) == 0 and off.value % 16 == 0
    assert off.value + 4 <= gdn.bwd_workspace_bytes(d)
    assert where(_desc()) == 2                                  # not packed
    assert lib.gdn_seqlens_status_offset(ctypes.byref(d), None, 0, None) == 1
    assert lib.gdn_status_str(8).decode() == "GDN_ERR_BAD_SEQLENS"
