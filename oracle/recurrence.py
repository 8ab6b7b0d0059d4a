"""TEST INFRASTRUCTURE ONLY: Python face of the fp64 token recurrence.

The arithmetic lives in gdn_recurrence.c (plain C, fp64, OpenMP over the
independent (sequence, head) pairs).  This file only converts arrays to fp64,
checks shapes and calls it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        f = lib.oracle_gdn_forward
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      P, P, P, P, P, ctypes.c_int, ctypes.c_double, P, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def as_f64(x) -> np.ndarray:
    """Upcast a torch tensor or array (bf16/f32/f64) to a C-contiguous fp64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().to(dtype=__import__("torch").float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrent_forward(q, k, v, beta, g, scale, h0=None, cu_seqlens=None,
                      gate="scalar", threads: int = 0, want_state: bool = True):
    """Token-by-token gated delta rule in fp64.

    Shapes follow the library: q, k [B, T, H, K]; v [B, T, H, V];
    beta [B, T, H]; g [B, T, H] (scalar gate) or [B, T, H, K] (per-key gate);
    h0 [N, H, K, V] or None.  With cu_seqlens (int64 [N+1]) B must be 1 and
    the T axis holds the packed sequences.  Returns (o [B,T,H,V], ht [N,H,K,V]).
    """
    q, k, v, beta, g = (as_f64(x) for x in (q, k, v, beta, g))
    h0 = as_f64(h0)
    B, T, H, K = q.shape
    V = v.shape[-1]
    per_key = gate == "per_key"
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
    N = len(cu) - 1
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch")
    if g.shape != (q.shape if per_key else q.shape[:3]):
        raise ValueError("gate shape mismatch")
    if h0 is not None and h0.shape != (N, H, K, V):
        raise ValueError("h0 shape mismatch")
    o = np.zeros((B, T, H, V), dtype=np.float64)
    ht = np.zeros((N, H, K, V), dtype=np.float64) if want_state else None
    rc = _load().oracle_gdn_forward(N, _ptr(cu), H, K, V, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(beta), _ptr(g), int(per_key), float(scale),
                                    _ptr(h0), _ptr(o), _ptr(ht), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_forward failed with %d" % rc)
    return o, ht


def recurrent_step(q, k, v, beta, g, scale, state, gate="scalar", threads: int = 0):
    """One decode token for N independent sequences (fp64).

    q, k [N, H, K]; v [N, H, V]; beta [N, H]; g [N, H] or [N, H, K];
    state [N, H, K, V].  Returns (o [N, H, V], new_state).
    """
    q, k, v, beta, g, state = (as_f64(x) for x in (q, k, v, beta, g, state))
    N = q.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    o, ht = recurrent_forward(q[None], k[None], v[None], beta[None], g[None], scale,
                              h0=state, cu_seqlens=cu, gate=gate, threads=threads)
    return o[0], ht
