"""Seeded synthetic workloads for the gated delta rule forward pass.

This module only draws random inputs; it contains none of the method's
arithmetic.  Both the HIP path and the fp64 oracle consume what it returns,
so the two always see bit-identical values.

Distributions follow the gate parameterisation of the page
"Gated Delta Network（GDN）", §3.1 (eq. 5): beta = sigmoid(.),
log alpha = -A * softplus(. + b) with a per-head magnitude A, and q, k
L2-normalised per token and head (§5 of the same page; the
"TileLang 实战：KDA 从零到一--Gated DeltaNet" page, §0, states the unit-norm
precondition).

Recipe.  A root numpy PCG64 stream seeded with `seed` draws
  1. A_h ~ U(lo, hi), one per head (fp64), then
  2. (packed workload only) the sequence lengths.
Every bulk tensor is then drawn in blocks of at most BLOCK tokens, block j of
tensor `name` of sequence n from its own PCG64 stream seeded with
SeedSequence([seed, n, TAG[name], j]) -- so blocks can be drawn on several
threads and the result does not depend on the thread count:
  q, k, v: float32 standard normals; beta noise, gate noise: fp64 standard
  normals; the initial state (if any): float32 N(0, std^2), one stream per
  sequence.
q and k are L2-normalised per (token, head) with fp64 accumulation and then
rounded (round-to-nearest-even) to the storage dtype; beta, g and states are
stored as float32.  The oracle receives these stored values upcast to fp64.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

__all__ = ["PrefillSpec", "DecodeSpec", "PREFILL", "DECODE", "make_prefill", "make_grads",
           "make_decode", "prefill_spec", "draw_lengths", "flops_per_token_head",
           "bwd_flops_per_token_head"]


@dataclass(frozen=True)
class PrefillSpec:
    name: str
    dtype: str                 # "f32" or "bf16" for q/k/v/o
    B: int
    T: int                     # tokens per sequence (ignored when lengths given)
    H: int
    K: int
    V: int
    chunk: int = 64
    gate: str = "scalar"       # "scalar" (GDN) or "per_key" (KDA)
    A_range: tuple = (1.0, 16.0)
    h0_std: Optional[float] = None     # None -> no initial state (zeros)
    lengths: Optional[tuple] = None    # packed mode: explicit lengths
    rand_lengths: Optional[tuple] = None  # packed mode: (count, lo, hi, tail)
    gate_shift: float = 0.5
    scale: Optional[float] = None      # default 1/sqrt(K)


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    dtype: str
    N: int
    H: int
    K: int
    V: int
    steps: int = 64
    gate: str = "scalar"
    A_range: tuple = (1.0, 16.0)
    state_std: float = 0.02
    gate_shift: float = 0.5
    scale: Optional[float] = None


# The five workloads.  Sizes are those of the gated delta rule pages'
# setting (d_k = d_v = 128, chunk 64; "Gated Delta Network（GDN）" §4.1(d)
# limits chunk to {16, 32, 64} and head dims to <= 256).
PREFILL = {
    0: PrefillSpec("tiny-gdn-f32", "f32", B=1, T=256, H=1, K=64, V=64,
                   A_range=(0.01, 1.0), h0_std=None),
    1: PrefillSpec("gdn-prefill-bf16-B4-T4096-H16-d128", "bf16", B=4, T=4096,
                   H=16, K=128, V=128, h0_std=0.02),
    2: PrefillSpec("gdn-varlen-bf16-N16-H32-d128", "bf16", B=1, T=0, H=32,
                   K=128, V=128, h0_std=None,
                   rand_lengths=(15, 128, 8192, 65536)),
    3: PrefillSpec("kda-prefill-bf16-B2-T8192-H16-d128", "bf16", B=2, T=8192,
                   H=16, K=128, V=128, gate="per_key", h0_std=None),
}
DECODE = {
    4: DecodeSpec("gdn-decode-f32state-N256-H32-d128", "bf16", N=256, H=32,
                  K=128, V=128, steps=64),
}


def prefill_spec(cid: int, **overrides) -> PrefillSpec:
    """Workload `cid` with some fields replaced (smaller test sizes)."""
    return replace(PREFILL[cid], **overrides)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _draw_lengths(rng, spec: PrefillSpec):
    if spec.lengths is not None:
        return [int(x) for x in spec.lengths]
    if spec.rand_lengths is not None:
        cnt, lo, hi, tail = spec.rand_lengths
        ls = [int(x) for x in rng.integers(lo, hi + 1, size=cnt)]
        if tail:
            ls.append(int(tail))
        return ls
    return None


BLOCK = 4096
TAG = {"q": 1, "k": 2, "v": 3, "beta": 4, "g": 5, "h0": 6, "do": 7, "dht": 8}
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1)))


def _stream(seed, n, name, j):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, n, TAG[name], j])))


def _blocked(seed, n, name, L, tail_shape, kind):
    """Draw a [L, *tail_shape] tensor block by block (see the recipe)."""
    dt = np.float32 if kind == "f32" else np.float64
    out = np.empty((L,) + tuple(tail_shape), dtype=dt)
    jobs = [(j, j * BLOCK, min(L, (j + 1) * BLOCK)) for j in range((L + BLOCK - 1) // BLOCK)]

    def run(job):
        j, a, b = job
        _stream(seed, n, name, j).standard_normal(out[a:b].shape, dtype=dt, out=out[a:b])
    if len(jobs) > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(run, jobs))
    else:
        for jb in jobs:
            run(jb)
    return out


def _unit_cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    """L2-normalise the last axis (fp64 accumulation), round to `dtype`."""
    t = torch.from_numpy(x).double()
    t = t / t.pow(2).sum(-1, keepdim=True).sqrt()
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def make_prefill(spec, seed: int = None, logits: bool = False) -> dict:
    """Draw one prefill workload.

    Returns a dict of CPU torch tensors in the layouts of the library:
      q, k [B, T, H, K], v [B, T, H, V] (dtype of the spec),
      beta [B, T, H] f32, g [B, T, H] or [B, T, H, K] f32 (natural-log gate),
      h0 [N, H, K, V] f32 or None, cu_seqlens int64 [N+1] or None,
    plus 'scale', 'chunk', 'gate', 'lengths', 'spec'.
    Packed workloads are returned with B = 1 and T = total tokens.
    With logits=True, beta and g hold the raw draws (the logits before the
    sigmoid and before the gate's softplus) and the dict adds 'A_log' [H] and
    'dt_bias' ([H], or [H, K] for the per-key gate) f32: the same draws as
    without it.
    """
    if isinstance(spec, int):
        spec = PREFILL[spec]
    if seed is None:
        seed = 0
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.uniform(spec.A_range[0], spec.A_range[1], size=spec.H)
    lengths = _draw_lengths(rng, spec)
    packed = lengths is not None
    if not packed:
        lengths = [spec.T] * spec.B
    H, K, V = spec.H, spec.K, spec.V
    per_key = spec.gate == "per_key"
    qs, ks, vs, bs, gs = [], [], [], [], []
    for n, L in enumerate(lengths):
        qs.append(_unit_cast(_blocked(seed, n, "q", L, (H, K), "f32"), spec.dtype))
        ks.append(_unit_cast(_blocked(seed, n, "k", L, (H, K), "f32"), spec.dtype))
        vs.append(_cast(_blocked(seed, n, "v", L, (H, V), "f32"), spec.dtype))
        bn = _blocked(seed, n, "beta", L, (H,), "f64")
        gn = _blocked(seed, n, "g", L, (H, K) if per_key else (H,), "f64")
        if logits:
            bs.append(torch.from_numpy(bn.astype(np.float32)))
            gs.append(torch.from_numpy(gn.astype(np.float32)))
            continue
        bs.append(torch.from_numpy(_sigmoid(bn).astype(np.float32)))
        a = A[None, :, None] if per_key else A[None, :]
        gs.append(torch.from_numpy((-a * _softplus(gn + spec.gate_shift)).astype(np.float32)))
    N = len(lengths)
    h0 = None
    if spec.h0_std is not None:
        h0 = torch.empty((N, H, K, V), dtype=torch.float32)
        for n in range(N):
            st = _stream(seed, n, "h0", 0)
            h0[n] = torch.from_numpy(st.standard_normal((H, K, V), dtype=np.float32)
                                     * np.float32(spec.h0_std))
    if packed:
        cat = lambda xs: torch.cat(xs, 0).unsqueeze(0)
        cu = torch.zeros(N + 1, dtype=torch.int64)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    else:
        cat = lambda xs: torch.stack(xs, 0)
        cu = None
    scale = spec.scale if spec.scale is not None else 1.0 / math.sqrt(K)
    out = dict(q=cat(qs), k=cat(ks), v=cat(vs), beta=cat(bs), g=cat(gs),
               h0=h0, cu_seqlens=cu, scale=float(scale), chunk=spec.chunk,
               gate=spec.gate, lengths=lengths, spec=spec)
    if logits:
        out["A_log"] = torch.from_numpy(np.log(A).astype(np.float32))
        out["dt_bias"] = torch.full((H, K) if per_key else (H,), spec.gate_shift, dtype=torch.float32)
    return out


def make_grads(d: dict, seed: int = None, dht_std: Optional[float] = 0.1) -> dict:
    """Upstream gradients for a backward call on the prefill workload d (as
    returned by make_prefill): 'do' shaped like v, float32 standard normals
    rounded to the q/k/v dtype, drawn per sequence and block like v (tag
    'do'); 'dht' [N, H, K, V] float32 N(0, dht_std^2), one stream per
    sequence (tag 'dht'), or None when dht_std is None."""
    spec = d["spec"]
    seed = 0 if seed is None else seed
    lengths = d["lengths"]
    H, K, V = spec.H, spec.K, spec.V
    parts = [_cast(_blocked(seed, n, "do", L, (H, V), "f32"), spec.dtype)
             for n, L in enumerate(lengths)]
    do = torch.cat(parts, 0).unsqueeze(0) if d["cu_seqlens"] is not None else torch.stack(parts, 0)
    dht = None
    if dht_std is not None:
        dht = torch.empty((len(lengths), H, K, V), dtype=torch.float32)
        for n in range(len(lengths)):
            dht[n] = torch.from_numpy(_stream(seed, n, "dht", 0).standard_normal(
                (H, K, V), dtype=np.float32) * np.float32(dht_std))
    return dict(do=do, dht=dht)


def draw_lengths(spec, seed: int = None):
    """Only the sequence lengths of a packed workload (cheap)."""
    if isinstance(spec, int):
        spec = PREFILL[spec]
    rng = np.random.Generator(np.random.PCG64(0 if seed is None else seed))
    rng.uniform(spec.A_range[0], spec.A_range[1], size=spec.H)
    return _draw_lengths(rng, spec)


def make_decode(spec, seed: int = None, logits: bool = False) -> dict:
    """Draw a decode workload: an initial state plus `steps` tokens.

    Returns state [N, H, K, V] f32 and per-step q, k [S, N, H, K],
    v [S, N, H, V] (dtype), beta [S, N, H] f32, g [S, N, H] (or [..., K]).
    Step s plays the role of sequence index s in the block recipe; the state
    is drawn in blocks of BLOCK sequences under the index S (= steps).
    logits=True: raw beta and g logits plus 'A_log' and 'dt_bias', as in
    make_prefill.
    """
    if isinstance(spec, int):
        spec = DECODE[spec]
    if seed is None:
        seed = 4
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.uniform(spec.A_range[0], spec.A_range[1], size=spec.H)
    S, N, H, K, V = spec.steps, spec.N, spec.H, spec.K, spec.V
    per_key = spec.gate == "per_key"
    q = np.stack([_blocked(seed, s, "q", N, (H, K), "f32") for s in range(S)])
    k = np.stack([_blocked(seed, s, "k", N, (H, K), "f32") for s in range(S)])
    v = np.stack([_blocked(seed, s, "v", N, (H, V), "f32") for s in range(S)])
    bn = np.stack([_blocked(seed, s, "beta", N, (H,), "f64") for s in range(S)])
    gn = np.stack([_blocked(seed, s, "g", N, (H, K) if per_key else (H,), "f64")
                   for s in range(S)])
    a = A[None, None, :, None] if per_key else A[None, None, :]
    state = _blocked(seed, S, "h0", N, (H, K, V), "f32") * np.float32(spec.state_std)
    scale = spec.scale if spec.scale is not None else 1.0 / math.sqrt(K)
    out = dict(q=_unit_cast(q, spec.dtype), k=_unit_cast(k, spec.dtype),
               v=_cast(v, spec.dtype),
               beta=torch.from_numpy(_sigmoid(bn).astype(np.float32)),
               g=torch.from_numpy((-a * _softplus(gn + spec.gate_shift)).astype(np.float32)),
               state=torch.from_numpy(state), scale=float(scale), gate=spec.gate,
               spec=spec)
    if logits:
        out["beta"] = torch.from_numpy(bn.astype(np.float32))
        out["g"] = torch.from_numpy(gn.astype(np.float32))
        out["A_log"] = torch.from_numpy(np.log(A).astype(np.float32))
        out["dt_bias"] = torch.full((H, K) if per_key else (H,), spec.gate_shift, dtype=torch.float32)
    return out


def flops_per_token_head(K: int, V: int, C: int) -> float:
    """Algorithmic MFMA flops per token-head of the chunked forward.

    Counted terms: the three K-by-V state products (V_new = U - W h, the
    state update and the inter-chunk read), the strictly-lower K K^T, W, U,
    the causal Q K^T (diagonal included), the intra-chunk read of V_new and
    the triangular inverse (C^2/3 per row).
    """
    return (6 * K * V + (C - 1) * K + (C + 1) * K + (C + 1) * V
            + (C + 1) * K + (C + 1) * V + C * C / 3.0)


def bwd_flops_per_token_head(K: int, V: int, C: int) -> float:
    """Algorithmic MFMA flops per token-head of the chunked backward, each
    product of its six steps counted once (2 flops per multiply-add,
    triangular operands at their average row length, as above):
      recompute: K K^T, the inverse, W, U, the causal Q K^T, V_new = U - W h
        and the state update (2 K V each);
      state-gradient recurrence: Ks dH, Qs^T dO, W^T dVn (2 K V each) and
        Aqk^T dO;
      per chunk: dO h^T, Vn dH^T, dVn h^T (2 K V each), the causal dO Vn^T,
        Pm K, Pm^T Q, T^T dVn, T^T dW, dVn V^T and dW K^T (full C x C),
        T^T dAinv T^T (two triangular C x C x C products) and the two
        strictly-lower dA K products.
    """
    kv = 16 * K * V
    k = ((C - 1) + 3 * (C + 1)          # K K^T, W, Q K^T
         + 2 * (C + 1) + (C + 1)        # Pm K, Pm^T Q, T^T dW
         + 2 * C + 2 * (C - 1)) * K     # dW K^T, dA K (both sides)
    v = (4 * (C + 1) + 2 * C) * V       # U, Aqk^T dO, dO Vn^T, T^T dVn, dVn V^T
    return float(kv + k + v + C * C / 3.0 + 2 * C * C)
