#!/usr/bin/env python3
"""Benchmark of the chunked gated delta rule forward on one MI355X.

A step is one pass of the whole prefill path (one gdn_chunk_fwd: for this
shape the fused kernel, which builds every intra-chunk product in LDS and
runs the state pass with the output in the same launch) over the GDN workload
B=4, T=4096, H=16, d_k=d_v=128, chunk 64, bf16 q/k/v with fp32 beta, gates
and states, inputs resident in HBM.  `value` is tokens/s (B*T tokens per
step).  The same run times the kernel of every step with HIP events on its
stream, the two-stage path (intra-chunk stage + state pass) for comparison,
the decode step (256 sequences x 32 heads, fp32 state in place, 64 steps),
the chunked backward on the prefill workload (gradients of q, k, v, beta, g
and h0 from seeded dO and dht), the per-key-gate (KDA) prefill B=2, T=8192,
H=16 (two-stage route) and its backward, the packed variable-length prefill
(16 sequences, 137 491 tokens, H=32; fused route), and the fp64 CPU oracle on
the host cores.

Every leg first runs its own call back to back for a fixed wall time
(--settle-s): the shader clock drops during the host's pauses (input
generation, the previous leg's host work) and needs a few milliseconds of
load to come back to its sustained rate, which a handful of warm-up launches
does not give.  Then W warm-up launches and the K timed ones.  The record
also carries the device (CU count, ROCm), the shader and memory clocks
sampled under the prefill's load, an Infinity-Cache-flushed median next to
the back-to-back prefill time, and the fp64 oracle timed on the host cores on
every workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-decode]
                  [--no-backward] [--no-kda] [--no-kda-backward] [--no-varlen]
                  [--no-variants]
                  [--only LEG]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gdn_synth  # noqa: E402

# MI355X published peaks
HBM_PEAK = 8.0e12            # bytes/s
BF16_PEAK = 2516.6e12        # dense MFMA flop/s (256 CU x 2.4 GHz x 4096)
METRIC = "GDN chunked-prefill tokens/s + % MFMA peak (H=16,d=128,T=4096); decode % HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_bytes(spec, n_seqs):
    """Algorithmic HBM bytes of one prefill pass, split by what must move
    them: the inputs q, k, v, beta, g (read by the intra-chunk stage, or by
    the fused kernel), and o, h0, ht (written / read by the state pass, or by
    the fused kernel)."""
    es = 2 if spec.dtype == "bf16" else 4
    th = spec.B * spec.T * spec.H
    gate = 4 * (spec.K if spec.gate == "per_key" else 1)
    intra = th * ((2 * spec.K + spec.V) * es + 4 + gate)
    state = 4 * spec.K * spec.V * spec.H * n_seqs
    scan = th * spec.V * es + state * (2 if spec.h0_std is not None else 1)
    return intra, scan


KERNEL_SOURCES = {"fused_kernel": ["k_fused.hip", "k_fused_body.hpp", "gdn_device.hpp"],
                  "intra_kernel": ["k_intra.hip", "gdn_device.hpp"],
                  "scan_kernel": ["k_scan.hip", "gdn_device.hpp"],
                  "step_kernel": ["k_step.hip", "gdn_device.hpp"],
                  "bwd_intra_kernel": ["k_intra.hip", "gdn_device.hpp"],
                  "bwd_state_scan_kernel": ["k_scan.hip", "gdn_device.hpp"],
                  "bwd_scan_kernel": ["k_bwd.hip", "gdn_device.hpp"],
                  "bwd_local_kernel": ["k_bwd.hip", "gdn_device.hpp"],
                  "kda_intra_kernel": ["k_intra.hip", "gdn_device.hpp"],
                  "kda_scan_kernel": ["k_scan.hip", "gdn_device.hpp"],
                  "kda_bwd_intra_kernel": ["k_intra.hip", "gdn_device.hpp"],
                  "kda_bwd_state_scan_kernel": ["k_scan.hip", "gdn_device.hpp"],
                  "kda_bwd_scan_kernel": ["k_bwd.hip", "gdn_device.hpp"],
                  "kda_bwd_local_kernel": ["k_bwd_kda.hip", "gdn_device.hpp"],
                  "varlen_fused_kernel": ["k_fused.hip", "k_fused_body.hpp", "gdn_device.hpp"]}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary
    (profiles/hbm_traffic.json, FETCH_SIZE + WRITE_SIZE scaled by a copy of
    known size), or None if the kernel's source changed since."""
    import hashlib
    path = os.path.join(HERE, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(HERE, "gated_delta_rule_14_amd", "csrc", f), "rb").read())
    return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha"] else None


def settle(fn, seconds):
    """Run fn() back to back for `seconds` of wall time, so that the GPU's
    clock is at its sustained rate when the timing starts."""
    t0 = time.perf_counter()
    while True:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


class ClockSampler:
    """Samples the shader (sclk) and memory (mclk) clocks with rocm-smi in a
    background thread while the GPU works; empty if the tool is absent."""

    def __init__(self):
        import threading
        self.samples, self.stop, self.th = [], False, threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        import subprocess
        # under a profiler its preloaded library would start with rocm-smi
        # (a Python script), initialise the GPU there and then exec the
        # interpreter; profiled runs do not report clocks
        if "rocprof" in os.environ.get("LD_PRELOAD", ""):
            return
        while not self.stop:
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                                   text=True, timeout=20)
                card = next(iter(json.loads(r.stdout).values()))
                mhz = lambda k: int(re.search(r"(\d+)", card[k]).group(1))  # noqa: E731
                self.samples.append((mhz("sclk clock speed:"), mhz("mclk clock speed:")))
            except Exception:
                return

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop = True
        self.th.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        sc = sorted(x[0] for x in self.samples)
        mc = sorted(x[1] for x in self.samples)
        return {"samples": len(sc), "sclk_mhz_min": sc[0], "sclk_mhz_median": sc[len(sc) // 2],
                "sclk_mhz_max": sc[-1], "mclk_mhz_min": mc[0], "mclk_mhz_max": mc[-1],
                "source": "rocm-smi --showclocks, sampled while the prefill leg ran back to back"}


def flushed_median(fn, reps, flush_bytes=512 << 20):
    """Median duration of fn() when a flush_bytes scratch write (larger than
    the 256 MB Infinity Cache) runs right before each launch, outside the
    timed events: fn's inputs then come from HBM."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r in range(reps):
        scratch.fill_(r & 0xff)
        ev[r][0].record()
        fn()
        ev[r][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
    del scratch
    return t[len(t) // 2]


def device_info():
    import platform
    p = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hbm_bytes": p.total_memory,
            "rocm": rocm, "torch_hip": torch.version.hip, "host_cpu": cpu,
            "host_affinity_cpus": len(os.sched_getaffinity(0)), "host": platform.machine()}


def events_time(fn, reps):
    """Average duration of fn() over reps back-to-back launches, from HIP
    events recorded on the current stream (the stream the kernels use)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def step_kernel_times(first, second, reps):
    """Average durations of first() and second() when launched alternately,
    as in a step, from HIP events recorded between the launches."""
    first()
    second()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * reps)]
    for r in range(reps):
        ev[3 * r].record()
        first()
        ev[3 * r + 1].record()
        second()
        ev[3 * r + 2].record()
    ev[-1].synchronize()
    a = sum(ev[3 * r].elapsed_time(ev[3 * r + 1]) for r in range(reps)) / reps / 1e3
    b = sum(ev[3 * r + 1].elapsed_time(ev[3 * r + 2]) for r in range(reps)) / reps / 1e3
    return a, b


def bench_prefill(args, gdn):
    spec = gdn_synth.PREFILL[1]
    log("generating", spec.name)
    d = gdn_synth.make_prefill(spec, 1)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, beta, g, h0 = (dev[n] for n in ("q", "k", "v", "beta", "g", "h0"))
    o = torch.empty_like(v)
    ht = torch.empty_like(h0)
    desc = gdn.fwd_desc(q, v, "scalar", 64, d["scale"])
    ws = torch.empty(gdn.workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    ws.zero_()

    def step():
        gdn.chunk_fwd(q, k, v, beta, g, d["scale"], h0=h0, o=o, ht=ht, workspace=ws)

    settle(step, args.settle_s)
    for _ in range(args.warmup):
        step()
    # timed region: wall clock around the K steps, and a HIP event pair on the
    # stream the kernel is launched on (one kernel per step, launched back to
    # back: the average launch duration is the pair's time over K)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    t_fused = ev[0].elapsed_time(ev[1]) / args.steps / 1e3
    log("prefill step %.1f us (fused kernel %.1f us)" % (dt * 1e6, t_fused * 1e6))
    # the single-pass kernel's synchronisation word: 0 unless a wait between
    # its waves gave up (results then wrong)
    sync_word = gdn.sync_status(desc, ws)
    if sync_word != 0:
        raise RuntimeError("the fused kernel reported a failed hand-off between its waves")
    t_flushed = flushed_median(step, 20)
    log("prefill with the Infinity Cache flushed before each call: %.1f us (median of 20)"
        % (t_flushed * 1e6))
    # the clocks under this leg's load, sampled after the timed region (the
    # sampler's last rocm-smi call leaves the GPU idle for a while)
    with ClockSampler() as clocks:
        settle(step, 1.0)

    # the two-stage path on the same inputs, for comparison: per-kernel
    # durations inside its step sequence (intra, scan, intra, ...)
    L = gdn.workspace_layout(desc)
    ws2 = torch.empty(L.total, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o)
    ht2 = torch.empty_like(ht)
    reps = max(args.steps, 10)
    two = (lambda: gdn.chunk_intra(q, k, v, beta, g, d["scale"], store_ainv=False, workspace=ws2,
                                   views=False),
           lambda: gdn.chunk_scan(desc, ws2, o2, h0=h0, ht=ht2))
    settle(lambda: (two[0](), two[1]()), args.settle_s)
    t_intra, t_scan = step_kernel_times(two[0], two[1], reps)
    del ws2
    log("two-stage path: intra %.1f us, scan %.1f us" % (t_intra * 1e6, t_scan * 1e6))

    b_in, b_out = prefill_bytes(spec, spec.B)
    b_all = b_in + b_out
    th = spec.B * spec.T * spec.H
    flops = gdn_synth.flops_per_token_head(spec.K, spec.V, spec.chunk) * th
    kernels = {
        "fused_kernel": {"us": t_fused * 1e6, "alg_bytes": b_all, "GBps": b_all / t_fused / 1e9,
                         "TFLOPs": flops / t_fused / 1e12,
                         "frac_mfma_bf16": flops / t_fused / BF16_PEAK,
                         "flushed_median_us": t_flushed * 1e6,
                         "flushed_frac_hbm": b_all / t_flushed / HBM_PEAK,
                         "sync_status": sync_word},
    }
    two_stage = {
        "intra_kernel": {"us": t_intra * 1e6, "alg_bytes": b_in, "GBps": b_in / t_intra / 1e9},
        "scan_kernel": {"us": t_scan * 1e6, "alg_bytes": b_out, "GBps": b_out / t_scan / 1e9},
    }
    roof = {"bound": "hbm", "kernel": "fused_kernel", "achieved": b_all / t_fused / 1e9,
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": b_all / t_fused / HBM_PEAK,
            "traffic": measured_traffic("fused_kernel")}
    kernels["fused_kernel"]["traffic"] = roof["traffic"]
    for name in two_stage:
        two_stage[name]["traffic"] = measured_traffic(name)
    path = {"alg_bytes": b_all, "GBps": b_all / dt / 1e9, "frac_hbm": b_all / dt / HBM_PEAK,
            "alg_flops": flops, "TFLOPs": flops / dt / 1e12, "frac_mfma_bf16": flops / dt / BF16_PEAK}
    return spec, dt, roof, path, kernels, two_stage, d, clocks.summary()


def bench_decode(args, gdn):
    spec = gdn_synth.DECODE[4]
    log("generating", spec.name)
    d = gdn_synth.make_decode(spec, 4)
    x = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    state = x["state"]
    o = torch.empty((spec.N, spec.H, spec.V), dtype=x["q"].dtype, device="cuda")

    def run_steps():
        for s in range(spec.steps):
            gdn.recurrent_step(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s], state,
                               d["scale"], o=o)

    settle(run_steps, args.settle_s)
    t = events_time(run_steps, 1) / spec.steps
    es = 2 if spec.dtype == "bf16" else 4
    pairs = spec.N * spec.H
    gate = 4 * (spec.K if spec.gate == "per_key" else 1)
    step_bytes = pairs * (2 * 4 * spec.K * spec.V + (2 * spec.K + 2 * spec.V) * es + 4 + gate)
    log("decode step %.1f us" % (t * 1e6))
    return d, {"workload": spec.name, "us_per_step": t * 1e6, "steps": spec.steps,
            "tokens_per_s": spec.N / t,
            "roofline": {"bound": "hbm", "kernel": "step_kernel",
                         "achieved": step_bytes / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": step_bytes / t / HBM_PEAK, "alg_bytes": step_bytes,
                         "traffic": measured_traffic("step_kernel")}}


def bench_backward(args, gdn, d, seed=1):
    """The chunked backward on a prefill workload (d: the scalar-gate prefill,
    or the per-key one): four kernels per call (intra-chunk recompute, state
    recompute, reverse state-gradient pass, per-chunk gradients), timed with
    HIP events over back-to-back calls."""
    spec = d["spec"]
    gate = spec.gate
    gr = gdn_synth.make_grads(d, seed)
    x = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, beta, g, h0 = (x[n] for n in ("q", "k", "v", "beta", "g", "h0"))
    do, dht = gr["do"].cuda(), gr["dht"].cuda()
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dbeta=torch.empty_like(beta), dg=torch.empty_like(g), dh0=torch.empty_like(dht))
    desc = gdn.fwd_desc(q, v, gate, spec.chunk, d["scale"])
    ws = torch.empty(gdn.bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    def call():
        gdn.chunk_bwd(q, k, v, beta, g, do, d["scale"], h0=h0, dht=dht, workspace=ws, out=out,
                      gate=gate)

    settle(call, args.settle_s)
    for _ in range(max(args.warmup // 10, 5)):
        call()
    reps = max(args.steps // 5, 5)
    t = events_time(call, reps)
    th = spec.B * spec.T * spec.H
    es = 2 if spec.dtype == "bf16" else 4
    state = 4 * spec.K * spec.V * spec.H * spec.B
    gb = 4 + 4 * (spec.K if gate == "per_key" else 1)   # beta and g of a token-head
    # inputs q, k, v, dO, beta, g, h0 (if any), dht; outputs dq, dk, dv, dbeta, dg, dh0
    alg_bytes = th * ((2 * spec.K + 2 * spec.V) * es + gb) + (2 if h0 is not None else 1) * state + \
        th * ((2 * spec.K + spec.V) * es + gb) + state
    flops = gdn_synth.bwd_flops_per_token_head(spec.K, spec.V, spec.chunk) * th
    log("%s backward %.1f us per call" % (gate, t * 1e6))
    pre = "kda_" if gate == "per_key" else ""
    return {"workload": spec.name, "us_per_call": t * 1e6, "calls": reps,
            "tokens_per_s": spec.B * spec.T / t, "alg_flops": flops,
            "TFLOPs": flops / t / 1e12, "frac_mfma_bf16": flops / t / BF16_PEAK,
            "alg_bytes": alg_bytes, "GBps": alg_bytes / t / 1e9, "frac_hbm": alg_bytes / t / HBM_PEAK,
            "workspace_bytes": ws.numel(),
            # HBM bytes per launch of each of its kernels, from the committed
            # counter summary (None where the source changed since)
            "traffic": {pre + k: measured_traffic(pre + k)
                        for k in ("bwd_intra_kernel", "bwd_state_scan_kernel", "bwd_scan_kernel",
                                  "bwd_local_kernel")}}


def bench_kda(args, gdn):
    """The per-key-gate workload (two-stage route): whole calls timed with an
    event pair around back-to-back calls, and its two kernels inside a call."""
    spec = gdn_synth.PREFILL[3]
    log("generating", spec.name)
    d = gdn_synth.make_prefill(spec, 3)
    x = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, beta, g = (x[n] for n in ("q", "k", "v", "beta", "g"))
    desc = gdn.fwd_desc(q, v, "per_key", spec.chunk, d["scale"])
    ws = torch.empty(gdn.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(v)
    ht = torch.empty((spec.B, spec.H, spec.K, spec.V), dtype=torch.float32, device="cuda")

    def call():
        gdn.chunk_fwd(q, k, v, beta, g, d["scale"], gate="per_key", o=o, ht=ht, workspace=ws)

    settle(call, args.settle_s)
    for _ in range(10):
        call()
    reps = max(args.steps // 5, 10)
    t = events_time(call, reps)
    t_flushed = flushed_median(call, 20)
    t_intra, t_scan = step_kernel_times(
        lambda: gdn.chunk_intra(q, k, v, beta, g, d["scale"], gate="per_key", store_ainv=False,
                                workspace=ws, views=False),
        lambda: gdn.chunk_scan(desc, ws, o, ht=ht), reps)
    b_in, b_out = prefill_bytes(spec, spec.B)
    log("KDA prefill %.1f us per call (intra %.1f, scan %.1f)" % (t * 1e6, t_intra * 1e6, t_scan * 1e6))
    return d, {"workload": spec.name, "us_per_call": t * 1e6, "tokens_per_s": spec.B * spec.T / t,
            "alg_bytes": b_in + b_out, "GBps": (b_in + b_out) / t / 1e9,
            "frac_hbm": (b_in + b_out) / t / HBM_PEAK, "flushed_median_us": t_flushed * 1e6,
            "kernels": {"intra_kernel": {"us": t_intra * 1e6, "alg_bytes": b_in,
                                         "GBps": b_in / t_intra / 1e9,
                                         "traffic": measured_traffic("kda_intra_kernel")},
                        "scan_kernel": {"us": t_scan * 1e6, "alg_bytes": b_out,
                                        "GBps": b_out / t_scan / 1e9,
                                        "traffic": measured_traffic("kda_scan_kernel")}}}


def bench_variants(args, gdn):
    """The prefill workload (B=4, T=4096, H=16, d=128, bf16) with each input
    option of the forward: raw gate and beta logits activated inside the
    kernel, beta in (0, 2), two value heads per q/k head (16 value heads on 8
    q/k heads) and q/k L2 normalisation; then the same workload at the other
    head sizes the single-pass kernel is built for, (K, V) = (64, 64),
    (128, 64), (64, 128).  Whole calls, timed with an event pair around
    back-to-back calls of the C entry point on arguments marshalled once (the
    binding's per-call checks would otherwise take longer than the kernel)."""
    import ctypes
    from gated_delta_rule_14_amd import _binding as B
    lib = gdn.load()
    spec = gdn_synth.PREFILL[1]
    log("generating", spec.name, "(raw logits)")
    d = gdn_synth.make_prefill(spec, 1, logits=True)
    x = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, beta, g, h0 = (x[n] for n in ("q", "k", "v", "beta", "g", "h0"))
    o, ht = torch.empty_like(v), torch.empty_like(h0)
    A_log, dt_bias = x["A_log"], x["dt_bias"]
    logits = gdn.activation(gate_logits=True, beta_sigmoid=True, A_log=A_log, dt_bias=dt_bias)
    # the same gates activated beforehand (input preparation), for the cases
    # that take activated g and beta
    g_act = -torch.exp(A_log) * torch.nn.functional.softplus(g + dt_bias)
    b_act = torch.sigmoid(beta)
    cases = {"plain": (q, k, g_act, b_act, None),
             "gate_beta_logits": (q, k, g, beta, logits),
             "neg_eig": (q, k, g, beta, gdn.activation(gate_logits=True, beta_sigmoid=True,
                                                       neg_eig=True, A_log=A_log, dt_bias=dt_bias)),
             "qk_l2norm": (q, k, g_act, b_act, gdn.activation(qk_l2norm=True)),
             "gva_m2": (q[:, :, ::2].contiguous(), k[:, :, ::2].contiguous(), g, beta, logits)}
    reps = max(args.steps // 5, 20)
    out = {"workload": spec.name}
    first = True
    for name, (qq, kk, gg, bb, act) in cases.items():
        desc = gdn.fwd_desc(qq, v, "scalar", spec.chunk, d["scale"])
        nbytes = gdn.workspace_bytes(desc, act)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        cargs = (ctypes.byref(desc), ctypes.byref(act) if act is not None else None,
                 B._ptr(qq), B._ptr(kk), B._ptr(v), B._ptr(bb), B._ptr(gg), B._ptr(h0), None,
                 B._ptr(o), B._ptr(ht), B._ptr(ws), nbytes, B._stream(None))
        B._check(lib.gdn_chunk_fwd_act(*cargs))
        if first:   # the clock settles again after the host-side input generation
            settle(lambda: lib.gdn_chunk_fwd_act(*cargs), args.settle_s)
            for _ in range(args.warmup):
                lib.gdn_chunk_fwd_act(*cargs)
            first = False
        out[name + "_us"] = 1e6 * events_time(lambda: lib.gdn_chunk_fwd_act(*cargs), reps)
    for K, V in ((64, 64), (128, 64), (64, 128)):
        sp = gdn_synth.prefill_spec(1, K=K, V=V)
        log("generating", sp.name, "at K=%d V=%d" % (K, V))
        dk = gdn_synth.make_prefill(sp, 1)
        xk = {n: dk[n].cuda() for n in ("q", "k", "v", "beta", "g", "h0")}
        ok, htk = torch.empty_like(xk["v"]), torch.empty_like(xk["h0"])
        desc = gdn.fwd_desc(xk["q"], xk["v"], "scalar", sp.chunk, dk["scale"])
        nbytes = gdn.workspace_bytes(desc)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        cargs = (ctypes.byref(desc), None, *(B._ptr(xk[n]) for n in ("q", "k", "v", "beta", "g", "h0")),
                 None, B._ptr(ok), B._ptr(htk), B._ptr(ws), nbytes, B._stream(None))
        B._check(lib.gdn_chunk_fwd_act(*cargs))
        settle(lambda: lib.gdn_chunk_fwd_act(*cargs), args.settle_s)
        out["head_k%d_v%d_us" % (K, V)] = 1e6 * events_time(lambda: lib.gdn_chunk_fwd_act(*cargs), reps)
    log("input options: " + ", ".join("%s %.1f us" % (n[:-3], t) for n, t in out.items()
                                     if n.endswith("_us")))
    return out


def bench_varlen(args, gdn):
    """The packed variable-length workload (fused route; the longest
    sequence, 65 536 tokens, sets the time): whole calls, events."""
    spec = gdn_synth.PREFILL[2]
    log("generating", spec.name)
    d = gdn_synth.make_prefill(spec, 2)
    x = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, beta, g, cu = (x[n] for n in ("q", "k", "v", "beta", "g", "cu_seqlens"))
    N = cu.numel() - 1
    desc = gdn.fwd_desc(q, v, "scalar", spec.chunk, d["scale"], N)
    ws = torch.zeros(gdn.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(v)
    ht = torch.empty((N, spec.H, spec.K, spec.V), dtype=torch.float32, device="cuda")

    def call():
        gdn.chunk_fwd(q, k, v, beta, g, d["scale"], cu_seqlens=cu, o=o, ht=ht, workspace=ws)

    settle(call, args.settle_s)
    for _ in range(5):
        call()
    reps = 10
    t = events_time(call, reps)
    sync_word = gdn.sync_status(desc, ws)
    if sync_word != 0:
        raise RuntimeError("the fused kernel reported a failed hand-off between its waves")
    tokens = int(q.shape[1])
    es = 2
    alg = tokens * spec.H * ((2 * spec.K + 2 * spec.V) * es + 8) + 4 * spec.K * spec.V * spec.H * N
    longest = max(d["lengths"])
    log("varlen prefill %.1f us per call (%d tokens, longest sequence %d)" % (t * 1e6, tokens, longest))
    return d, {"workload": spec.name, "us_per_call": t * 1e6, "tokens": tokens, "sequences": N,
            "sync_status": sync_word,
            "longest": longest, "tokens_per_s": tokens / t, "alg_bytes": alg,
            "GBps": alg / t / 1e9, "frac_hbm": alg / t / HBM_PEAK,
            "us_per_chunk_of_longest": t * 1e6 / ((longest + spec.chunk - 1) // spec.chunk),
            "traffic": measured_traffic("varlen_fused_kernel")}


def oracle_threads():
    """Host threads for the oracle: every CPU this process may run on, but no
    more than OMP_NUM_THREADS when the environment sets it (the host's share
    of CPUs for one GPU)."""
    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(cores, int(env)) if env.isdigit() and int(env) > 0 else cores


def _repeat(fn, min_s, max_s=30.0):
    done, t0 = 0, time.perf_counter()
    while True:
        fn()
        done += 1
        el = time.perf_counter() - t0
        if el >= min_s or el / done * (done + 1) > max_s:
            return done, el


def cpu_baseline(d, threads, min_s=8.0):
    """The fp64 token recurrence over the whole prefill workload, repeated
    for >= min_s of wall time; conversions to fp64 are not timed."""
    import oracle
    args = [oracle.as_f64(d[n]) for n in ("q", "k", "v", "beta", "g")]
    h0 = oracle.as_f64(d["h0"])
    B, T = d["q"].shape[:2]
    done, el = _repeat(lambda: oracle.recurrent_forward(*args, d["scale"], h0=h0, threads=threads),
                       min_s)
    return {"value": done * B * T / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole workload (B=4, T=4096, H=16, d=128) run %d times by the fp64 "
                      "token recurrence, %.1f s wall" % (done, el)}


def cpu_baselines_other(varlen_d, kda_d, decode_d, threads, budget_s=6.0):
    """The oracle on the other workloads, each a bounded sample of about
    budget_s seconds, scaled to whole-workload tokens/s."""
    import oracle
    out = {}
    if varlen_d is not None:    # packed: groups of heads over all 16 sequences
        d = varlen_d
        H = d["q"].shape[2]
        T = d["q"].shape[1]
        heads, el, grp = 0, 0.0, 8
        while heads < H and el < budget_s:
            sl = slice(heads, heads + grp)
            a = [oracle.as_f64(d[n][:, :, sl]) for n in ("q", "k", "v", "beta", "g")]
            t0 = time.perf_counter()
            oracle.recurrent_forward(*a, d["scale"], cu_seqlens=d["cu_seqlens"], threads=threads)
            el += time.perf_counter() - t0
            heads += grp
            del a
        out["varlen"] = {"value": T * heads / H / el, "unit": "tokens/s", "cores": threads,
                         "kind": "oracle", "sample": "heads 0-%d of %d over all %d packed sequences "
                         "(%d tokens), %.1f s wall" % (heads - 1, H, d["cu_seqlens"].numel() - 1, T, el)}
    if kda_d is not None:
        d = kda_d
        a = [oracle.as_f64(d[n]) for n in ("q", "k", "v", "beta", "g")]
        B, T = d["q"].shape[:2]
        done, el = _repeat(lambda: oracle.recurrent_forward(*a, d["scale"], gate="per_key",
                                                            threads=threads), budget_s)
        out["kda"] = {"value": done * B * T / el, "unit": "tokens/s", "cores": threads,
                      "kind": "oracle", "sample": "the whole per-key-gate workload (B=2, T=8192, "
                      "H=16) run %d times, %.1f s wall" % (done, el)}
        del a
    if decode_d is not None:    # 64 steps of every sequence = a 64-token recurrence each
        d = decode_d
        a = [oracle.as_f64(d[n].transpose(0, 1).contiguous()) for n in ("q", "k", "v", "beta", "g")]
        st = oracle.as_f64(d["state"])
        S, N = d["q"].shape[:2]
        done, el = _repeat(lambda: oracle.recurrent_forward(*a, d["scale"], h0=st, threads=threads),
                           budget_s)
        out["decode"] = {"value": done * N / (el / S), "unit": "tokens/s (sequences per step time)",
                         "cores": threads, "kind": "oracle",
                         "sample": "all %d sequences x 32 heads, %d consecutive steps (as one %d-token "
                         "recurrence per sequence), run %d times, %.1f s wall" % (N, S, S, done, el)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU clock settles during the first ~100 launches
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-kda", action="store_true")
    ap.add_argument("--no-kda-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of back-to-back calls before each leg's warm-up and timing")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "kda", "kda_backward", "varlen",
                                       "variants"],
                    help="run the prefill leg and this one only (for per-leg profiles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (a known-size kernel to scale "
                         "hardware byte counters by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import gated_delta_rule_14_amd as gdn
    gdn.load()
    torch.cuda.init()
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        for leg in ("decode", "backward", "kda", "kda_backward", "varlen", "variants"):
            if leg != args.only and not (leg == "kda" and args.only == "kda_backward"):
                setattr(args, "no_" + leg, True)
        args.no_cpu = True
    dev = device_info()
    spec, dt, roof, path, kernels, two_stage, d, clocks = bench_prefill(args, gdn)
    dec_d, decode = (None, None) if args.no_decode else bench_decode(args, gdn)
    backward = None if args.no_backward else bench_backward(args, gdn, d)
    kda_d, kda = (None, None) if args.no_kda else bench_kda(args, gdn)
    kda_backward = None if (args.no_kda_backward or kda_d is None) else bench_backward(args, gdn, kda_d, 3)
    var_d, varlen = (None, None) if args.no_varlen else bench_varlen(args, gdn)
    variants = None if args.no_variants else bench_variants(args, gdn)
    cpu, cpu_other = None, None
    if not args.no_cpu:
        threads = oracle_threads()
        cpu = cpu_baseline(d, threads)
        cpu_other = cpu_baselines_other(var_d, kda_d, dec_d, threads)
        log("oracle on the host: %s" % ", ".join("%s %.0f tokens/s" % (n, r["value"])
                                                for n, r in [("prefill", cpu)] + list(cpu_other.items())))
    line = {
        "metric": METRIC,
        "value": spec.B * spec.T / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "T": spec.T, "H": spec.H, "K": spec.K,
                   "V": spec.V, "chunk": spec.chunk, "gate": spec.gate, "h0": "N(0,0.02^2)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baselines_other": cpu_other,
        "device_info": dev,
        "clocks_under_load": clocks,
        "settle_s": args.settle_s,
        "path": path,
        "mfma_pct_of_bf16_peak": 100.0 * path["frac_mfma_bf16"],
        "kernels": kernels,
        "two_stage": two_stage,
        "decode": decode,
        "backward": backward,
        "kda": kda,
        "kda_backward": kda_backward,
        "varlen": varlen,
        "input_options": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
