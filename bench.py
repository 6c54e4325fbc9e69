#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X; prints ONE JSON line.

Step = one chunkwise prefill of the gated-linear-attention workload
``gla_B1H16_L32768_d128`` (B=1, H=16, L=32768, d_k=d_v=128, bf16 q/k/v,
fp32 diagonal log-gates, chunk 64): state pass, segment scan and main pass,
inputs resident in HBM.  ``value`` is sequence tokens per second.

Timing of every prefill-like part (the prefill, its backward and training
step, the packed, scalar-gate, retention and delta prefills): warm-up
steps, then K steps, each after a 512 MiB write and a 512 MiB read that
evict the 256 MB Infinity Cache, and bracketed by HIP events on the stream; ``ms_per_step``
is their mean (``step_ms`` adds the median, the minimum and the mean of K
steps run back to back without the flush).  Per-kernel averages come from
a further K flushed steps.  Decode steps run back to back (1 GiB of state
per step leaves nothing to reuse).

Also reported, in the same line:
* ``roofline``: the dominant kernel (the main chunk pass), its algorithmic
  bytes per launch over its average duration measured with HIP events that
  the library records on the launch stream, against 8 TB/s; ``traffic`` is
  the measured HBM bytes per launch from rocprofv3 counters (see
  profiles/), null when the kernel sources changed since.
* ``decode``: 1000 consecutive recurrent steps of
  ``decode_retention_256x32_d128`` (256 sequences x 32 heads, fp32 state,
  gamma = 0.97): algorithmic GB/s and its roofline.
* ``backward``: the chunkwise backward of the same prefill (dq, dk, dv,
  log-gate gradient and dS0 from seeded dout), per-kernel times and the
  roofline of the per-chunk gradient kernel.
* ``varlen``: the packed-sequence prefill of ``gla_varlen_32seq_H16_d128``
  (32 sequences, seeded lengths in [1, 4096]) and one decode step of all of
  them from their final states.
* ``scalar_gate``: the same prefill with one gate per token and head
  (``scalar_gate_B1H16_L32768_d128``), which drops the d_k-wide gate stream.
* ``configs``: every prefill workload of the workload table (plain linear
  attention L=64 d=16 fp32; plain linear attention B=4 H=8 L=2048 d=64
  normalised; retention B=2 H=16 L=8192 d=128; the headline) with tokens/s,
  TFLOP/s, GB/s, the step's fraction of its attainable roofline and its main
  pass's roofline, and the decode workload plain and with phi = elu+1 and
  the normaliser.
* ``retention_groupnorm``: the retention workload with the fused group-norm
  / swish-gate output epilogue.
* ``delta``: the delta rule's prefill (``delta_B16H16_L4096_d128``) and
  100 decode steps at the decode workload's shape.
* ``cpu_baseline``: the fp64 oracle (test infrastructure, untuned) on the
  same prefill workload drawn on the host, timed on this machine's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import itertools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("chunkwise fwd tokens/s + % bf16 MFMA peak (H16 d128 L32k); "
          "decode HBM GB/s")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PROFILES = os.path.join(ROOT, "profiles")
# the prefill workloads timed beside the headline, in the workload table's order
PREFILL_CONFIGS = ("linear_elu1_L64_d16_fp32", "linear_elu1_B4H8_L2048_d64",
                   "retention_B2H16_L8192_d128", "gla_B1H16_L32768_d128")


def kernel_source_hash():
    """Hash of the sources the main chunk kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_attention_amd", "csrc")
    for f in ("chunk_kernel.h", "la_device.h", "la_internal.h", "chunk_bf16_d128.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_attention_amd", "csrc")
    for f in ("decode_kernel.hip", "la_device.h", "la_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def bwd_source_hash():
    """Hash of the sources the per-chunk gradient kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_attention_amd", "csrc")
    for f in ("bwd_kernel.h", "la_device.h", "la_internal.h", "bwd_bf16_d128.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def delta_source_hash():
    """Hash of the sources the delta-rule kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_attention_amd", "csrc")
    for f in ("delta_kernel.h", "tile_ops.h", "la_device.h", "la_internal.h", "delta_bf16_d128.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name, src_hash):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none or it was taken from other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


FLUSH_BYTES = 512 << 20


class CacheFlush:
    """Writes a 512 MiB scratch buffer, twice the 256 MB Infinity Cache, and
    then reads another 512 MiB buffer, so that a step timed after it finds
    none of its inputs cached (the 34 MB and 270 MB workloads would
    otherwise run partly from the cache when repeated back to back) and no
    dirty lines of the flush itself left to write back.  A write alone made
    the event-timed step of the 806 MB prefill about 30 us longer than the
    same step after a read, or with no flush at all, while the per-kernel
    durations stayed the same: the timed region billed the flush's tail."""

    def __init__(self, torch, dev, on=True):
        self.torch = torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if on else None
        self.rbuf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if on else None
        self.acc = torch.empty((), dtype=torch.float32, device=dev) if on else None
        self.n = 0

    def __call__(self):
        if self.buf is not None:
            self.n += 1
            self.buf.fill_(float(self.n & 7))
            self.torch.sum(self.rbuf, dim=0, out=self.acc)


def time_steps(torch, step, args, flush):
    """Step times in ms: `warmup` steps, then `steps` steps each after a
    cache flush and bracketed by events on the current stream (mean, median,
    min), and the mean of as many steps run back to back without flushes."""
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t0) / args.steps * 1e3
    return {"mean": sum(per) / len(per), "median": per[len(per) // 2], "min": per[0],
            "back_to_back": b2b}


def kernel_avgs(torch, api, step, args, flush, names):
    """Average duration (us) of each named kernel family over `steps` steps,
    each after a cache flush, from the library's per-launch HIP events."""
    api.la_profile_begin()
    for _ in range(args.steps):
        flush()
        step()
    torch.cuda.synchronize()
    api.la_profile_end()
    out = {}
    for name in names:
        n, ms = api.la_profile_query(name)
        out[name] = (ms / n * 1e3) if n else None
    return out


def step_times(t):
    out = {"median": round(t["median"], 4), "min": round(t["min"], 4),
           "back_to_back": round(t["back_to_back"], 4)}
    if "graph" in t:
        out["graph_replay"] = round(t["graph"], 4)
    return out


FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 matrix peak


def esize(w):
    return 4 if str(w.dtype).endswith("float32") else 2


def prefill_bytes(w):
    """Algorithmic bytes of one prefill: q, k, v read and out written in the
    input type (+ fp32 log-gates: d_k per token-head for the diagonal gate,
    one for the scalar gate) per token-head, plus the fp32 final state (and
    normaliser) per (b,h)."""
    gate = {2: 4 * w.dk, 3: 4}.get(w.gate_mode, 0)
    per_th = esize(w) * (2 * w.dk + 2 * w.dv) + gate
    fin = w.dk * w.dv * 4 + (w.dk * 4 if w.normalize else 0)
    return w.B * w.H * w.L * per_th + w.B * w.H * fin


def prefill_flops(w):
    """Dense chunk-form flops: 2C(dk+dv) + 4 dk dv per token-head."""
    return w.B * w.H * w.L * (2 * w.chunk * (w.dk + w.dv) + 4 * w.dk * w.dv)


def attainable_frac(w, ms):
    """Fraction of the attainable roofline of one step: the larger of its
    HBM floor and its matrix-core floor over the measured step time."""
    peak_f = (BF16_PEAK_TFLOPS if esize(w) == 2 else FP32_PEAK_TFLOPS) * 1e12
    floor_s = max(prefill_bytes(w) / (HBM_PEAK_GBS * 1e9), prefill_flops(w) / peak_f)
    return floor_s / (ms * 1e-3), floor_s * 1e6


def bench_prefill(args, torch, api, workloads, name=None):
    w = workloads.WORKLOADS[name or workloads.PREFILL_HEADLINE]
    dev = torch.device("cuda", 0)
    inp = workloads.workload_inputs(w.name, seed=0, device=dev)
    q, k, v, la = inp["q"], inp["k"], inp["v"], inp["log_alpha"]
    ldt = api.LA_BF16 if esize(w) == 2 else api.LA_F32
    desc = api.make_desc(w.B, w.H, w.L, w.dk, w.dv, ldt, w.phi, w.normalize, 0)
    P = api.la_chunk_fwd_segments(desc, w.chunk)
    need = api.la_chunk_fwd_workspace_bytes(desc, w.chunk)
    out = torch.empty_like(v)
    S_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    z_final = (torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device=dev)
               if w.normalize else None)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    lib = api.load_library()
    dref = ctypes.byref(desc)
    g_host = torch.tensor(w.gamma or (0.0,), dtype=torch.float32)
    if w.gate_mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR):
        gate = la.data_ptr()
    elif w.gate_mode == api.LA_GATE_GAMMA:
        gate = ctypes.c_void_p(g_host.data_ptr())
    else:
        gate = None
    argv = (dref, q.data_ptr(), k.data_ptr(), v.data_ptr(), w.gate_mode, gate,
            None, None, w.chunk, out.data_ptr(), S_final.data_ptr(),
            None if z_final is None else z_final.data_ptr(), ws.data_ptr(), need, sp)

    def step():
        st = lib.la_chunk_fwd(*argv)
        if st != 0:
            raise RuntimeError(api.la_last_error_message())

    flush = CacheFlush(torch, dev, not args.no_flush)
    times = time_steps(torch, step, args, flush)
    # a second pass over as many steps with per-kernel HIP events on the stream
    kern = {name: {"avg_us": us} for name, us in
            kernel_avgs(torch, api, step, args, flush,
                        ("chunk_main", "chunk_sub", "chunk_state", "state_scan")).items()}
    # the same step's launches captured once in a HIP graph and replayed
    # (what a caller that captures its step gets): same protocol, and the
    # replayed output must equal the direct call's bit for bit
    ref = out.clone()
    side = torch.cuda.Stream(dev)
    gargv = argv[:-1] + (ctypes.c_void_p(side.cuda_stream),)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        if lib.la_chunk_fwd(*gargv) != 0:
            raise RuntimeError(api.la_last_error_message())
    gtimes = time_steps(torch, graph.replay, args, flush)
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("graph replay differs from the direct call")
    times["graph"] = gtimes["mean"]

    ms_step = times["mean"]
    tokens = w.B * w.L
    bytes_alg = prefill_bytes(w)
    flops = prefill_flops(w)
    main_us = kern["chunk_main"]["avg_us"]
    achieved = bytes_alg / (main_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = measured_traffic(f"chunk_main_{w.name}", khash)
    for fam in kern:
        kern[fam]["traffic"] = measured_traffic(f"{fam}_{w.name}", khash)
    frac, floor_us = attainable_frac(w, ms_step)
    return {
        "w": w, "P": P, "ms_step": ms_step, "tokens_per_s": tokens / (ms_step * 1e-3),
        "times": step_times(times),
        "kernels": kern, "bytes": bytes_alg, "flops": flops,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "chunk_main",
                     "bytes_per_launch": bytes_alg, "avg_launch_us": round(main_us, 2)},
        "mfma_pct": 100.0 * flops / (ms_step * 1e-3) /
                    ((BF16_PEAK_TFLOPS if esize(w) == 2 else FP32_PEAK_TFLOPS) * 1e12),
        "hbm_pct_step": 100.0 * bytes_alg / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "attainable_frac": frac, "floor_us": floor_us,
    }


def config_entry(pre):
    """One config's figures for the line's ``configs`` object."""
    w = pre["w"]
    ms = pre["ms_step"]
    return {"workload": w.name, "ms_per_step": round(ms, 4), "step_ms": pre["times"],
            "tokens_per_s": round(pre["tokens_per_s"], 1),
            "tflops": round(pre["flops"] / (ms * 1e-3) / 1e12, 3),
            "gbs": round(pre["bytes"] / (ms * 1e-3) / 1e9, 1),
            "matrix_peak_pct": round(pre["mfma_pct"], 3),
            "hbm_peak_pct_step": round(pre["hbm_pct_step"], 2),
            "attainable_roofline_frac_step": round(pre["attainable_frac"], 4),
            "floor_us": round(pre["floor_us"], 2),
            "segments": pre["P"],
            "kernels_avg_us": {k: (round(v["avg_us"], 2) if v["avg_us"] else None)
                               for k, v in pre["kernels"].items()},
            "kernels_traffic_bytes": {k: (round(v["traffic"]) if v.get("traffic") else None)
                                      for k, v in pre["kernels"].items() if v["avg_us"]},
            "step_traffic_vs_algorithmic": step_traffic_ratio(pre),
            "roofline": pre["roofline"]}


def step_traffic_ratio(pre):
    """Measured HBM bytes of every launch of one step (from the committed
    counter records of its kernels) over the algorithmic bytes, or None
    when a launched kernel has no current record.  The sub-chunk kernel,
    when no segment needs it, only reads one flag per workgroup."""
    tot = 0.0
    for fam, v in pre["kernels"].items():
        if not v["avg_us"] or fam == "chunk_sub":
            continue
        if not v.get("traffic"):
            return None
        tot += v["traffic"]
    return round(tot / pre["bytes"], 3)


def backward_bytes(w):
    """Algorithmic bytes of one backward of the prefill (no S0, no dS_final):
    q, k, v, dout read and dq, dk, dv written in bf16, log-gates read and
    their gradient written in fp32, per token-head, plus dS0 per (b,h)."""
    per_th = 2 * (4 * w.dk + 3 * w.dv) + (8 * w.dk if w.gate_mode == 2 else 0)
    return w.B * w.H * w.L * per_th + w.B * w.H * w.dk * w.dv * 4


def backward_kernel_bytes(w, chunk, segments):
    """Bytes the gradient kernel must move as designed: the token tensors of
    the backward and dS0, the state before every chunk in bf16, and, with
    several segments per (b,h), the fp32 state gradient entering each."""
    nchunks = -(-w.L // chunk)
    bh = w.B * w.H
    return backward_bytes(w) + bh * nchunks * w.dk * w.dv * 2 + \
        (bh * segments * w.dk * w.dv * 4 if segments > 1 else 0)


def bench_backward(args, torch, api, workloads):
    w = workloads.WORKLOADS[workloads.PREFILL_HEADLINE]
    dev = torch.device("cuda", 0)
    inp = workloads.workload_inputs(w.name, seed=0, device=dev)
    grads = workloads.backward_inputs(w.B, w.H, w.L, w.dk, w.dv, torch.bfloat16, seed=100,
                                      device=dev, with_state_grad=False)
    q, k, v, la, do = inp["q"], inp["k"], inp["v"], inp["log_alpha"], grads["dout"]
    desc = api.make_desc(w.B, w.H, w.L, w.dk, w.dv, api.LA_BF16, w.phi, False, 0)
    chunk = api.la_chunk_bwd_chunk(desc)
    need = api.la_chunk_bwd_workspace_bytes(desc)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dla = torch.empty_like(la)
    dS0 = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = api.load_library()
    argv = (ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
            w.gate_mode, la.data_ptr(), None, None, None, dq.data_ptr(), dk.data_ptr(),
            dv.data_ptr(), dla.data_ptr(), dS0.data_ptr(), ws.data_ptr(), need, sp)

    def step():
        st = lib.la_chunk_bwd(*argv)
        if st != 0:
            raise RuntimeError(api.la_last_error_message())

    flush = CacheFlush(torch, dev, not args.no_flush)
    times = time_steps(torch, step, args, flush)
    # a training step: the forward that keeps its boundary states, then the
    # backward from them
    nst = api.la_chunk_train_states_bytes(desc)
    states = torch.empty(nst // 4 + 4, dtype=torch.float32, device=dev)
    out = torch.empty_like(v)
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    fneed = api.la_chunk_fwd_workspace_bytes(desc, chunk)
    fws = torch.empty(max(fneed // 4, 1), dtype=torch.float32, device=dev)
    fargv = (ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), w.gate_mode,
             la.data_ptr(), None, out.data_ptr(), Sf.data_ptr(), states.data_ptr(), nst,
             fws.data_ptr(), fneed, sp)
    bargv = argv[:9] + (states.data_ptr(),) + argv[10:]

    def train_step():
        if lib.la_chunk_fwd_train(*fargv) != 0 or lib.la_chunk_bwd(*bargv) != 0:
            raise RuntimeError(api.la_last_error_message())

    ttimes = time_steps(torch, train_step, args, flush)
    train_ms = ttimes["mean"]

    kern = {k: (round(v, 2) if v else None) for k, v in kernel_avgs(
        torch, api, step, args, flush, ("chunk_state", "state_scan", "chunk_store", "chunk_bwd")).items()}
    ms_step = times["mean"]
    bw_us = kern["chunk_bwd"]
    kb = backward_kernel_bytes(w, chunk, api.la_chunk_fwd_segments(desc, chunk))
    achieved = kb / (bw_us * 1e-6) / 1e9
    alg = backward_bytes(w)
    return {
        "workload": w.name, "chunk": chunk, "ms_per_step": round(ms_step, 4),
        "step_ms": step_times(times),
        "tokens_per_s": round(w.B * w.L / (ms_step * 1e-3), 1),
        "train_step": {"what": "la_chunk_fwd_train + la_chunk_bwd from its states",
                       "ms_per_step": round(train_ms, 4), "step_ms": step_times(ttimes),
                       "tokens_per_s": round(w.B * w.L / (train_ms * 1e-3), 1)},
        "algorithmic_bytes": alg,
        "pct_of_hbm_peak_step": round(100.0 * alg / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 2),
        "kernels_avg_us": kern,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"chunk_bwd_{w.name}", bwd_source_hash()),
                     "kernel": "chunk_bwd", "bytes_per_launch": kb,
                     "avg_launch_us": bw_us},
    }


def bench_varlen(args, torch, api, workloads, segments=0):
    """Packed-sequence prefill of the varlen workload, then one decode step
    of every sequence from its S_final (the hand-off)."""
    spec = workloads.VARLEN_SPEC
    lens = workloads.varlen_lengths(spec["n"], spec["lo"], spec["hi"], spec["seed"])
    N, H, d, chunk = len(lens), spec["H"], spec["d"], spec["chunk"]
    T, maxlen = sum(lens), max(lens)
    dev = torch.device("cuda", 0)
    inp = workloads.prefill_inputs(1, H, T, d, d, torch.bfloat16, workloads.GATE_DIAG, seed=0,
                                   device=dev)
    q, k, v, la = inp["q"], inp["k"], inp["v"], inp["log_alpha"]
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32,
                      device=dev)
    desc = api.make_desc(N, H, T, d, d, api.LA_BF16, 0, False, segments)
    need = api.la_chunk_fwd_varlen_workspace_bytes(desc, maxlen, chunk)
    out = torch.empty_like(v)
    S = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = api.load_library()
    argv = (ctypes.byref(desc), cu.data_ptr(), maxlen, q.data_ptr(), k.data_ptr(), v.data_ptr(),
            2, la.data_ptr(), None, None, chunk, out.data_ptr(), S.data_ptr(), None,
            ws.data_ptr(), need, sp)

    def step():
        st = lib.la_chunk_fwd_varlen(*argv)
        if st != 0:
            raise RuntimeError(api.la_last_error_message())

    flush = CacheFlush(torch, dev, not args.no_flush)
    times = time_steps(torch, step, args, flush)
    kern = {k: (round(v, 2) if v else None) for k, v in kernel_avgs(
        torch, api, step, args, flush, ("seq_order", "chunk_main", "chunk_sub", "chunk_state",
                                        "state_scan")).items()}
    # hand-off: one decode step of all N sequences from their prefill states
    qd, kd, vd, lad = workloads.decode_tokens(N, H, d, d, 1, seed=1, device=dev, gate=True)
    od = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    ddesc = api.make_desc(N, H, 1, d, d, api.LA_BF16, 0, False, 0)
    st = lib.la_decode_step(ctypes.byref(ddesc), qd[0].data_ptr(), kd[0].data_ptr(),
                            vd[0].data_ptr(), 2, lad[0].data_ptr(), S.data_ptr(), None,
                            od.data_ptr(), sp)
    if st != 0:
        raise RuntimeError(api.la_last_error_message())
    torch.cuda.synchronize()
    ms_step = times["mean"]
    per_th = 2 * (3 * d) + 4 * d + 2 * d          # q, k, v, log-gates in; out
    alg = H * T * per_th + N * H * d * d * 4
    main_us = kern["chunk_main"]
    achieved = alg / (main_us * 1e-6) / 1e9
    return {
        "workload": workloads.VARLEN_HEADLINE, "sequences": N, "tokens": T, "max_seqlen": maxlen,
        "segments": api.la_chunk_fwd_segments(api.make_desc(N, H, maxlen, d, d, api.LA_BF16,
                                                            0, False, 0), chunk),
        "ms_per_step": round(ms_step, 4), "step_ms": step_times(times),
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "algorithmic_bytes": alg,
        "pct_of_hbm_peak_step": round(100.0 * alg / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 2),
        "kernels_avg_us": kern,
        "decode_hand_off_finite": bool(torch.isfinite(od.float()).all().item()),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"chunk_main_{workloads.VARLEN_HEADLINE}",
                                                 kernel_source_hash()),
                     "kernel": "chunk_main", "bytes_per_launch": alg, "avg_launch_us": main_us},
    }


def bench_retention_groupnorm(args, torch, api, workloads):
    """The retention workload with the fused group-norm / swish-gate output
    epilogue (la_chunk_fwd_groupnorm); the plain retention prefill is one of
    the configs."""
    name = "retention_B2H16_L8192_d128"
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    inp = workloads.workload_inputs(name, seed=0, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    gen = workloads.generator(404, dev)
    gnw = 1.0 + 0.5 * torch.randn((w.H, w.dv), generator=gen, device=dev)
    gnb = 0.3 * torch.randn((w.H, w.dv), generator=gen, device=dev)
    gate = torch.randn((w.B, w.H, w.L, w.dv), generator=gen, device=dev).to(torch.bfloat16)
    desc = api.make_desc(w.B, w.H, w.L, w.dk, w.dv, api.LA_BF16, w.phi, False, 0)
    need = api.la_chunk_fwd_workspace_bytes(desc, w.chunk)
    out = torch.empty_like(v)
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
    g_host = torch.tensor(w.gamma, dtype=torch.float32)
    gp = ctypes.c_void_p(g_host.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = api.load_library()
    gn = api.LaGroupNorm(gnw.data_ptr(), gnb.data_ptr(), gate.data_ptr(), 1e-5)
    argv = (ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), w.gate_mode, gp,
            None, None, w.chunk, ctypes.byref(gn), out.data_ptr(), S.data_ptr(), None,
            ws.data_ptr(), need, sp)

    def step():
        if lib.la_chunk_fwd_groupnorm(*argv) != 0:
            raise RuntimeError(api.la_last_error_message())

    flush = CacheFlush(torch, dev, not args.no_flush)
    t = time_steps(torch, step, args, flush)
    main_us = kernel_avgs(torch, api, step, args, flush, ("chunk_main",))["chunk_main"]
    ms = t["mean"]
    extra = w.B * w.H * w.L * w.dv * 2 + 2 * w.H * w.dv * 4    # swish gate (bf16), scale, shift
    alg = prefill_bytes(w) + extra
    achieved = alg / (main_us * 1e-6) / 1e9
    return {"workload": name + "_groupnorm_swish", "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
            "ms_per_step": round(ms, 4), "step_ms": step_times(t),
            "main_avg_us": round(main_us, 2), "extra_bytes": extra,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": None, "kernel": "chunk_main",
                         "bytes_per_launch": alg, "avg_launch_us": round(main_us, 2)}}


def bench_delta(args, torch, api, workloads):
    """Delta-rule prefill of delta_B16H16_L4096_d128 and 100 decode steps of
    the decode workload's shape (256 sequences x 32 heads, d = 128)."""
    sp = workloads.DELTA_SPEC
    B, H, L, d = sp["B"], sp["H"], sp["L"], sp["d"]
    dev = torch.device("cuda", 0)
    inp = workloads.delta_inputs(B, H, L, d, d, torch.bfloat16, seed=0, device=dev)
    q, k, v, beta = inp["q"], inp["k"], inp["v"], inp["beta"]
    out = torch.empty_like(v)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 0)
    sp_ = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = api.load_library()
    argv = (ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(), None,
            out.data_ptr(), S.data_ptr(), sp_)

    def step():
        if lib.la_delta_fwd(*argv) != 0:
            raise RuntimeError(api.la_last_error_message())

    flush = CacheFlush(torch, dev, not args.no_flush)
    ptimes = time_steps(torch, step, args, flush)
    ms = ptimes["mean"]
    kus = kernel_avgs(torch, api, step, args, flush, ("delta_chunk",))["delta_chunk"]
    del flush
    per_th = 2 * 4 * d + 4          # q, k, v, out bf16 + beta fp32
    alg = B * H * L * per_th + B * H * d * d * 4
    C = api.la_delta_chunk(desc)
    flops_chunk = 2 * C * C * d * 4 + 2 * C * d * d * 4   # K K^T, Q K^T, W, U, P U'; W S, Q S, K^T U' (+T V)
    flops = B * H * (-(-L // C)) * flops_chunk
    del q, k, v, beta, out, S, inp
    # decode: 256 x 32 pairs, d = 128, state N(0,1)
    w = workloads.WORKLOADS[workloads.DECODE_HEADLINE]
    S0, _ = workloads.decode_state(w.B, w.H, w.dk, w.dv, seed=0, device=dev)
    dsteps = 100
    dq, dk_, dv_, _ = workloads.decode_tokens(w.B, w.H, w.dk, w.dv, dsteps, seed=1, device=dev)
    dk_ = (dk_.float() / dk_.float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    dbeta = torch.full((w.B, w.H), 0.5, dtype=torch.float32, device=dev)
    Sd = S0.clone()
    od = torch.empty((w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    ddesc = api.make_desc(w.B, w.H, 1, w.dk, w.dv, api.LA_BF16, 0, False, 0)

    def dstep(t):
        if lib.la_delta_decode_step(ctypes.byref(ddesc), dq[t].data_ptr(), dk_[t].data_ptr(),
                                    dv_[t].data_ptr(), dbeta.data_ptr(), Sd.data_ptr(),
                                    od.data_ptr(), sp_) != 0:
            raise RuntimeError(api.la_last_error_message())

    for t in range(10):
        dstep(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(dsteps):
        dstep(t)
    torch.cuda.synchronize()
    dus = (time.perf_counter() - t0) / dsteps * 1e6
    api.la_profile_begin()
    for t in range(dsteps):
        dstep(t)
    torch.cuda.synchronize()
    api.la_profile_end()
    n, dms = api.la_profile_query("delta_decode")
    dkus = dms / n * 1e3
    step_bytes = 2 * w.B * w.H * w.dk * w.dv * 4 + w.B * w.H * (4 * w.dk * 2 + 4)
    return {
        "prefill": {"workload": workloads.DELTA_HEADLINE, "ms_per_step": round(ms, 4),
                    "step_ms": step_times(ptimes),
                    "tokens_per_s": round(B * L / (ms * 1e-3), 1), "kernel_avg_us": round(kus, 2),
                    "algorithmic_bytes": alg, "tflops": round(flops / (kus * 1e-6) / 1e12, 2),
                    "roofline": {"bound": "hbm", "achieved": round(alg / (kus * 1e-6) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(alg / (kus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "traffic": measured_traffic(
                                     f"delta_chunk_{workloads.DELTA_HEADLINE}", delta_source_hash()),
                                 "kernel": "delta_chunk"}},
        "decode": {"shape": "256 sequences x 32 heads, d=128, bf16 tokens, fp32 state",
                   "us_per_step": round(dus, 2), "kernel_avg_us": round(dkus, 2),
                   "bytes_per_step": step_bytes,
                   "roofline": {"bound": "hbm", "achieved": round(step_bytes / (dkus * 1e-6) / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(step_bytes / (dkus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("delta_decode_256x32_d128",
                                                            delta_source_hash()),
                                "kernel": "delta_decode"}},
    }


def bench_decode(args, torch, api, workloads, with_z=False):
    """Consecutive recurrent steps of the decode workload (retention, gamma =
    0.97, phi = identity, no normaliser).  ``with_z``: the same steps with
    phi = elu+1 and the normaliser, z0 = 1 + |N(0,1)| following gamma."""
    w = workloads.WORKLOADS[workloads.DECODE_HEADLINE]
    dev = torch.device("cuda", 0)
    steps = args.decode_steps
    S0, z0 = workloads.decode_state(w.B, w.H, w.dk, w.dv, seed=0, device=dev, with_z=with_z)
    q, k, v, _ = workloads.decode_tokens(w.B, w.H, w.dk, w.dv, steps, seed=1, device=dev)
    S = S0.clone()
    z = z0.clone() if with_z else None
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    gamma = torch.tensor(w.gamma, dtype=torch.float32)
    g_ptr = ctypes.c_void_p(gamma.data_ptr())
    phi = api.LA_PHI_ELU1 if with_z else w.phi
    desc = api.make_desc(w.B, w.H, 1, w.dk, w.dv, api.LA_BF16, phi, with_z, 0)
    dref = ctypes.byref(desc)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = api.load_library()
    qp = [q[t].data_ptr() for t in range(steps)]
    kp = [k[t].data_ptr() for t in range(steps)]
    vp = [v[t].data_ptr() for t in range(steps)]
    Sp, op = S.data_ptr(), out.data_ptr()
    zp = None if z is None else z.data_ptr()

    def reset():
        S.copy_(S0)
        if z is not None:
            z.copy_(z0)

    def run(n):
        for t in range(n):
            st = lib.la_decode_step(dref, qp[t], kp[t], vp[t], w.gate_mode, g_ptr, Sp,
                                    zp, op, sp)
            if st != 0:
                raise RuntimeError(api.la_last_error_message())

    run(min(steps, 20))
    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    reset()
    torch.cuda.synchronize()
    api.la_profile_begin()
    run(steps)
    torch.cuda.synchronize()
    api.la_profile_end()
    n, ms = api.la_profile_query("decode")
    avg_us = ms / n * 1e3
    state_bytes = w.B * w.H * w.dk * w.dv * 4 + (w.B * w.H * w.dk * 4 if with_z else 0)
    step_bytes = 2 * state_bytes + w.B * w.H * (2 * w.dk + 2 * w.dv) * 2   # + tokens and out
    us_step = elapsed / steps * 1e6
    gbs = step_bytes / (us_step * 1e-6) / 1e9
    achieved = step_bytes / (avg_us * 1e-6) / 1e9
    del q, k, v
    name = w.name + ("_z_elu1" if with_z else "")
    return {
        "workload": name, "steps": steps, "us_per_step": round(us_step, 2),
        "value": round(gbs, 1), "unit": "GB/s", "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "steps_per_s": round(1e6 / us_step, 1), "tokens_per_s": round(w.B * 1e6 / us_step, 1),
        "bytes_per_step": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"decode_{name}", decode_source_hash()),
                     "kernel": "decode", "avg_launch_us": round(avg_us, 2)},
    }


def cpu_baseline(workloads, w):
    """The fp64 oracle, as it stands, on the same prefill workload drawn on
    the host (all 16 heads, all 32768 tokens)."""
    import oracle
    inp = workloads.workload_inputs(w.name, seed=0, device="cpu")
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    la = inp["log_alpha"].double().numpy()
    host = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    nthreads = max(1, min(w.B * w.H, host or 1, 16))
    t0 = time.perf_counter()
    oracle.run(q, k, v, gate_mode=w.gate_mode, log_alpha=la, phi=w.phi,
               normalize=w.normalize, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": round(w.B * w.L / dt, 1), "unit": "tokens/s", "cores": nthreads,
            "nproc": host, "kind": "oracle",
            "sample": f"whole workload {w.name} (B={w.B}, H={w.H}, L={w.L}) drawn on the host; "
                      f"fp64 token loop, {nthreads} threads over (b,h) pairs, {dt:.2f} s"}


def hbm_copy_ceiling(torch, nbytes=1 << 30, reps=10):
    """The practical HBM ceiling beside the 8 TB/s peak: a plain 1 GiB
    device-to-device copy (torch's copy kernel), timed with events on the
    stream; bytes = read + write."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    del src, dst
    return {"what": "1 GiB device-to-device copy, read + write bytes", "us": round(us, 2),
            "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def gpu_warmup(torch, seconds=1.0):
    """About a second of bf16 matrix products before anything is timed, so
    that the first timed launches do not run at idle clocks (the kernel
    durations of a part run first in a process fell by 5-10% over its first
    launches without it)."""
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            b = a @ a
        torch.cuda.synchronize()
    del a, b


def copy_calibration(torch, nbytes=1 << 30):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": nbytes, "launches": 3}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-scalar", action="store_true")
    ap.add_argument("--no-retention", action="store_true")
    ap.add_argument("--no-delta", action="store_true")
    ap.add_argument("--segments", type=int, default=0,
                    help="segments per (b,h) for --only varlen (0 = automatic)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-flush", action="store_true",
                    help="time prefill-like steps without the cache flush before each")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "varlen", "scalar", "retention", "delta",
                             "copy"], default=None,
                    help="run one part only (copy: a 1 GiB device copy used to scale "
                         "rocprofv3 byte counters); prints no metric line")
    ap.add_argument("--workload", default=None, choices=list(PREFILL_CONFIGS),
                    help="prefill workload for --only prefill (default: the headline)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill configs and the normalised decode run")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); sharding over several GPUs is designed, not implemented.",
              file=sys.stderr)
        return 2

    import torch
    from recurrent_attention_amd import api, workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    api.load_library()

    if args.only == "copy":
        copy_calibration(torch)
        return 0
    gpu_warmup(torch)
    if args.only == "decode":
        print(json.dumps({"decode": bench_decode(args, torch, api, workloads),
                          "decode_z": bench_decode(args, torch, api, workloads, True)}), flush=True)
        return 0
    if args.only == "backward":
        print(json.dumps(bench_backward(args, torch, api, workloads)), flush=True)
        return 0
    if args.only == "varlen":
        print(json.dumps(bench_varlen(args, torch, api, workloads, args.segments)), flush=True)
        return 0
    if args.only == "delta":
        print(json.dumps(bench_delta(args, torch, api, workloads)), flush=True)
        return 0
    if args.only == "retention":
        print(json.dumps(bench_retention_groupnorm(args, torch, api, workloads)), flush=True)
        return 0
    if args.only == "scalar":
        sc = bench_prefill(args, torch, api, workloads, "scalar_gate_B1H16_L32768_d128")
        print(json.dumps({"ms_per_step": sc["ms_step"], "kernels": sc["kernels"],
                          "roofline": sc["roofline"]}), flush=True)
        return 0
    if args.only == "prefill":
        pre = bench_prefill(args, torch, api, workloads, args.workload)
        print(json.dumps(config_entry(pre)), flush=True)
        return 0
    def part(name, fn):
        t0 = time.perf_counter()
        r = fn()
        print(f"bench: {name} {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        return r

    pre = part("prefill", lambda: bench_prefill(args, torch, api, workloads))
    w_head = pre["w"].name
    dec = None if args.no_decode else part("decode", lambda: bench_decode(args, torch, api, workloads))
    bwd = None if args.no_backward else part("backward", lambda: bench_backward(args, torch, api, workloads))
    vl = None if args.no_varlen else part("varlen", lambda: bench_varlen(args, torch, api, workloads))
    sc = None if args.no_scalar else part("scalar gate", lambda: bench_prefill(
        args, torch, api, workloads, "scalar_gate_B1H16_L32768_d128"))
    ret = None if args.no_retention else part("retention group norm", lambda: bench_retention_groupnorm(
        args, torch, api, workloads))
    cfgs = {}
    dec_z = None
    if not args.no_configs:
        for cname in PREFILL_CONFIGS:
            cfgs[cname] = pre if cname == w_head else part(cname, lambda: bench_prefill(
                args, torch, api, workloads, cname))
        dec_z = None if args.no_decode else part("decode with z", lambda: bench_decode(
            args, torch, api, workloads, True))
    dl = None if args.no_delta else part("delta", lambda: bench_delta(args, torch, api, workloads))
    w = pre["w"]
    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_step"], 4),
        "step_ms": pre["times"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded torch.randn on the GPU (q,k,v ~ N(0,1)/sqrt(d) in bf16, "
                "log-gates logsigmoid(N(0,1))/16 in fp32)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "gate": "diag", "segments": pre["P"],
                   "parallelism": "single GPU"},
        "pct_of_bf16_mfma_peak": round(pre["mfma_pct"], 3),
        "tflops": round(pre["flops"] / (pre["ms_step"] * 1e-3) / 1e12, 2),
        "pct_of_hbm_peak_step": round(pre["hbm_pct_step"], 2),
        "attainable_roofline_frac_step": round(pre["attainable_frac"], 4),
        "step_traffic_vs_algorithmic": step_traffic_ratio(pre),
        "kernels_avg_us": {k: (round(v["avg_us"], 2) if v["avg_us"] else None)
                           for k, v in pre["kernels"].items()},
        "roofline": pre["roofline"],
    }
    if cfgs:
        line["configs"] = {n: config_entry(c) for n, c in cfgs.items()}
        if dec is not None:
            line["configs"][dec["workload"]] = {k: dec[k] for k in (
                "us_per_step", "value", "unit", "steps_per_s", "tokens_per_s", "roofline")}
            if dec_z is not None:
                line["configs"][dec_z["workload"]] = dec_z
    if dec is not None:
        line["decode"] = dec
    if bwd is not None:
        line["backward"] = bwd
    if vl is not None:
        line["varlen"] = vl
    if ret is not None:
        line["retention_groupnorm"] = ret
    if dl is not None:
        line["delta"] = dl
    if sc is not None:
        line["scalar_gate"] = {
            "workload": sc["w"].name, "ms_per_step": round(sc["ms_step"], 4),
            "step_ms": sc["times"],
            "tokens_per_s": round(sc["tokens_per_s"], 1),
            "pct_of_bf16_mfma_peak": round(sc["mfma_pct"], 3),
            "kernels_avg_us": {k: (round(v["avg_us"], 2) if v["avg_us"] else None)
                               for k, v in sc["kernels"].items()},
            "roofline": sc["roofline"]}
    line["hbm_copy_ceiling"] = hbm_copy_ceiling(torch)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(workloads, w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
