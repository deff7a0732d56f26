"""Throughput of the fused causal GQA + RoPE attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
build the RoPE cos/sin tables, then run the fused forward (RoPE on Q/K tiles,
online softmax, O and LSE) on the long-context workload B=1, T=8192,
n_head=32, n_kv_head=8, head_dim=128, bf16 I/O, RoPE base 500000, causal,
with both products (Q.K^T and P.V) on bf16 matrix-core operands. Inputs are
already resident in HBM when the timed region starts.

Prints one JSON line. `value` is algorithmic TFLOP/s of the step (causal
FLOPs counted exactly: 4*d per visible (query, key) pair per query head).
The forward is given a workspace, so the keys are rotated once by a small
kernel before the attention kernel; both run inside the timed step, enqueued
through the forward's two halves (cgr_attn_fwd_rotate_keys, then
cgr_gqa_rope_attn_fwd_rotated: the kernels and bits of one
cgr_gqa_rope_attn_fwd call) so that the attention kernel has HIP events of
its own. `roofline` reports that kernel alone: its mean launch duration (and
median) from those events on the launch stream, against the MI355X dense
bf16 MFMA peak, with the whole call beside it and the graphics clock
sampled from amd-smi meanwhile, and the same kernel with the library's
default f16 Q.K^T operand (`roofline.f16_operands`); `traffic` is HBM bytes per launch from rocprofv3
counters (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
read from profiles/ and reported only while the kernel sources still hash to
the value recorded with them. `cpu_baseline` times the float64 oracle on a
bounded sample of the same workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--qk bf16|f16]
  python bench.py --copy-calibration   (plain copies, for counter scaling)
  python bench.py --all-configs        (one JSON line per workload configuration,
                                        attention call only; not the headline line;
                                        --only NAME: that workload alone; --graph: also
                                        replayed from a HIP graph)
  python bench.py --backward           (one JSON line for the backward on the same
                                        workload; not the headline line; --varlen: on the
                                        packed MQA batch of 32 sequences instead)
  python bench.py --decode             (one JSON line for decode against a KV cache,
                                        16 sequences x 1 new token; not the headline line)
  python bench.py --window W           (the forward or --backward line with a causal
                                        sliding window of W keys; not the headline line)
  python bench.py --qkv                (one JSON line for the fused RMSNorm + q/k/v projection
                                        + RoPE step of the same model; not the headline line)
  python bench.py --fp8                (the long-context forward with e4m3 q/k/v and e4m3 matrix
                                        products, against the fp8 peak; not the headline line)
  python bench.py --wide               (the forward line at head_dim 256: T=8192, 16 query and
                                        8 K/V heads; not the headline line)
  python bench.py --padded             (the forward line on a right-padded batch of 4 x 8192
                                        tokens, valid lengths U[2048, 8192]; FLOPs over the
                                        valid tokens; not the headline line)
--qk sets the forward line's Q.K^T operand type: bf16 by default for the
headline line, the library's default f16 for the --window, --wide and --padded
lines.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal GQA+RoPE attention fwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
WORKLOAD = "long_context_T8192_H32_KV8_d128"
VARLEN_WORKLOAD = "varlen_mqa_32seqs_16to2048_H16_KV1_d128"
PADDED_WORKLOAD = "padded_B4_T8192_len2048to8192_H32_KV8_d128"
WIDE_WORKLOAD = "long_context_T8192_H16_KV8_d256"
PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
KERNEL_SOURCES = ["attn_fwd_kernel.h", "device_common.h", "attn_fwd_d128.hip"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", f"attn_fwd_{WORKLOAD}.counters.txt")
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_gqa_rope_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(qk: str = "bf16"):
    """HBM bytes per launch from the committed counter summary, if still current
    and taken on the attention kernel with this Q.K^T operand type."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for ln in open(COUNTERS_FILE):
        if ":" in ln and not ln.startswith("#"):
            key, val = ln.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash() or kv.get("qk_operand", "f16") != qk:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class ClockSampler:
    """The graphics clock (MHz) and the socket power (W) under the step's load, from amd-smi.

    amd-smi's clock readings trail the load by the better part of a second
    (the first readings of a burst still show the idle clock), so measure()
    runs the step back to back for `seconds`, samples every 5 ms on a thread,
    and keeps only the samples of the last `tail` seconds. Per sample it takes
    the per-XCD clocks (gpu metrics ``current_gfxclks``) where the driver
    gives them, else the single GFX clock. summary() is None where amd-smi is
    unavailable."""

    def __init__(self):
        self._handle = None
        self._kept = []
        self._watts = []
        self._source = None
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) == 1:
                self._handle = handles[0]
                self._amdsmi = amdsmi
        except Exception:
            self._handle = None

    def _read(self):
        try:
            m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
            per = [float(c) for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
            if per:
                return per, "amd-smi gpu metrics current_gfxclks (per XCD)"
        except Exception:
            pass
        try:
            c = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)["clk"]
            if isinstance(c, (int, float)) and c > 0:
                return [float(c)], "amd-smi GFX clock"
        except Exception:
            pass
        return None, None

    def _power(self):
        try:
            p = self._amdsmi.amdsmi_get_power_info(self._handle).get("socket_power")
            return float(p) if isinstance(p, (int, float)) and 0 < p < 10000 else None
        except Exception:
            return None

    def _cap(self):
        # The socket power limit in W (amd-smi reports it in microwatts).
        try:
            c = self._amdsmi.amdsmi_get_power_cap_info(self._handle).get("power_cap")
            if isinstance(c, (int, float)) and c > 0:
                return round(c / 1e6, 1) if c > 1e5 else float(c)
        except Exception:
            pass
        return None

    def measure(self, step, seconds: float = 2.0, tail: float = 0.8):
        """Run `step` back to back for `seconds` while sampling, and go on
        running it until the sampler thread has stopped, so that the caller
        goes straight on to its warmup and timed steps: an idle gap of a few
        milliseconds here lets the clock drop, and the next ~10 ms of steps
        then run up to 20 % slower while it climbs back. finish() keeps the
        samples of the last `tail` seconds of the sampled load."""
        import torch
        self._samples, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                v, src = self._read()
                if v is not None:
                    self._samples.append((time.perf_counter(), v, src, self._power()))
                stop.wait(0.005)

        self._thread = None
        if self._handle is not None:
            self._thread = threading.Thread(target=loop, daemon=True)
            self._thread.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
        self._t_end, self._tail = time.perf_counter(), tail
        # Stop the sampler, keeping the load on until it has exited: its amd-smi
        # calls would compete with the timed steps' launches, and waiting for
        # it with the GPU idle would let the clock drop.
        stop.set()
        while self._thread is not None and self._thread.is_alive():
            for _ in range(8):
                step()
            torch.cuda.synchronize()

    def finish(self):
        if self._thread is None:
            return
        self._thread.join()
        self._thread = None
        lo, hi = self._t_end - self._tail, self._t_end
        self._kept = [(v, src) for t, v, src, _ in self._samples if lo <= t <= hi]
        self._watts = [w for t, _, _, w in self._samples if lo <= t <= hi and w is not None]
        self._source = self._kept[-1][1] if self._kept else None

    def summary(self):
        if not self._kept:
            return None
        means = [sum(v) / len(v) for v, _ in self._kept]
        n_x = len(self._kept[-1][0])
        per_x = [statistics.median(v[i] for v, _ in self._kept if len(v) == n_x) for i in range(n_x)]
        return {"median": round(statistics.median(means), 1), "xcd_min": min(per_x), "xcd_max": max(per_x),
                "samples": len(self._kept),
                "socket_power_w": round(statistics.median(self._watts), 1) if self._watts else None,
                "power_cap_w": self._cap(),
                "source": f"{self._source} and power info socket_power, the last 0.8 s of 2 s of back-to-back "
                          "steps before the warmup steps"}


def cpu_baseline(inputs, w) -> dict:
    """The float64 oracle, as it stands, on the whole workload (every query
    head at the full T = 8192), about 10 s on 16 host cores."""
    import numpy as np  # noqa: F401
    import oracle
    import workloads as W

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or None
    except Exception:
        pass
    t0 = time.perf_counter()
    oracle.attention_dense(inputs["q"], inputs["k"], inputs["v"], causal=True, base=w.base, style=w.rope_style)
    dt = time.perf_counter() - t0
    flops = W.algorithmic_flops(w.n_head, w.head_dim, [w.T] * w.B, True)
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"float64 numpy oracle on the whole workload (B={w.B} T={w.T}, {w.n_head} query heads, "
                  f"{w.n_kv_head} K/V heads, causal), {dt:.1f} s",
    }


def copy_calibration(torch, dev) -> None:
    """Plain device copies of COPY_BYTES each: the reference for FETCH_SIZE/WRITE_SIZE scaling."""
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copies": 3}), flush=True)


def all_configs(torch, cgr, W, dev, steps: int, warmup: int, graph: bool = False, only=None) -> None:
    """Time the attention call alone on every workload configuration (HIP events on
    the launch stream, mean over `steps` launches after `warmup`). With `graph`,
    also the same `steps` calls captured once in a HIP graph and replayed (no
    per-call host work: the device time of launch-bound configurations)."""
    stream = torch.cuda.current_stream(dev)
    for w in W.WORKLOADS.values():
        if only and w.name != only:
            continue
        inputs = W.make_inputs(w)
        q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
        max_pos = inputs["max_seqlen"] if w.varlen else w.T
        cos, sin = cgr.rope_tables(max_pos, w.head_dim, w.base, device=dev)
        o = torch.empty_like(q)
        if w.varlen:
            cu = inputs["cu_seqlens"].to(dev)
            lengths = (inputs["cu_seqlens"][1:] - inputs["cu_seqlens"][:-1]).tolist()
            lse = torch.empty((w.n_head, q.shape[0]), dtype=torch.float32, device=dev)
            # bf16: room for the once-rotated keys as well as the schedule.
            need = cgr.cgr_attn_fwd_varlen_workspace_size(len(lengths), q.shape[0])
            if w.dtype == "bf16":
                need = max(need, cgr.cgr_attn_fwd_varlen_rotated_workspace_size(len(lengths), q.shape[0],
                                                                                w.n_kv_head, w.head_dim))
            ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)

            def call():
                cgr.gqa_rope_attn_fwd_varlen(q, k, v, cu, int(inputs["max_seqlen"]), cos, sin,
                                             causal=w.causal, rope_style=w.rope_style, out=o, lse=lse,
                                             workspace=ws)
        else:
            lengths = [w.T] * w.B
            lse = torch.empty((w.B, w.n_head, w.T), dtype=torch.float32, device=dev)
            ws = torch.empty(cgr.cgr_attn_fwd_workspace_size(w.B, w.T, w.n_kv_head, w.head_dim),
                             dtype=torch.uint8, device=dev) if w.dtype == "bf16" else False

            def call():
                cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, causal=w.causal, rope_style=w.rope_style,
                                      out=o, lse=lse, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        clock = ClockSampler()
        clock.measure(call)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        clock.finish()
        us = e0.elapsed_time(e1) * 1e3 / steps
        flops = W.algorithmic_flops(w.n_head, w.head_dim, lengths, w.causal)
        tf = flops / (us * 1e-6) / 1e12
        cs = clock.summary() or {}
        line = {"workload": w.name, "io": "f32" if w.dtype == "f32" else "bf16", "us_per_call": round(us, 2),
                "flops": flops, "tflops": round(tf, 3), "pct_of_bf16_peak": round(100.0 * tf / PEAK_TFLOPS, 2),
                "clock_mhz": cs.get("median"), "socket_power_w": cs.get("socket_power_w")}
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(steps):
                    call()
            # Replays back to back for half a second first: the capture leaves
            # the GPU idle long enough for its clock to drop.
            t_w = time.perf_counter()
            while time.perf_counter() - t_w < 0.5:
                g.replay()
                torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            gus = e0.elapsed_time(e1) * 1e3 / steps
            line.update(graph_us_per_call=round(gus, 2), graph_tflops=round(flops / (gus * 1e-6) / 1e12, 3))
        print(json.dumps(line), flush=True)


BWD_METRIC = "causal GQA+RoPE attention bwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"


def cpu_baseline_bwd(inputs, dout, w) -> dict:
    """The float64 oracle's backward, as it stands, on one of the 8 K/V groups
    (its 4 query heads) at the full T = 8192: an eighth of the workload."""
    import oracle
    import workloads as W

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or None
    except Exception:
        pass
    G = w.n_head // w.n_kv_head
    t0 = time.perf_counter()
    oracle.attention_bwd_group(inputs["q"], inputs["k"], inputs["v"], dout, 0, 0, causal=True,
                               base=w.base, style=w.rope_style)
    dt = time.perf_counter() - t0
    flops = W.algorithmic_flops_bwd(G, w.head_dim, [w.T], True)
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"float64 numpy oracle backward, B=1 T={w.T}, K/V head 0 and its {G} query "
                  f"heads, causal: 1/{w.n_kv_head} of the workload, {dt:.1f} s",
    }


def backward(torch, cgr, W, dev, steps: int, warmup: int, with_cpu: bool, window: int = 0,
             varlen: bool = False) -> None:
    """One step = one backward call (prepass, dk/dv kernel, dq kernel) on the
    long-context workload (varlen: the packed MQA batch); o and lse come from
    one forward before timing."""
    w = W.get(VARLEN_WORKLOAD if varlen else WORKLOAD)
    inputs = W.make_inputs(w)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    dout_cpu = W.make_dout(w, inputs["q"])
    dout = dout_cpu.to(dev)
    kw = dict(causal=True, rope_style=w.rope_style, window=window)
    if varlen:
        cu, ms = inputs["cu_seqlens"].to(dev), inputs["max_seqlen"]
        lens = [int(n) for n in inputs["lengths"]]
        cos, sin = cgr.rope_tables(ms, w.head_dim, w.base, device=dev)
        o, lse = cgr.gqa_rope_attn_fwd_varlen(q, k, v, cu, ms, cos, sin, **kw)
        nbytes = cgr.cgr_attn_bwd_varlen_workspace_size(len(lens), sum(lens), w.n_head, w.n_kv_head, w.head_dim)
    else:
        lens = [w.T] * w.B
        cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=dev)
        o, lse = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, **kw)
        nbytes = cgr.cgr_attn_bwd_workspace_size(w.B, w.T, w.n_head, w.n_kv_head, w.head_dim)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        if varlen:
            cgr.gqa_rope_attn_bwd_varlen(q, k, v, o, lse, dout, cu, ms, cos, sin, **kw, dq=dq, dk=dk, dv=dv,
                                         workspace=ws)
        else:
            cgr.gqa_rope_attn_bwd(q, k, v, o, lse, dout, cos, sin, **kw, dq=dq, dk=dk, dv=dv, workspace=ws)

    # As for the forward: 2 s of back-to-back calls (the sustained clock and
    # power), then the warmup and timed calls with no idle gap.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    clock = ClockSampler()
    clock.measure(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    clock.finish()
    wall = time.perf_counter() - t0
    flops = W.algorithmic_flops_bwd(w.n_head, w.head_dim, lens, True, window)
    ms_step = wall * 1e3 / steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    achieved = flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": BWD_METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": len(lens), "T": max(lens), "total_tokens": sum(lens), "n_head": w.n_head,
            "n_kv_head": w.n_kv_head, "head_dim": w.head_dim, "rope_base": w.base, "rope_pairs": w.rope_style,
            "mask": "causal", "io": "bf16", "qk_operand": "f16", "accumulate": "f32",
            "step": "gqa_rope_attn_bwd_varlen" if varlen else "gqa_rope_attn_bwd",
            "window": window, "flops_per_step": flops,
            "pct_of_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS, 2),
        },
        "roofline": {
            "clock_mhz": clock.summary(),
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": "the backward call: bwd_prep_kernel + attn_bwd_dkdv_kernel + attn_bwd_dq_kernel "
                      "(head_dim 128, f16 QK, causal, interleaved)",
            "kernel_ms": round(call_ms, 5),
        },
        "cpu_baseline": cpu_baseline_bwd(inputs, dout_cpu, w) if with_cpu and window == 0 and not varlen else None,
    }
    print(json.dumps(result), flush=True)


DECODE_WORKLOAD = "decode_B16_Tq1_cache4096to8192_H32_KV8_d128"
DECODE_METRIC = "causal GQA+RoPE decode against a KV cache, GB/s moved on 1 MI355X; % of HBM peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def cpu_baseline_decode(x, w) -> dict:
    """The float64 oracle's decode, as it stands, on 4 of the 16 sequences."""
    import oracle
    import workloads as W

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or None
    except Exception:
        pass
    n = 4
    lens = x["cache_seqlens"][:n].numpy()
    t0 = time.perf_counter()
    oracle.attention_decode(x["q"][:n], x["k"][:n], x["v"][:n], lens, base=w.base, style=w.rope_style)
    dt = time.perf_counter() - t0
    nbytes = W.decode_bytes(w.replace(B=n), lens)
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"float64 numpy oracle decode, sequences 0-{n - 1} of {w.B} (cache lengths "
                  f"{', '.join(str(int(L)) for L in lens)}), {dt:.1f} s",
    }


def decode(torch, cgr, W, dev, steps: int, warmup: int, with_cpu: bool) -> None:
    """One step = one decode call; the cache is filled (keys rotated by
    cgr_rope_rotate) before timing."""
    w = W.DECODE_WORKLOADS[DECODE_WORKLOAD]
    x = W.make_decode_inputs(w)
    B, S, KV, D = x["k"].shape
    cos, sin = cgr.rope_tables(w.capacity, D, w.base, device=dev)
    pos = torch.arange(S, dtype=torch.int32, device=dev).repeat(B)
    kc = cgr.rope_rotate(x["k"].to(dev).reshape(B * S, KV, D), pos, cos, sin,
                         rope_style=w.rope_style).reshape(B, S, KV, D)
    vc = x["v"].to(dev)
    q = x["q"].to(dev)
    lens = x["cache_seqlens"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, w.n_head, w.Tq), dtype=torch.float32, device=dev)
    ws = torch.empty(cgr.cgr_attn_decode_workspace_size(B, w.Tq, x["max_seqlen"], w.n_head, KV, D),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        cgr.gqa_rope_attn_decode(q, kc, vc, lens, x["max_seqlen"], cos, sin, rope_style=w.rope_style,
                                 out=o, lse=lse, workspace=ws)

    # As for the forward: 2 s of back-to-back calls (the sustained clock and
    # power), then the warmup and timed calls with no idle gap.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    clock = ClockSampler()
    clock.measure(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    clock.finish()
    wall = time.perf_counter() - t0
    nbytes = W.decode_bytes(w, x["cache_seqlens"].tolist())
    ms_step = wall * 1e3 / steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": DECODE_METRIC,
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": DECODE_WORKLOAD, "B": B, "Tq": w.Tq, "cache_capacity": S,
            "cache_lengths": f"U[{w.len_lo}, {w.len_hi}], sum {int(x['cache_seqlens'].sum())}",
            "n_head": w.n_head, "n_kv_head": KV, "head_dim": D, "rope_base": w.base,
            "rope_pairs": w.rope_style, "mask": "causal, aligned with the cache end", "io": "bf16",
            "step": "gqa_rope_attn_decode", "bytes_per_step": nbytes,
            "tokens_per_s": round(B * w.Tq / (ms_step * 1e-3), 1),
            "pct_of_peak": round(100.0 * nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "clock_mhz": clock.summary(),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "the decode call: attn_decode_kernel + decode_combine_kernel (head_dim 128, interleaved)",
            "kernel_ms": round(call_ms, 5),
        },
        "cpu_baseline": cpu_baseline_decode(x, w) if with_cpu else None,
    }
    print(json.dumps(result), flush=True)


FP8_WORKLOAD = "fp8_long_context_T8192_H32_KV8_d128"
FP8_METRIC = "causal GQA+RoPE attention fwd with fp8 (e4m3) operands, TFLOP/s on 1 MI355X; % of fp8 MFMA peak"
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published


def fp8(torch, cgr, W, dev, steps: int, warmup: int) -> None:
    """One step = one cgr_gqa_rope_attn_fwd_fp8 call (the key/value tile
    preparation and the attention kernel) on the long-context workload with its
    q, k, v quantized per tensor to e4m3; the RoPE tables are built once."""
    w = W.get(FP8_WORKLOAD)
    x = W.make_fp8_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.n_head, w.T), dtype=torch.float32, device=dev)
    ws = torch.empty(cgr.cgr_attn_fwd_fp8_workspace_size(w.B, w.T, w.n_kv_head, w.head_dim), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        cgr.gqa_rope_attn_fwd_fp8(q, k, v, x["q_descale"], x["k_descale"], x["v_descale"], cos, sin, out=o, lse=lse,
                                  workspace=ws)

    # As for the forward: 2 s of back-to-back calls (the sustained clock and
    # power), then the warmup and timed calls with no idle gap.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    clock = ClockSampler()
    clock.measure(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    clock.finish()
    wall = time.perf_counter() - t0
    flops = W.algorithmic_flops(w.n_head, w.head_dim, [w.T] * w.B, True)
    ms_step = wall * 1e3 / steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    achieved = flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": FP8_METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3",
        "data": "synthetic",
        "config": {
            "workload": FP8_WORKLOAD, "B": w.B, "T": w.T, "n_head": w.n_head, "n_kv_head": w.n_kv_head,
            "head_dim": w.head_dim, "rope_base": w.base, "rope_pairs": w.rope_style, "mask": "causal",
            "io": "e4m3 q/k/v (per-tensor descales), bf16 o", "qk_operand": "e4m3", "pv_operand": "e4m3",
            "accumulate": "f32", "step": "gqa_rope_attn_fwd_fp8", "flops_per_step": flops,
            "pct_of_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 2),
        },
        "roofline": {
            "clock_mhz": clock.summary(),
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": "the fp8 call: fp8_prep_kernel (keys rotated, tile images) + attn_fwd_fp8_kernel "
                      "(head_dim 128, causal, interleaved); HIP events around the call",
            "kernel_ms": round(call_ms, 5),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


QKV_WORKLOAD = "qkv_long_context_T8192_C4096_H32_KV8_d128"
QKV_METRIC = "fused RMSNorm + q/k/v projection + RoPE TFLOP/s on 1 MI355X; % of bf16 MFMA peak"


def cpu_baseline_qkv(x, w) -> dict:
    """The float64 oracle, as it stands, on the first 512 of the 8192 tokens."""
    import oracle

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or None
    except Exception:
        pass
    n = 512
    t0 = time.perf_counter()
    oracle.rmsnorm_qkv_rope(x["x"][:n], x["norm_weight"], w.eps, x["w_qkv"], x["positions"][:n].numpy(),
                            w.n_head, w.n_kv_head, base=w.base, style=w.rope_style)
    dt = time.perf_counter() - t0
    O = (w.n_head + 2 * w.n_kv_head) * w.head_dim
    return {
        "value": round(2.0 * n * w.n_embd * O / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"float64 numpy oracle, tokens 0-{n - 1} of {w.B * w.T}, {dt:.2f} s",
    }


def qkv(torch, cgr, W, dev, steps: int, warmup: int, with_cpu: bool) -> None:
    """One step = one cgr_rmsnorm_qkv_rope call (q and k rotated)."""
    w = W.QKV_WORKLOADS[QKV_WORKLOAD]
    x = W.make_qkv_inputs(w)
    N, C = x["x"].shape
    O = x["w_qkv"].shape[0]
    xs, g, wq, pos = (x[n].to(dev) for n in ("x", "norm_weight", "w_qkv", "positions"))
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=dev)
    q = torch.empty((N, w.n_head, w.head_dim), dtype=torch.bfloat16, device=dev)
    k = torch.empty((N, w.n_kv_head, w.head_dim), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    ws = torch.empty(cgr.cgr_rmsnorm_qkv_rope_workspace_size(N, C, w.n_head, w.n_kv_head, w.head_dim),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        cgr.rmsnorm_qkv_rope(xs, g, w.eps, wq, pos, w.n_head, w.n_kv_head, cos, sin, rope_style=w.rope_style,
                             q=q, k=k, v=v, workspace=ws)

    # As for the forward: 2 s of back-to-back calls (the sustained clock and
    # power), then the warmup and timed calls with no idle gap.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    clock = ClockSampler()
    clock.measure(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    clock.finish()
    wall = time.perf_counter() - t0
    flops = 2 * N * C * O
    ms_step = wall * 1e3 / steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    achieved = flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": QKV_METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": QKV_WORKLOAD, "tokens": N, "n_embd": C, "n_head": w.n_head, "n_kv_head": w.n_kv_head,
            "head_dim": w.head_dim, "rope_base": w.base, "rope_pairs": w.rope_style, "eps": w.eps,
            "rotate": "q and k", "step": "rmsnorm_qkv_rope", "flops_per_step": flops,
            "pct_of_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS, 2),
        },
        "roofline": {
            "clock_mhz": clock.summary(),
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": "the call: qkv_prep_kernel + qkv_gemm_kernel (head_dim 128, interleaved)",
            "kernel_ms": round(call_ms, 5),
        },
        "cpu_baseline": cpu_baseline_qkv(x, w) if with_cpu else None,
    }
    print(json.dumps(result), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--all-configs", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="with --all-configs: also time the calls captured in a HIP graph and replayed")
    ap.add_argument("--only", default=None, help="with --all-configs: this workload only")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--varlen", action="store_true", help="with --backward: the packed MQA batch")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--window", type=int, default=0)
    ap.add_argument("--qkv", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="the long-context forward with e4m3 q/k/v and e4m3 matrix products")
    ap.add_argument("--wide", action="store_true",
                    help="head_dim 256: B=1 T=8192 H=16 KV=8 (the long-context width in wider heads)")
    ap.add_argument("--padded", action="store_true",
                    help="right-padded dense batch: B=4 entries of T=8192, valid lengths U[2048, 8192]")
    ap.add_argument("--qk", choices=("bf16", "f16"), default=None,
                    help="the forward's Q.K^T operand type (default: bf16 for the headline line, else f16)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention of one GPU's head share is the unit that would shard).",
              file=sys.stderr)
        return 2

    import torch

    import causal_gqa_rope_amd as cgr
    import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return 0
    if args.all_configs:
        all_configs(torch, cgr, W, dev, args.steps, args.warmup, graph=args.graph, only=args.only)
        return 0
    if args.backward:
        backward(torch, cgr, W, dev, args.steps, args.warmup, not args.no_cpu_baseline, args.window,
                 varlen=args.varlen)
        return 0
    if args.decode:
        decode(torch, cgr, W, dev, args.steps, args.warmup, not args.no_cpu_baseline)
        return 0
    if args.qkv:
        qkv(torch, cgr, W, dev, args.steps, args.warmup, not args.no_cpu_baseline)
        return 0
    if args.fp8:
        fp8(torch, cgr, W, dev, args.steps, args.warmup)
        return 0

    w = W.get(WIDE_WORKLOAD if args.wide else WORKLOAD)
    seqlens, lens = None, [w.T] * w.B
    if args.padded:
        w = W.custom(PADDED_WORKLOAD, B=4, T=w.T, n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
                     base=w.base, seed=21)
        lens = W.padded_lengths(w.B, 2048, w.T, seed=21)
        seqlens = torch.tensor(lens, dtype=torch.int32, device=dev)
    inputs = W.make_inputs(w)
    q = inputs["q"].to(dev)
    k = inputs["k"].to(dev)
    v = inputs["v"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.n_head, w.T), dtype=torch.float32, device=dev)
    cos = torch.empty((w.T, w.head_dim // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    lib = cgr.library()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def tables():
        cgr._check(lib.cgr_rope_tables(w.T, w.head_dim, w.base, cgr._ptr(cos), cgr._ptr(sin), sptr))

    ws = torch.empty(cgr.cgr_attn_fwd_workspace_size(w.B, w.T, w.n_kv_head, w.head_dim), dtype=torch.uint8,
                     device=dev)
    kw = dict(rope_style=w.rope_style, seqlens=seqlens)

    # The forward with a workspace, in its two halves (the same kernels and bits
    # as one cgr_gqa_rope_attn_fwd call): the key rotation, then the attention
    # kernel alone between its own pair of HIP events.
    headline = args.window == 0 and not args.padded and not args.wide
    # The headline line computes both products on bf16 operands, the type the
    # method's statement names; the library's default Q.K^T operand is f16 (three
    # more mantissa bits, for inputs with large keys), measured beside it.
    qk = args.qk or ("bf16" if headline else "f16")

    def rotate():
        cgr.attn_fwd_rotate_keys(k, cos, sin, ws, qk_operand=qk, **kw)

    def attention():
        cgr.gqa_rope_attn_fwd_rotated(q, k, v, cos, sin, ws, causal=True, window=args.window, out=o, lse=lse,
                                      qk_operand=qk, **kw)

    def step():
        tables()
        rotate()
        attention()

    # The clock under this load: 2 s of back-to-back steps before the warmup
    # steps. From idle the GPU takes a good part of a second to reach the clock
    # it holds under sustained load, so this also keeps the timed steps from
    # measuring that ramp (a few warmup steps alone last only milliseconds).
    # The warmup and timed steps follow it with no host work in between (the
    # events exist beforehand, the clock sampler stops afterwards): even a few
    # idle milliseconds let the clock drop and slow the next ~20 steps.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    clock = ClockSampler()
    clock.measure(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        tables()
        ev[i][0].record(stream)
        rotate()
        ev[i][1].record(stream)
        attention()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.finish()

    flops = W.algorithmic_flops(w.n_head, w.head_dim, lens, True, args.window)
    ms_step = wall * 1e3 / args.steps
    kern = [b.elapsed_time(c) for _, b, c in ev]
    call = [a.elapsed_time(c) for a, _, c in ev]
    rot = [a.elapsed_time(b) for a, b, _ in ev]
    kernel_ms, kernel_med = sum(kern) / len(kern), statistics.median(kern)
    call_ms, call_med = sum(call) / len(call), statistics.median(call)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = read_traffic(qk) if headline else None
    clock_main = clock.summary()

    # The same step with the other Q.K^T operand type: the attention kernel
    # alone, at its own sustained clock and power.
    other_ops, other = None, "f16" if qk == "bf16" else "bf16"
    if headline:
        ws_b = torch.empty_like(ws)

        def step_b():
            tables()
            cgr.attn_fwd_rotate_keys(k, cos, sin, ws_b, qk_operand=other, **kw)
            attention_b()

        def attention_b():
            cgr.gqa_rope_attn_fwd_rotated(q, k, v, cos, sin, ws_b, causal=True, out=o, lse=lse, qk_operand=other,
                                          **kw)

        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        clock.measure(step_b)
        for _ in range(args.warmup):
            step_b()
        torch.cuda.synchronize()
        for i in range(args.steps):
            tables()
            cgr.attn_fwd_rotate_keys(k, cos, sin, ws_b, qk_operand=other, **kw)
            evb[i][0].record(stream)
            attention_b()
            evb[i][1].record(stream)
        torch.cuda.synchronize()
        clock.finish()
        kb = [a.elapsed_time(b) for a, b in evb]
        kb_ms = sum(kb) / len(kb)
        other_ops = {"qk_operand": other, "pv_operand": "bf16", "kernel_ms": round(kb_ms, 5),
                    "kernel_ms_median": round(statistics.median(kb), 5),
                    "achieved": round(flops / (kb_ms * 1e-3) / 1e12, 3),
                    "frac": round(flops / (kb_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4),
                    "clock_mhz": clock.summary()}

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if qk == "bf16" else "f16/bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "T": w.T, "n_head": w.n_head, "n_kv_head": w.n_kv_head,
            "head_dim": w.head_dim, "rope_base": w.base, "rope_pairs": w.rope_style, "mask": "causal",
            "io": "bf16", "qk_operand": qk, "pv_operand": "bf16", "accumulate": "f32",
            **({"valid_lengths": lens} if args.padded else {}),
            "step": "rope_tables + attn_fwd_rotate_keys + gqa_rope_attn_fwd_rotated (= gqa_rope_attn_fwd)",
            "before_warmup": "2 s of untimed steps (the clock_mhz sample), so the timed steps run at the sustained clock",
            "window": args.window, "flops_per_step": flops,
            "pct_of_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": f"attn_fwd_dense_kernel (head_dim {w.head_dim}, bf16 I/O, {qk} QK, causal, {w.rope_style}); "
                      "HIP events around its launch alone, on the launch stream",
            "kernel_ms": round(kernel_ms, 5),
            "kernel_ms_median": round(kernel_med, 5),
            "achieved_at_median": round(flops / (kernel_med * 1e-3) / 1e12, 3),
            "call_ms": round(call_ms, 5),
            "call_ms_median": round(call_med, 5),
            "call_tflops": round(flops / (call_ms * 1e-3) / 1e12, 3),
            "rotate_keys_ms": round(sum(rot) / len(rot), 5),
            "clock_mhz": clock_main,
            **({f"{other}_operands": other_ops} if other_ops else {}),
        },
        "cpu_baseline": None if args.no_cpu_baseline or not headline else cpu_baseline(inputs, w),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
