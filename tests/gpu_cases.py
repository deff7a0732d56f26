"""Shared helpers of the GPU parity tests: run a workload through the HIP path
(the C-ABI via the Python binding) and through the float64 oracle on the same
seeded inputs, and measure the difference."""

from __future__ import annotations

import sys

import numpy as np
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W

# Tolerances of the comparison (max abs error over all O elements; median
# relative error over the nonzero oracle elements; LSE by max abs error).
TOL = {
    "f32": dict(max_abs=1e-4, med_rel=None),
    "bf16": dict(max_abs=2e-2, med_rel=5e-3),
}


def announce(msg: str) -> None:
    print(f"\n[gpu case] {msg}", file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    nz = ref != 0
    med = float(np.median(diff[nz] / np.abs(ref[nz]))) if nz.any() else 0.0
    return float(diff.max()) if diff.size else 0.0, med


def assert_close(name, o, ref_o, lse, ref_lse, dtype):
    tol = TOL[dtype]
    assert np.isfinite(o).all(), f"{name}: non-finite output"
    mx, med = errors(o, ref_o)
    lmx, _ = errors(lse, ref_lse)
    msg = f"{name}: O max abs {mx:.3e}, median rel {med:.3e}; LSE max abs {lmx:.3e}"
    print(msg, file=sys.stderr, flush=True)
    assert mx <= tol["max_abs"], msg
    if tol["med_rel"] is not None:
        assert med <= tol["med_rel"], msg
    assert lmx <= tol["max_abs"], msg
    return mx, med, lmx


def to_dev(inputs: dict, dev) -> dict:
    out = dict(inputs)
    for key in ("q", "k", "v", "cu_seqlens"):
        if key in inputs:
            out[key] = inputs[key].to(dev)
    return out


def run_gpu(w: W.Workload, inputs: dict, dev, qk_operand: str = "f16", scale=None):
    """The HIP path on a workload's tensors (already on `dev`). Returns torch (o, lse)."""
    max_pos = inputs["max_seqlen"] if w.varlen else w.T
    cos, sin = cgr.rope_tables(max(max_pos, 1), w.head_dim, w.base, device=dev)
    if w.varlen:
        return cgr.gqa_rope_attn_fwd_varlen(
            inputs["q"], inputs["k"], inputs["v"], inputs["cu_seqlens"], inputs["max_seqlen"], cos,
            sin, causal=w.causal, rope_style=w.rope_style, qk_operand=qk_operand,
            softmax_scale=scale)
    return cgr.gqa_rope_attn_fwd(inputs["q"], inputs["k"], inputs["v"], cos, sin, causal=w.causal,
                                 rope_style=w.rope_style, qk_operand=qk_operand,
                                 softmax_scale=scale)


def run_oracle(w: W.Workload, inputs: dict, scale=None):
    if w.varlen:
        return oracle.attention_varlen(inputs["q"], inputs["k"], inputs["v"],
                                       inputs["cu_seqlens"].numpy(), causal=w.causal, base=w.base,
                                       style=w.rope_style, scale=scale)
    return oracle.attention_dense(inputs["q"], inputs["k"], inputs["v"], causal=w.causal,
                                  base=w.base, style=w.rope_style, scale=scale)


def default_grid(B: int, T: int, H: int, KV: int, d: int) -> int:
    """Workgroups of a dense bf16 call on the default (8-wave) instances: units
    of hp heads x 256/hp query rows, hp the largest power of two <= 8 dividing
    the group size. The library runs calls whose count is below the device's
    compute units on its 4-wave instances (without window or split entries)."""
    nw = 4 if d == 256 else 8
    G, hp = H // KV, 1
    while 2 * hp <= nw and G % (2 * hp) == 0:
        hp *= 2
    bm = 32 * nw // hp
    return -(-T // bm) * B * (H // hp)


def compute_units(dev) -> int:
    return torch.cuda.get_device_properties(dev).multi_processor_count
