"""GPU parity of the backward: dq, dk, dv from the HIP path through the C-ABI
against the float64 oracle's chain rule, on the same seeded q, k, v and dL/dO.

The forward that feeds the backward (o, lse) is the HIP forward, as in
training; the oracle recomputes everything from q, k, v and dL/dO alone.

Bar (per gradient tensor, derived from an emulation of the kernels' rounding
points on these workloads: f16 rotated q/k, bf16 P, f16 dS, f32 sums, one
bf16 rounding of each output, D from the bf16 O; the emulation reaches at most
7.4e-3 and 4.7e-3):
  max |got - ref| <= 2e-2 * max |ref|, and ||got - ref||_F <= 1e-2 ||ref||_F.
"""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, f64, to_dev

pytestmark = pytest.mark.gpu

BWD_TOL = dict(norm_max=2e-2, rel_fro=1e-2)


def grad_errors(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    scale = float(np.abs(ref).max())
    norm_max = float(diff.max()) / scale if scale > 0 else float(diff.max())
    nrm = float(np.linalg.norm(ref))
    rel_fro = float(np.linalg.norm(got - ref)) / nrm if nrm > 0 else float(np.linalg.norm(got - ref))
    return norm_max, rel_fro


def assert_grads_close(name, got, ref):
    msgs = []
    ok = True
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), f"{name}: non-finite {n}"
        nm, rf = grad_errors(g, r)
        msgs.append(f"{n}: max {nm:.2e} of max|ref| {np.abs(r).max():.3g}, rel fro {rf:.2e}")
        ok = ok and nm <= BWD_TOL["norm_max"] and rf <= BWD_TOL["rel_fro"]
    msg = f"{name}: " + "; ".join(msgs)
    print(msg, flush=True)
    assert ok, msg


def fwd_bwd(w, x, dev, qk="f16"):
    """HIP forward then HIP backward; returns (dq, dk, dv) on the device and dL/dO on the CPU."""
    d = to_dev(x, dev)
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=dev)
    o, lse = cgr.gqa_rope_attn_fwd(d["q"], d["k"], d["v"], cos, sin, causal=w.causal,
                                   rope_style=w.rope_style, qk_operand=qk)
    dout = W.make_dout(w, x["q"])
    grads = cgr.gqa_rope_attn_bwd(d["q"], d["k"], d["v"], o, lse, dout.to(dev), cos, sin,
                                  causal=w.causal, rope_style=w.rope_style, qk_operand=qk)
    return grads, dout


def oracle_bwd(w, x, dout):
    return oracle.attention_dense_bwd(x["q"], x["k"], x["v"], dout, causal=w.causal, base=w.base,
                                      style=w.rope_style)


BF16_WORKLOADS = ["nanollama3_train_B8_T256_H6_KV2_d64", "nanollama3_pages_B8_T256_H6_KV3_d64",
                  "nanollama3_train_B8_T256_H6_KV2_d64_half", "nanollama3_train_B8_T256_H6_KV2_d64_nomask",
                  "qwen05b_prefill_T77_H14_KV2_d64_koutliers",
                  "qwen05b_prefill_T77_H14_KV2_d64_koutliers_half"]


@pytest.mark.parametrize("name", BF16_WORKLOADS)
def test_backward_workload_full(gpu, name):
    w = W.get(name)
    announce(f"backward {name}: full comparison")
    x = W.make_inputs(w)
    grads, dout = fwd_bwd(w, x, gpu)
    assert_grads_close(name, [f64(g) for g in grads], oracle_bwd(w, x, dout))


# (T, H, KV, d, causal, style, B): single and two tokens, tile and block
# boundaries (32-row steps, 64-key tiles, 128-key and 256-row blocks), ragged
# tails, MHA, GQA, MQA, every head_dim, both masks and pairings, B > 1.
EDGE = [
    (1, 4, 2, 64, True, "interleaved", 1),
    (2, 2, 1, 128, True, "interleaved", 1),
    (31, 8, 8, 128, True, "interleaved", 1),
    (65, 8, 1, 128, True, "half", 1),
    (129, 4, 2, 32, True, "interleaved", 1),
    (129, 4, 2, 32, False, "half", 1),
    (300, 8, 2, 128, True, "interleaved", 1),
    (300, 8, 2, 128, False, "interleaved", 1),
    (521, 4, 4, 64, True, "half", 1),
    (1000, 8, 2, 128, True, "interleaved", 1),
    (200, 6, 2, 64, True, "interleaved", 3),
]


@pytest.mark.parametrize("T,H,KV,d,causal,style,B", EDGE,
                         ids=[f"T{e[0]}_H{e[1]}_KV{e[2]}_d{e[3]}_{'causal' if e[4] else 'nomask'}_{e[5]}_B{e[6]}"
                              for e in EDGE])
def test_backward_edge_shapes(gpu, T, H, KV, d, causal, style, B):
    w = W.custom(f"bwd_edge_T{T}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, causal=causal,
                 rope_style=style, seed=100 + T + d)
    announce(f"backward edge {w}")
    x = W.make_inputs(w)
    grads, dout = fwd_bwd(w, x, gpu)
    assert_grads_close(w.name, [f64(g) for g in grads], oracle_bwd(w, x, dout))


def test_backward_bf16_qk_operand(gpu):
    w = W.get("nanollama3_train_B8_T256_H6_KV2_d64")
    announce("backward with bf16 Q.K^T operands")
    x = W.make_inputs(w)
    grads, dout = fwd_bwd(w, x, gpu, qk="bf16")
    assert_grads_close(w.name + "_qkbf16", [f64(g) for g in grads], oracle_bwd(w, x, dout))


def test_backward_is_deterministic(gpu):
    w = W.custom("bwd_det", T=700, n_head=8, n_kv_head=2, head_dim=128, seed=5)
    announce("backward determinism, T=700 H8 KV2 d128")
    x = W.make_inputs(w)
    (dq1, dk1, dv1), _ = fwd_bwd(w, x, gpu)
    (dq2, dk2, dv2), _ = fwd_bwd(w, x, gpu)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def test_backward_long_context_full_size(gpu):
    """The long-context workload at full size, in the launch configuration the
    benchmark times: every gradient of two whole K/V groups (the group's 4 query
    heads for dq, its K/V head for dk and dv) against the oracle, the rest
    checked finite."""
    w = W.get("long_context_T8192_H32_KV8_d128")
    announce(f"backward {w.name}: full size, K/V groups 0 and 7 in full")
    x = W.make_inputs(w)
    grads, dout = fwd_bwd(w, x, gpu)
    dq, dk, dv = (f64(g) for g in grads)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    G = w.n_head // w.n_kv_head
    for kv in (0, 7):
        rq, rk, rv = oracle.attention_bwd_group(x["q"], x["k"], x["v"], dout, 0, kv, causal=True,
                                                base=w.base)
        assert_grads_close(f"{w.name} kv{kv}", [dq[0, :, kv * G:(kv + 1) * G], dk[0, :, kv], dv[0, :, kv]],
                           [rq, rk, rv])


def test_backward_binding_checks(gpu):
    w = W.custom("bwd_chk", T=16, n_head=4, n_kv_head=2, head_dim=64)
    x = to_dev(W.make_inputs(w), gpu)
    cos, sin = cgr.rope_tables(16, 64, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin)
    with pytest.raises(cgr.CgrError):  # f32 tensors
        cgr.gqa_rope_attn_bwd(x["q"].float(), x["k"], x["v"], o, lse, o, cos, sin)
    with pytest.raises(cgr.CgrError):  # dout of the wrong shape
        cgr.gqa_rope_attn_bwd(x["q"], x["k"], x["v"], o, lse, o[:, :8].contiguous(), cos, sin)
    with pytest.raises(cgr.CgrError):  # workspace too small
        cgr.gqa_rope_attn_bwd(x["q"], x["k"], x["v"], o, lse, o, cos, sin,
                              workspace=torch.empty(256, dtype=torch.uint8, device=gpu))
