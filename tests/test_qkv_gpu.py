"""GPU parity of the fused pre-attention step (RMSNorm, q/k/v projections,
RoPE) through the C-ABI against the float64 oracle on the same seeded inputs.

Bar per output tensor (as for the backward): max |got - ref| <= 2e-2 max |ref|
and ||got - ref||_F <= 1e-2 ||ref||_F. The arithmetic rounds W diag(norm
weight) once to bf16 (relative 2^-9 per weight, independent across the
C-term sums) and each output once to bf16 (2^-9): a few 1e-3 of the scale.
"""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, assert_close, f64
from tests.test_bwd_gpu import grad_errors

pytestmark = pytest.mark.gpu

TOL = dict(norm_max=2e-2, rel_fro=1e-2)


def check(name, got, ref):
    msgs, ok = [], True
    for n, g, r in zip(("q", "k", "v"), got, ref):
        assert np.isfinite(g).all(), f"{name}: non-finite {n}"
        nm, rf = grad_errors(g, r)
        msgs.append(f"{n}: max {nm:.2e} of max|ref| {np.abs(r).max():.3g}, rel fro {rf:.2e}")
        ok = ok and nm <= TOL["norm_max"] and rf <= TOL["rel_fro"]
    msg = f"{name}: " + "; ".join(msgs)
    print(msg, flush=True)
    assert ok, msg


def run(w, x, dev, rotate_q=True, rotate_k=True):
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=dev)
    return cgr.rmsnorm_qkv_rope(x["x"].to(dev), x["norm_weight"].to(dev), w.eps, x["w_qkv"].to(dev),
                                x["positions"].to(dev), w.n_head, w.n_kv_head, cos, sin, rope_style=w.rope_style,
                                rotate_q=rotate_q, rotate_k=rotate_k)


def ref(w, x, rotate_q=True, rotate_k=True):
    return oracle.rmsnorm_qkv_rope(x["x"], x["norm_weight"], w.eps, x["w_qkv"], x["positions"].numpy(),
                                   w.n_head, w.n_kv_head, base=w.base, style=w.rope_style, rotate_q=rotate_q,
                                   rotate_k=rotate_k)


@pytest.mark.parametrize("name", list(W.QKV_WORKLOADS))
def test_qkv_workload_full(gpu, name):
    """Both workloads in full, the long-context one in the benchmark's launch configuration."""
    w = W.QKV_WORKLOADS[name]
    announce(f"rmsnorm_qkv_rope {name}")
    x = W.make_qkv_inputs(w)
    got = run(w, x, gpu)
    check(name, [f64(t) for t in got], ref(w, x))


# (B, T, C, H, KV, d, style, rotate q, rotate k): ragged token counts (not a
# multiple of the 256-token tile), n_embd down to one 32-wide step and widths
# that are not a multiple of 64 (the 32-wide K-step instance), output features
# that end inside a 256-feature tile, heads that split a tile across q/k/v,
# every head_dim, both pairings, each rotation choice.
EDGE = [
    (1, 300, 256, 4, 2, 64, "interleaved", True, True),
    (2, 260, 160, 6, 2, 64, "interleaved", True, True),
    (3, 77, 32, 2, 1, 32, "half", True, False),
    (1, 513, 384, 6, 3, 64, "half", False, True),
    (2, 129, 512, 4, 4, 128, "interleaved", False, False),
    (1, 1, 128, 8, 1, 128, "half", True, True),
]


@pytest.mark.parametrize("B,T,C,H,KV,d,style,rq,rk", EDGE,
                         ids=[f"B{e[0]}_T{e[1]}_C{e[2]}_H{e[3]}_KV{e[4]}_d{e[5]}_{e[6]}_q{int(e[7])}k{int(e[8])}"
                              for e in EDGE])
def test_qkv_edge_shapes(gpu, B, T, C, H, KV, d, style, rq, rk):
    w = W.QkvWorkload(f"qkv_edge_T{T}_C{C}", B=B, T=T, n_embd=C, n_head=H, n_kv_head=KV, head_dim=d,
                      base=10000.0, seed=90 + T + C, rope_style=style)
    announce(f"rmsnorm_qkv_rope edge {w}")
    x = W.make_qkv_inputs(w)
    got = run(w, x, gpu, rq, rk)
    check(w.name, [f64(t) for t in got], ref(w, x, rq, rk))


def test_qkv_feeds_the_attention_forward(gpu):
    """RMSNorm + projections (RoPE left to the attention call) into the HIP
    forward, against the oracle's same two steps."""
    w = W.QKV_WORKLOADS["qkv_nanollama3_B8_T256_C384_H6_KV3_d64"]
    announce("rmsnorm_qkv_rope -> gqa_rope_attn_fwd, nanollama3 block")
    x = W.make_qkv_inputs(w)
    q, k, v = run(w, x, gpu, rotate_q=False, rotate_k=False)
    B, T, d = w.B, w.T, w.head_dim
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(q.view(B, T, w.n_head, d), k.view(B, T, w.n_kv_head, d),
                                   v.view(B, T, w.n_kv_head, d), cos, sin)
    rq, rk, rv = ref(w, x, False, False)
    ro, rl = oracle.attention_dense(rq.reshape(B, T, w.n_head, d), rk.reshape(B, T, w.n_kv_head, d),
                                    rv.reshape(B, T, w.n_kv_head, d), causal=True, base=w.base)
    assert_close("qkv->attention", f64(o), ro, f64(lse), rl, "bf16")


def test_qkv_bad_position_reports_and_leaves_row(gpu):
    w = W.QkvWorkload("qkv_bad", B=1, T=40, n_embd=64, n_head=2, n_kv_head=1, head_dim=32, base=1e4, seed=5)
    x = W.make_qkv_inputs(w)
    pos = x["positions"].clone()
    pos[7] = 40  # tables cover 40 positions: 0 .. 39
    cos, sin = cgr.rope_tables(40, 32, 1e4, device=gpu)
    q = torch.full((40, 2, 32), 3.0, dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(cgr.cgr_rmsnorm_qkv_rope_workspace_size(40, 64, 2, 1, 32), dtype=torch.uint8, device=gpu)
    cgr.rmsnorm_qkv_rope(x["x"].to(gpu), x["norm_weight"].to(gpu), w.eps, x["w_qkv"].to(gpu), pos.to(gpu), 2, 1,
                         cos, sin, q=q, workspace=ws)
    assert cgr.cgr_varlen_device_status(ws) == 1
    assert torch.all(q[7] == 3.0)
    rq, _, _ = ref(w, x)
    keep = [i for i in range(40) if i != 7]
    assert np.abs(f64(q)[keep] - rq[keep]).max() <= 2e-2 * np.abs(rq).max()
    cgr.rmsnorm_qkv_rope(x["x"].to(gpu), x["norm_weight"].to(gpu), w.eps, x["w_qkv"].to(gpu),
                         x["positions"].to(gpu), 2, 1, cos, sin, workspace=ws)
    assert cgr.cgr_varlen_device_status(ws) == 0
