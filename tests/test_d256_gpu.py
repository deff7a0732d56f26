"""GPU parity of the head_dim 256 forward (bf16 I/O) through the C-ABI against
the float64 oracle on the same seeded inputs: dense and packed batches, both
masks and pairings, both Q.K^T operand types, a sliding window, right padding,
and the full-size long-context workload in the launch configuration the
benchmark times (sampled rows). Bar: the forward's bf16 bar (max abs 2e-2 and
median relative 5e-3 on O, max abs 2e-2 on the LSE)."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, assert_close, f64

pytestmark = pytest.mark.gpu

# (B, T, H, KV, causal, style, qk, window, workspace): ragged T across the
# 128-row unit and 32-key tile, GQA/MQA/MHA, no mask, bf16 Q.K^T, a window,
# with and without the once-rotated keys, one-token sequences.
DENSE = [
    (2, 300, 8, 2, True, "interleaved", "f16", 0, True),
    (1, 1000, 4, 1, True, "half", "f16", 0, False),
    (2, 129, 4, 4, False, "interleaved", "f16", 0, True),
    (1, 77, 2, 1, True, "half", "bf16", 0, True),
    (1, 700, 4, 2, True, "interleaved", "f16", 100, True),
    (3, 1, 2, 1, True, "interleaved", "f16", 0, True),
]


@pytest.mark.parametrize("B,T,H,KV,causal,style,qk,win,ws", DENSE,
                         ids=[f"B{c[0]}_T{c[1]}_H{c[2]}_KV{c[3]}_{'causal' if c[4] else 'nomask'}_{c[5]}_{c[6]}_"
                              f"W{c[7]}_{'ws' if c[8] else 'nows'}" for c in DENSE])
def test_d256_dense(gpu, B, T, H, KV, causal, style, qk, win, ws):
    w = W.custom(f"d256_T{T}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=256, base=500000.0, causal=causal,
                 rope_style=style, seed=500 + T + H)
    announce(f"d256 dense {w.name} B{B} H{H} KV{KV} causal={causal} {style} qk={qk} W={win} ws={ws}")
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(T, 256, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(x["q"].to(gpu), x["k"].to(gpu), x["v"].to(gpu), cos, sin, causal=causal,
                                   rope_style=style, qk_operand=qk, window=win,
                                   workspace=None if ws else False)
    ro, rl = oracle.attention_dense(x["q"], x["k"], x["v"], causal=causal, base=w.base, style=style,
                                    window=win)
    assert_close(w.name, f64(o), ro, f64(lse), rl, "bf16")


def test_d256_packed(gpu):
    lens = [5, 300, 1, 700, 0, 129]
    H, KV, d = 4, 2, 256
    gen = torch.Generator("cpu").manual_seed(71)
    total = sum(lens)
    q = torch.randn((total, H, d), generator=gen).to(torch.bfloat16)
    k = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    announce(f"d256 packed lens={lens}")
    cos, sin = cgr.rope_tables(max(lens), d, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cu.to(gpu), max(lens), cos, sin)
    ro, rl = oracle.attention_varlen(q, k, v, cu.numpy(), causal=True, base=1e4)
    assert_close("d256 packed", f64(o), ro, f64(lse), rl, "bf16")


def test_d256_padded(gpu):
    lens = [300, 0, 129, 33]
    w = W.custom("d256_pad", B=4, T=300, n_head=4, n_kv_head=2, head_dim=256, base=1e4, seed=77)
    announce(f"d256 padded lens={lens}")
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(300, 256, 1e4, device=gpu)
    q, k, v = (x[n].to(gpu) for n in ("q", "k", "v"))
    o = torch.full_like(q, 7.0)
    lse = torch.full((4, 4, 300), 7.0, dtype=torch.float32, device=gpu)
    cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, out=o, lse=lse,
                          seqlens=torch.tensor(lens, dtype=torch.int32, device=gpu))
    ro, rl = oracle.attention_padded(x["q"], x["k"], x["v"], lens, base=1e4)
    go, gl = f64(o), f64(lse)
    for b, n in enumerate(lens):
        assert (go[b, n:] == 7.0).all() and (gl[b, :, n:] == 7.0).all()
    assert_close("d256 padded", np.concatenate([go[b, :n].ravel() for b, n in enumerate(lens)]),
                 np.concatenate([ro[b, :n].ravel() for b, n in enumerate(lens)]),
                 np.concatenate([gl[b, :, :n].ravel() for b, n in enumerate(lens)]),
                 np.concatenate([rl[b, :, :n].ravel() for b, n in enumerate(lens)]), "bf16")


def test_d256_pre_rotated_keys_give_the_same_bits(gpu):
    w = W.custom("d256_bits", B=1, T=500, n_head=4, n_kv_head=2, head_dim=256, base=5e5, seed=79)
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(500, 256, w.base, device=gpu)
    q, k, v = (x[n].to(gpu) for n in ("q", "k", "v"))
    o1, l1 = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, workspace=False)
    o2, l2 = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_d256_long_context_full_size_sampled(gpu):
    """The head_dim 256 long-context workload in the benchmark's launch configuration, sampled rows."""
    w = W.get("long_context_T8192_H16_KV8_d256")
    announce(f"{w.name}: full-size run, sampled rows")
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(x["q"].to(gpu), x["k"].to(gpu), x["v"].to(gpu), cos, sin)
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(8)
    ts = [0, 1, 31, 32, 127, 128, 4095, 8063, 8064, 8191] + [int(t) for t in rng.integers(0, w.T, 30)]
    rows = [(0, t, int(rng.integers(0, w.n_head))) for t in ts] + [(0, 8191, h) for h in range(w.n_head)]
    ro, rl = oracle.attention_rows(x["q"], x["k"], x["v"], rows, causal=True, base=w.base)
    go = np.stack([o[b, t, h] for (b, t, h) in rows])
    gl = np.array([lse[b, h, t] for (b, t, h) in rows])
    assert_close(w.name + " (sampled)", go, ro, gl, rl, "bf16")
