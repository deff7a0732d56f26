"""GPU parity of decode against a KV cache and of RoPE on rows at given
positions: the HIP path through the C-ABI against the float64 oracle on the
same seeded inputs.

The cache is built the way a server appends to it: the un-rotated keys go
through cgr_rope_rotate at their positions (HIP), then cgr_gqa_rope_attn_decode
attends the new queries to it. The oracle sees only the un-rotated q, k, v and
the cache lengths. Bar: the forward's bf16 bar (max abs 2e-2 and median
relative 5e-3 on O, max abs 2e-2 on the LSE).
"""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, assert_close, f64

pytestmark = pytest.mark.gpu


def build_cache(k, base, d, capacity, dev, style):
    """Rotate every cache row at its position with the HIP kernel."""
    B, S, KV, D = k.shape
    cos, sin = cgr.rope_tables(capacity, d, base, device=dev)
    pos = torch.arange(S, dtype=torch.int32, device=dev).repeat(B)
    kr = cgr.rope_rotate(k.to(dev).reshape(B * S, KV, D), pos, cos, sin, rope_style=style).reshape(B, S, KV, D)
    return kr, cos, sin


def run_decode(w, x, dev):
    kr, cos, sin = build_cache(x["k"], w.base, w.head_dim, w.capacity, dev, w.rope_style)
    return cgr.gqa_rope_attn_decode(x["q"].to(dev), kr, x["v"].to(dev), x["cache_seqlens"].to(dev),
                                    x["max_seqlen"], cos, sin, rope_style=w.rope_style)


def oracle_decode(w, x):
    return oracle.attention_decode(x["q"], x["k"], x["v"], x["cache_seqlens"].numpy(), base=w.base,
                                   style=w.rope_style)


def custom(name, lens, **kw):
    w = W.DecodeWorkload(name, **kw, len_lo=0, len_hi=0)
    gen = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.Tq, w.n_head, w.head_dim), generator=gen)
    k = torch.randn((w.B, w.capacity, w.n_kv_head, w.head_dim), generator=gen)
    v = torch.randn((w.B, w.capacity, w.n_kv_head, w.head_dim), generator=gen)
    x = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16),
             cache_seqlens=torch.tensor(lens, dtype=torch.int32), max_seqlen=max(lens))
    return w, x


# (B, Tq, capacity, H, KV, d, lengths, style, base): one-token caches, lengths
# at and around the 32-key tile, ragged tails, several chunks per sequence,
# GQA/MHA/MQA, more query rows than one 32-column block (MQA with Tq = 4),
# every head_dim, both pairings.
CASES = [
    (4, 1, 300, 8, 2, 128, [1, 37, 256, 300], "interleaved", 10000.0),
    (3, 4, 200, 16, 1, 64, [4, 100, 200], "half", 10000.0),
    (2, 3, 129, 6, 3, 32, [129, 64], "interleaved", 1e6),
    (5, 1, 1000, 14, 2, 64, [31, 32, 33, 999, 1000], "interleaved", 1e6),
    (2, 2, 4100, 8, 8, 128, [4100, 2049], "half", 500000.0),
    (1, 1, 8192, 16, 1, 128, [8192], "interleaved", 10000.0),
]


@pytest.mark.parametrize("B,Tq,S,H,KV,d,lens,style,base", CASES,
                         ids=[f"B{c[0]}_Tq{c[1]}_S{c[2]}_H{c[3]}_KV{c[4]}_d{c[5]}_{c[7]}" for c in CASES])
def test_decode_cases(gpu, B, Tq, S, H, KV, d, lens, style, base):
    w, x = custom(f"decode_B{B}_Tq{Tq}_S{S}", lens, B=B, Tq=Tq, capacity=S, n_head=H, n_kv_head=KV,
                  head_dim=d, base=base, seed=7 + S + d, rope_style=style)
    announce(f"decode {w.name} H{H} KV{KV} d{d} lens={lens} {style}")
    o, lse = run_decode(w, x, gpu)
    ro, rl = oracle_decode(w, x)
    assert_close(w.name, f64(o), ro, f64(lse), rl, "bf16")


def test_decode_workload_full_size(gpu):
    """The benchmark's decode workload in its launch configuration, every output row."""
    w = W.DECODE_WORKLOADS["decode_B16_Tq1_cache4096to8192_H32_KV8_d128"]
    announce(f"decode {w.name}: full size, every row")
    x = W.make_decode_inputs(w)
    o, lse = run_decode(w, x, gpu)
    ro, rl = oracle_decode(w, x)
    assert_close(w.name, f64(o), ro, f64(lse), rl, "bf16")


def test_decode_matches_forward_last_rows(gpu):
    """Decode of the last Tq tokens equals the HIP forward's last Tq rows on the
    same tokens to within the two kernels' rounding (both against the oracle)."""
    T, H, KV, d = 700, 8, 2, 128
    wf = W.custom("fwd_700", T=T, n_head=H, n_kv_head=KV, head_dim=d, seed=31)
    xf = W.make_inputs(wf)
    cos, sin = cgr.rope_tables(T, d, wf.base, device=gpu)
    of, lf = cgr.gqa_rope_attn_fwd(xf["q"].to(gpu), xf["k"].to(gpu), xf["v"].to(gpu), cos, sin)
    Tq = 5
    kr, cos2, sin2 = build_cache(xf["k"], wf.base, d, T, gpu, "interleaved")
    od, ld = cgr.gqa_rope_attn_decode(xf["q"][:, T - Tq:].contiguous().to(gpu), kr, xf["v"].to(gpu),
                                      torch.tensor([T], dtype=torch.int32, device=gpu), T, cos2, sin2)
    assert np.abs(f64(od) - f64(of)[:, T - Tq:]).max() <= 2e-2
    assert np.abs(f64(ld) - f64(lf)[:, :, T - Tq:]).max() <= 2e-2


def test_decode_bad_lengths_report_and_leave_output(gpu):
    w, x = custom("decode_bad", [5, 2, 40], B=3, Tq=3, capacity=40, n_head=4, n_kv_head=2, head_dim=64,
                  base=1e4, seed=3)
    kr, cos, sin = build_cache(x["k"], w.base, 64, 40, gpu, "interleaved")
    poison = torch.full((3, 3, 4, 64), 7.0, dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(cgr.cgr_attn_decode_workspace_size(3, 3, 40, 4, 2, 64), dtype=torch.uint8, device=gpu)
    lens = torch.tensor([5, 2, 40], dtype=torch.int32, device=gpu)  # 2 < Tq
    o, _ = cgr.gqa_rope_attn_decode(x["q"].to(gpu), kr, x["v"].to(gpu), lens, 40, cos, sin, out=poison,
                                    workspace=ws)
    assert cgr.cgr_varlen_device_status(ws) == 1
    assert torch.all(o[1] == 7.0)
    ro, _ = oracle.attention_decode(x["q"][[0, 2]], x["k"][[0, 2]], x["v"][[0, 2]], [5, 40], base=w.base)
    assert np.abs(f64(o[[0, 2]]) - ro).max() <= 2e-2
    lens_ok = torch.tensor([5, 3, 40], dtype=torch.int32, device=gpu)
    cgr.gqa_rope_attn_decode(x["q"].to(gpu), kr, x["v"].to(gpu), lens_ok, 40, cos, sin, workspace=ws)
    assert cgr.cgr_varlen_device_status(ws) == 0


def test_decode_is_deterministic(gpu):
    w, x = custom("decode_det", [3000, 1500], B=2, Tq=2, capacity=3000, n_head=8, n_kv_head=2,
                  head_dim=128, base=1e4, seed=9)
    o1, l1 = run_decode(w, x, gpu)
    o2, l2 = run_decode(w, x, gpu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,d,style", [(torch.bfloat16, 128, "interleaved"), (torch.float32, 64, "half"),
                                           (torch.bfloat16, 32, "half"), (torch.float32, 128, "interleaved")])
def test_rope_rotate(gpu, dtype, d, style):
    announce(f"rope_rotate {dtype} d{d} {style}")
    gen = torch.Generator("cpu").manual_seed(d)
    N, nh, P = 257, 3, 5000
    x = torch.randn((N, nh, d), generator=gen).to(dtype)
    pos = torch.randint(0, P, (N,), generator=gen, dtype=torch.int32)
    cos, sin = cgr.rope_tables(P, d, 5e5, device=gpu)
    out = cgr.rope_rotate(x.to(gpu), pos.to(gpu), cos, sin, rope_style=style)
    ref = oracle.apply_rope(x.double().numpy(), pos.numpy(), 5e5, style)
    # f32 tables, f32 arithmetic, one rounding to the I/O type.
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(f64(out) - ref).max() <= tol


def test_rope_rotate_bad_position(gpu):
    cos, sin = cgr.rope_tables(16, 64, 1e4, device=gpu)
    x = torch.ones((3, 2, 64), dtype=torch.bfloat16, device=gpu)
    out = torch.full_like(x, 5.0)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    cgr.rope_rotate(x, torch.tensor([0, 16, 3], dtype=torch.int32, device=gpu), cos, sin, out=out,
                    status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert torch.all(out[1] == 5.0) and torch.all(out[0] == 1.0)


def test_decode_head_major_cache_layout(gpu):
    """A head-major [B, KV, S, d] cache passed as a strided [B, S, KV, d] view."""
    w, x = custom("decode_hm", [700, 333, 1], B=3, Tq=1, capacity=700, n_head=8, n_kv_head=4, head_dim=128,
                  base=1e4, seed=12)
    kr, cos, sin = build_cache(x["k"], w.base, 128, 700, gpu, "interleaved")
    khm = kr.transpose(1, 2).contiguous().transpose(1, 2)
    vhm = x["v"].to(gpu).transpose(1, 2).contiguous().transpose(1, 2)
    assert khm.stride(1) == 128 and khm.stride(2) == 700 * 128
    o, lse = cgr.gqa_rope_attn_decode(x["q"].to(gpu), khm, vhm, x["cache_seqlens"].to(gpu), 700, cos, sin)
    ro, rl = oracle_decode(w, x)
    assert_close(w.name, f64(o), ro, f64(lse), rl, "bf16")
