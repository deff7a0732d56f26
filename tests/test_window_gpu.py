"""GPU parity of the causal sliding window (keys 0 <= i - j < W) in the
forward (dense, packed, f32 and bf16), the backward and decode, against the
float64 oracle with the same window. Bars: those of the unwindowed tests."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, assert_close, f64, to_dev
from tests.test_bwd_gpu import assert_grads_close

pytestmark = pytest.mark.gpu

# (T, H, KV, d, window, io, style): windows shorter than a key tile, across
# tile and block boundaries, W = 1 (each row sees itself), W = T (plain
# causal), every head_dim, both pairings, f32 and bf16.
FWD = [
    (300, 8, 2, 128, 64, "bf16", "interleaved"),
    (1000, 8, 2, 128, 257, "bf16", "interleaved"),
    (521, 4, 4, 64, 1, "bf16", "half"),
    (129, 4, 2, 32, 31, "f32", "interleaved"),
    (700, 6, 3, 64, 700, "bf16", "interleaved"),
    (2048, 16, 4, 128, 1000, "bf16", "half"),
    (200, 4, 1, 128, 50, "f32", "half"),
]


@pytest.mark.parametrize("T,H,KV,d,win,io,style", FWD,
                         ids=[f"T{c[0]}_H{c[1]}_KV{c[2]}_d{c[3]}_W{c[4]}_{c[5]}_{c[6]}" for c in FWD])
def test_window_forward_dense(gpu, T, H, KV, d, win, io, style):
    w = W.custom(f"win_T{T}_W{win}", T=T, n_head=H, n_kv_head=KV, head_dim=d, dtype=io, rope_style=style,
                 seed=40 + T + win)
    announce(f"window forward {w.name} H{H} KV{KV} d{d} {io} {style}")
    x = W.make_inputs(w)
    d_ = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(d_["q"], d_["k"], d_["v"], cos, sin, rope_style=style, window=win)
    ro, rl = oracle.attention_dense(x["q"], x["k"], x["v"], causal=True, base=w.base, style=style, window=win)
    assert_close(w.name, f64(o), ro, f64(lse), rl, io)


def test_window_forward_packed(gpu):
    lens = [5, 300, 1, 2000, 77, 0, 129]
    win = 128
    gen = torch.Generator("cpu").manual_seed(61)
    total, H, KV, d = sum(lens), 8, 2, 128
    q = torch.randn((total, H, d), generator=gen).to(torch.bfloat16)
    k = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    announce(f"window forward packed lens={lens} W={win}")
    cos, sin = cgr.rope_tables(max(lens), d, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cu.to(gpu), max(lens), cos, sin,
                                          window=win)
    ro, rl = oracle.attention_varlen(q, k, v, cu.numpy(), causal=True, base=1e4, window=win)
    assert_close("packed window", f64(o), ro, f64(lse), rl, "bf16")


def test_window_forward_full_size_sampled(gpu):
    """The long-context workload with a 1024-token window, sampled rows."""
    w = W.get("long_context_T8192_H32_KV8_d128")
    win = 1024
    announce(f"{w.name} with window {win}: sampled rows")
    x = W.make_inputs(w)
    d_ = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(d_["q"], d_["k"], d_["v"], cos, sin, window=win)
    o, lse = f64(o), f64(lse)
    rng = np.random.default_rng(5)
    rows = [(0, t, int(rng.integers(0, 32))) for t in [0, 1, 1023, 1024, 1025, 2047, 4096, 8191]]
    rows += [(0, int(t), int(rng.integers(0, 32))) for t in rng.integers(0, w.T, 40)]
    ro, rl = oracle.attention_rows(x["q"], x["k"], x["v"], rows, causal=True, base=w.base, window=win)
    go = np.stack([o[b, t, h] for (b, t, h) in rows])
    gl = np.array([lse[b, h, t] for (b, t, h) in rows])
    assert_close(f"{w.name} W{win} sampled", go, ro, gl, rl, "bf16")


BWD = [
    (300, 8, 2, 128, 64, 1),
    (1000, 8, 2, 128, 300, 1),
    (200, 6, 2, 64, 17, 3),
    (129, 4, 1, 32, 1, 1),
]


@pytest.mark.parametrize("T,H,KV,d,win,B", BWD, ids=[f"T{c[0]}_H{c[1]}_KV{c[2]}_d{c[3]}_W{c[4]}_B{c[5]}" for c in BWD])
def test_window_backward(gpu, T, H, KV, d, win, B):
    w = W.custom(f"win_bwd_T{T}_W{win}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, seed=70 + T + win)
    announce(f"window backward {w.name} H{H} KV{KV} d{d} B{B}")
    x = W.make_inputs(w)
    d_ = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(d_["q"], d_["k"], d_["v"], cos, sin, window=win)
    dout = W.make_dout(w, x["q"])
    grads = cgr.gqa_rope_attn_bwd(d_["q"], d_["k"], d_["v"], o, lse, dout.to(gpu), cos, sin, window=win)
    ref = oracle.attention_dense_bwd(x["q"], x["k"], x["v"], dout, causal=True, base=w.base, window=win)
    assert_grads_close(w.name, [f64(g) for g in grads], ref)


@pytest.mark.parametrize("win,Tq,lens", [(100, 2, [10, 500, 4096, 33]), (1, 1, [1, 70, 3000]),
                                         (4000, 3, [3, 4100, 2000])])
def test_window_decode(gpu, win, Tq, lens):
    B, S, H, KV, d = len(lens), max(lens), 8, 2, 128
    gen = torch.Generator("cpu").manual_seed(80 + win)
    q = torch.randn((B, Tq, H, d), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, S, KV, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, S, KV, d), generator=gen).to(torch.bfloat16)
    announce(f"window decode W={win} Tq={Tq} lens={lens}")
    cos, sin = cgr.rope_tables(S, d, 1e4, device=gpu)
    pos = torch.arange(S, dtype=torch.int32, device=gpu).repeat(B)
    kr = cgr.rope_rotate(k.to(gpu).reshape(B * S, KV, d), pos, cos, sin).reshape(B, S, KV, d)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    o, lse = cgr.gqa_rope_attn_decode(q.to(gpu), kr, v.to(gpu), lens_t.to(gpu), S, cos, sin, window=win)
    ro, rl = oracle.attention_decode(q, k, v, lens, base=1e4, window=win)
    assert_close(f"decode W{win}", f64(o), ro, f64(lse), rl, "bf16")


@pytest.mark.parametrize("magnitude", [40.0, 140.0])
def test_window_scores_far_above_the_diagonal_tile(gpu, magnitude):
    """Windowed units whose rows fit one key tile take their reference from the
    tile holding each row's own key and then walk the window's earlier tiles;
    here keys early in every window score far above the diagonal tile's (by
    ~76 log2 units at magnitude 140), so the row sums pass their bound and the
    unit must fall back to the rescaling loop and still match the oracle."""
    T, H, KV, win = 300, 8, 2, 200
    w = W.custom("win_growth", B=1, T=T, n_head=H, n_kv_head=KV, head_dim=128, base=1e4, seed=23)
    announce(f"window {win}: scores far above the diagonal tile, magnitude {magnitude}")
    x = W.make_inputs(w)
    q = x["q"].float()
    k = x["k"].float().clone()
    for kvh in range(KV):
        dirn = q[0, :, 4 * kvh:4 * kvh + 4].mean(dim=(0, 1))
        k[0, 100:200, kvh] = k[0, 100:200, kvh] + magnitude * dirn / dirn.norm()
    x["k"] = k.to(torch.bfloat16)
    d_ = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(T, 128, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(d_["q"], d_["k"], d_["v"], cos, sin, window=win)
    ro, rl = oracle.attention_dense(x["q"], x["k"], x["v"], causal=True, base=w.base, window=win)
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow must route to the rescaling loop"
    assert_close(f"window growth {magnitude}", o, ro, lse, rl, "bf16")
