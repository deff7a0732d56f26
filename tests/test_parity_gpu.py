"""GPU parity: the HIP path through the C-ABI against the float64 oracle on the
same seeded inputs, element by element, at sizes that span several tiles and a
ragged tail, and on sampled rows at the full long-context and packed sizes."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import (TOL, announce, assert_close, compute_units, default_grid, f64, run_gpu,
                             run_oracle, to_dev)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_fp32_T64_H4_KV2_d32", "nanollama3_train_B8_T256_H6_KV2_d64",
         "qwen05b_prefill_T77_H14_KV2_d64_koutliers"] + list(W.PARITY_EXTRAS)


@pytest.mark.parametrize("P,d,base", [(8192, 128, 5e5), (2048, 128, 1e4), (77, 64, 1e6),
                                      (64, 32, 1e4), (17, 2, 1e4), (300, 6, 3.5)])
def test_rope_tables(gpu, P, d, base):
    announce(f"rope_tables P={P} d={d} base={base}")
    cos, sin = cgr.rope_tables(P, d, base, device=gpu)
    rc, rs = oracle.rope_tables(P, d, base)
    # float64 evaluation, one rounding to float32: within half an ulp of 1.0.
    assert np.abs(f64(cos) - rc).max() <= 2.0 ** -24
    assert np.abs(f64(sin) - rs).max() <= 2.0 ** -24


@pytest.mark.parametrize("name", SMALL)
def test_workload_full(gpu, name):
    w = W.get(name)
    announce(f"{name}: full comparison")
    x = W.make_inputs(w)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    ro, rl = run_oracle(w, x)
    assert_close(name, f64(o), ro, f64(lse), rl, w.dtype)


def test_long_context_full_size(gpu):
    """The full long-context workload (B=1, T=8192, 32 query heads, 8 K/V heads,
    head_dim 128) in the launch configuration the benchmark times, compared with
    the float64 oracle on every element of O (33.5 M) and of the LSE (262,144
    rows): max abs and median relative error over the whole config. Both Q.K^T
    operand types: the default f16 and bf16 (the operand type the method's
    statement names, which the benchmark also times)."""
    w = W.get("long_context_T8192_H32_KV8_d128")
    x = W.make_inputs(w)
    xd = to_dev(x, gpu)
    ro, rl = run_oracle(w, x)
    for qk in ("f16", "bf16"):
        announce(f"{w.name}: full-size run ({qk} Q.K^T operands), every element against the oracle")
        o, lse = run_gpu(w, xd, gpu, qk_operand=qk)
        assert_close(f"{w.name} ({qk} operands, every element)", f64(o), ro, f64(lse), rl, w.dtype)


def test_varlen_workload_full_size(gpu):
    """The full packed MQA workload (32 sequences, 32,226 tokens, 16 query heads,
    one K/V head, head_dim 128) in the launch configuration the benchmark times
    (keys rotated once into the workspace), every element against the oracle."""
    w = W.get("varlen_mqa_32seqs_16to2048_H16_KV1_d128")
    announce(f"{w.name}: full-size run, every element against the oracle")
    x = W.make_inputs(w)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    ro, rl = run_oracle(w, x)
    assert_close(w.name + " (every element)", f64(o), ro, f64(lse), rl, w.dtype)


EDGE = [
    # B, T, H, KV, d, dtype, causal, style
    (1, 1, 1, 1, 128, "bf16", True, "interleaved"),
    (3, 1, 4, 2, 64, "bf16", False, "half"),
    (2, 2, 2, 1, 32, "f32", True, "half"),
    (1, 31, 4, 4, 64, "bf16", True, "interleaved"),
    (2, 63, 6, 3, 128, "bf16", False, "interleaved"),
    (1, 64, 8, 1, 128, "bf16", True, "half"),
    (1, 65, 2, 2, 32, "bf16", True, "interleaved"),
    (2, 127, 4, 2, 64, "f32", True, "interleaved"),
    (1, 129, 4, 1, 128, "bf16", True, "interleaved"),
    (1, 300, 8, 2, 128, "bf16", False, "half"),
    (1, 521, 4, 2, 128, "bf16", True, "interleaved"),
    (2, 200, 3, 1, 64, "f32", False, "half"),
    (1, 1000, 8, 2, 128, "bf16", True, "interleaved"),
]


@pytest.mark.parametrize("B,T,H,KV,d,dtype,causal,style", EDGE,
                         ids=["-".join(map(str, e)) for e in EDGE])
def test_edge_shapes(gpu, B, T, H, KV, d, dtype, causal, style):
    w = W.custom("edge", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, dtype=dtype, causal=causal,
                 rope_style=style, base=10000.0, seed=B * 1000 + T)
    announce(f"edge {w}")
    x = W.make_inputs(w)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    ro, rl = run_oracle(w, x)
    assert_close("edge", f64(o), ro, f64(lse), rl, dtype)


VARLEN = [
    # lengths, H, KV, d, dtype, causal, style
    ([5, 1, 0, 130, 64, 257, 1], 4, 1, 128, "bf16", True, "interleaved"),
    ([0, 300, 17], 6, 2, 64, "bf16", False, "half"),
    ([129, 128, 127, 2], 4, 4, 32, "f32", True, "interleaved"),
    ([1], 2, 1, 64, "bf16", True, "half"),
    ([700, 0, 0, 33], 8, 2, 128, "bf16", True, "interleaved"),
]


def packed_inputs(lengths, H, KV, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    total = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0).to(torch.int32)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((total, H, d), generator=g).to(dt)
    k = torch.randn((total, KV, d), generator=g).to(dt)
    v = torch.randn((total, KV, d), generator=g).to(dt)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, max_seqlen=max(lengths), lengths=torch.tensor(lengths))


@pytest.mark.parametrize("lengths,H,KV,d,dtype,causal,style", VARLEN,
                         ids=[f"v{i}" for i in range(len(VARLEN))])
def test_varlen_small_full(gpu, lengths, H, KV, d, dtype, causal, style):
    announce(f"varlen lengths={lengths} H={H} KV={KV} d={d} {dtype} causal={causal} {style}")
    x = packed_inputs(lengths, H, KV, d, dtype, seed=len(lengths) * 7 + d)
    w = W.custom("varlen", n_head=H, n_kv_head=KV, head_dim=d, dtype=dtype, causal=causal,
                 rope_style=style, base=5e5, num_seqs=len(lengths), len_lo=0, len_hi=1)
    xd = to_dev(x, gpu)
    o, lse = run_gpu(w, xd, gpu)
    ro, rl = run_oracle(w, x)
    assert_close("varlen", f64(o), ro, f64(lse), rl, dtype)


def test_varlen_equals_dense_per_sequence(gpu):
    """A packed batch is, bit for bit, the dense forward of each of its sequences."""
    lengths = [200, 77, 1, 129]
    announce(f"varlen vs dense, lengths {lengths}")
    x = packed_inputs(lengths, 8, 2, 128, "bf16", seed=5)
    xd = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(256, 128, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["cu_seqlens"], 200, cos, sin)
    cu = x["cu_seqlens"].tolist()
    for s, L in enumerate(lengths):
        a = cu[s]
        od, ld = cgr.gqa_rope_attn_fwd(xd["q"][None, a:a + L].contiguous(), xd["k"][None, a:a + L].contiguous(),
                                       xd["v"][None, a:a + L].contiguous(), cos, sin)
        assert torch.equal(o[a:a + L], od[0])
        assert torch.equal(lse[:, a:a + L], ld[0])


def test_deterministic_and_fully_written(gpu):
    w = W.get("nanollama3_train_B8_T256_H6_KV2_d64")
    announce("determinism + poison fill")
    x = to_dev(W.make_inputs(w), gpu)
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    outs = []
    for _ in range(2):
        o = torch.full_like(x["q"], float("nan"))
        lse = torch.full((w.B, w.n_head, w.T), float("nan"), device=gpu)
        cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, out=o, lse=lse)
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # Packed: poison both, run twice.
    xv = to_dev(packed_inputs([100, 0, 333, 5], 4, 1, 128, "bf16", 9), gpu)
    cos, sin = cgr.rope_tables(333, 128, 1e4, device=gpu)
    res = []
    for _ in range(2):
        o = torch.full_like(xv["q"], float("nan"))
        lse = torch.full((4, xv["q"].shape[0]), float("nan"), device=gpu)
        cgr.gqa_rope_attn_fwd_varlen(xv["q"], xv["k"], xv["v"], xv["cu_seqlens"], 333, cos, sin,
                                     out=o, lse=lse)
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        res.append((o, lse))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_causal_row0_is_value_row0(gpu):
    """Query 0 may only see key 0: its output is V[0] of its K/V head, exactly."""
    w = W.get("long_context_T8192_H32_KV8_d128").replace(T=300)
    announce("causal row 0")
    x = to_dev(W.make_inputs(w), gpu)
    o, _ = run_gpu(w, x, gpu)
    G = w.n_head // w.n_kv_head
    for h in range(w.n_head):
        assert torch.equal(o[:, 0, h], x["v"][:, 0, h // G])


def test_softmax_scale_and_no_lse(gpu):
    w = W.custom("scale", B=2, T=150, n_head=4, n_kv_head=2, head_dim=64, base=1e4, seed=3)
    announce("explicit softmax scale, lse omitted")
    x = W.make_inputs(w)
    xd = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(150, 64, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin, softmax_scale=0.05,
                                   return_lse=False)
    assert lse is None
    ro, _ = oracle.attention_dense(x["q"], x["k"], x["v"], base=1e4, scale=0.05)
    from tests.gpu_cases import errors
    mx, med = errors(f64(o), ro)
    assert mx <= TOL["bf16"]["max_abs"] and med <= TOL["bf16"]["med_rel"], (mx, med)


def test_qk_bf16_operand_option(gpu):
    """bf16 Q.K^T operands: same kernels, coarser rounding; within tolerance on
    N(0,1) inputs (the outlier workload needs the default f16 operands)."""
    w = W.get("nanollama3_train_B8_T256_H6_KV2_d64")
    announce("qk operand bf16")
    x = W.make_inputs(w)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu, qk_operand="bf16")
    ro, rl = run_oracle(w, x)
    assert_close("qk-bf16", f64(o), ro, f64(lse), rl, "bf16")


@pytest.mark.parametrize("rotated", [False, True], ids=["schedule_ws", "rotated_ws"])
@pytest.mark.parametrize("cu,code", [([1, 5, 9], 1), ([0, 6, 4, 9], 2), ([0, 2, 9], 3),
                                     ([0, 4, 8], 4)])
def test_malformed_cu_seqlens_schedules_nothing(gpu, cu, code, rotated):
    announce(f"malformed cu_seqlens {cu} rotated-keys workspace={rotated}")
    total = 9
    q = torch.randn(total, 2, 64, device=gpu).to(torch.bfloat16)
    kv = torch.randn(total, 1, 64, device=gpu).to(torch.bfloat16)
    cos, sin = cgr.rope_tables(8, 64, 1e4, device=gpu)
    o = torch.full_like(q, float("nan"))
    n = (cgr.cgr_attn_fwd_varlen_rotated_workspace_size(len(cu) - 1, total, 1, 64) if rotated
         else cgr.cgr_attn_fwd_varlen_workspace_size(len(cu) - 1, total))
    ws = torch.zeros(n, dtype=torch.uint8, device=gpu)
    cgr.gqa_rope_attn_fwd_varlen(q, kv, kv, torch.tensor(cu, dtype=torch.int32, device=gpu), 6,
                                 cos, sin, out=o, workspace=ws)
    assert cgr.cgr_varlen_device_status(ws) == code
    assert torch.isnan(o).all(), "a malformed batch must leave the output untouched"


def test_host_checks_with_real_tensors(gpu):
    announce("host-side argument checks")
    q = torch.zeros(1, 8, 4, 64, device=gpu, dtype=torch.bfloat16)
    kv = torch.zeros(1, 8, 3, 64, device=gpu, dtype=torch.bfloat16)
    cos, sin = cgr.rope_tables(8, 64, 1e4, device=gpu)
    with pytest.raises(cgr.CgrError) as e:
        cgr.gqa_rope_attn_fwd(q, kv, kv, cos, sin)
    assert e.value.status == cgr.CGR_ERR_INVALID_ARG
    short_cos, short_sin = cgr.rope_tables(7, 64, 1e4, device=gpu)
    kv = torch.zeros(1, 8, 2, 64, device=gpu, dtype=torch.bfloat16)
    with pytest.raises(cgr.CgrError):
        cgr.gqa_rope_attn_fwd(q, kv, kv, short_cos, short_sin)
    q96 = torch.zeros(1, 8, 4, 96, device=gpu, dtype=torch.bfloat16)
    c96, s96 = cgr.rope_tables(8, 96, 1e4, device=gpu)
    with pytest.raises(cgr.CgrError) as e:
        cgr.gqa_rope_attn_fwd(q96, q96[:, :, :2].contiguous(), q96[:, :, :2].contiguous(), c96, s96)
    assert e.value.status == cgr.CGR_ERR_UNSUPPORTED


def test_runs_on_the_callers_stream(gpu):
    w = W.custom("stream", B=1, T=500, n_head=4, n_kv_head=1, head_dim=128, base=1e4, seed=8)
    announce("side stream")
    x = W.make_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xd = to_dev(x, gpu)
        cos, sin = cgr.rope_tables(500, 128, 1e4, device=gpu)
        o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin)
    s.synchronize()
    ro, rl = run_oracle(w, x)
    assert_close("stream", f64(o), ro, f64(lse), rl, "bf16")


@pytest.mark.parametrize("magnitude", [140.0, 250.0, 600.0])
def test_scores_growing_far_beyond_the_first_tile(gpu, magnitude):
    """Keys in later tiles score far above every key of the first tile: by up
    to ~76 log2 units at magnitude 140, where 2^(s - m) against the first
    tile's reference stays inside the float range (the fast path holds), and
    by ~135 and ~300 at 250 and 600, past that range: there the unit must take
    the rescaling path. Either way it matches the oracle."""
    w = W.custom("growth", B=1, T=300, n_head=4, n_kv_head=2, head_dim=128, base=1e4, seed=21)
    announce(f"scores growing beyond the first tile's reference, magnitude {magnitude}")
    x = W.make_inputs(w)
    q = x["q"].float()
    k = x["k"].float().clone()
    # Keys 150.. align with each head group's mean query direction, scaled up.
    for kvh in range(2):
        dirn = q[0, :, 2 * kvh:2 * kvh + 2].mean(dim=(0, 1))
        k[0, 150:, kvh] = k[0, 150:, kvh] + magnitude * dirn / dirn.norm()
    x["k"] = k.to(torch.bfloat16)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    ro, rl = run_oracle(w, x)
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow must route to the rescaling path"
    if magnitude <= 140.0:
        assert_close("growth", o, ro, lse, rl, "bf16")
    else:
        # Scores reach ~300 log2 units here, so the one rounding of the rotated
        # operands to f16 (relative 2^-11) moves each by ~0.1 and the fixed
        # 2e-2 bar no longer applies. The bar is derived from the formats
        # instead (tests/error_bounds.py): per element, 8 standard deviations
        # of the first-order error of f16 q*scale*log2(e) and k, bf16 p, plus
        # the bf16 rounding of O itself and 1e-4 of slack.
        check_growth_against_format_bar(x, w, o, lse, ro, rl)


def check_growth_against_format_bar(x, w, o, lse, ro, rl):
    from tests.error_bounds import BF16, F16, attention_sigma, bar, check_within
    T, H, KV, d = w.T, w.n_head, w.n_kv_head, w.head_dim
    pos = np.arange(T)
    qr = oracle.apply_rope(x["q"][0], pos, w.base, w.rope_style)
    kr = oracle.apply_rope(x["k"][0], pos, w.base, w.rope_style)
    c = np.log2(np.e) / np.sqrt(d)
    vis = np.tril(np.ones((T, T), dtype=bool))
    v = f64(x["v"][0])
    for h in range(H):
        kv = h // (H // KV)
        _, _, so, sl = attention_sigma(qr[:, h] * c, kr[:, kv], v[:, kv], vis, qfmt=F16, kfmt=F16, pfmt=BF16)
        check_within(f"growth head {h} O", o[0, :, h], ro[0, :, h], bar(so, ro[0, :, h], z=8, out_u=2.0 ** -9, slack=1e-4))
        check_within(f"growth head {h} LSE", lse[0, h], rl[0, h], bar(sl, rl[0, h], z=8, out_u=0.0, slack=1e-4))


def test_first_tile_dominates(gpu):
    """Keys of the first tile score far above all later keys: later
    probabilities underflow against the first tile's reference, as they do
    against the exact row max."""
    w = W.custom("sink", B=1, T=400, n_head=4, n_kv_head=1, head_dim=64, base=1e4, seed=22)
    announce("first tile dominates")
    x = W.make_inputs(w)
    q = x["q"].float()
    k = x["k"].float().clone()
    dirn = q[0].mean(dim=(0, 1))
    k[0, :8, 0] = k[0, :8, 0] + 30.0 * dirn / dirn.norm()
    x["k"] = k.to(torch.bfloat16)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    ro, rl = run_oracle(w, x)
    assert_close("sink", f64(o), ro, f64(lse), rl, "bf16")


@pytest.mark.parametrize("B,T,H,KV,d,causal,style", [(4, 2100, 8, 2, 128, True, "interleaved"),
                                                     (4, 2100, 8, 2, 64, False, "half"),
                                                     (4, 4100, 6, 3, 32, True, "half")])
def test_pre_rotated_keys_give_the_same_bits(gpu, B, T, H, KV, d, causal, style):
    """With a workspace the keys are rotated once up front; without, on every
    tile: the same arithmetic in the same order, so the same bits. (Grids that
    fill the device, so both calls run the default instances.)"""
    assert default_grid(B, T, H, KV, d) >= compute_units(gpu)
    w = W.custom("prerot", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, causal=causal, rope_style=style,
                 seed=T + d)
    x = to_dev(W.make_inputs(w), gpu)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    o1, l1 = cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, causal=causal, rope_style=style,
                                   workspace=False)
    o2, l2 = cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, causal=causal, rope_style=style)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("T,H,KV,d,causal,style,win,padded", [
    (300, 8, 2, 128, True, "interleaved", 0, False),
    (129, 4, 1, 64, False, "half", 0, True),
    (1000, 6, 3, 32, True, "half", 100, False),
    (200, 4, 2, 256, True, "interleaved", 0, True),
])
def test_rotate_keys_then_rotated_gives_the_same_bits(gpu, T, H, KV, d, causal, style, win, padded):
    """cgr_attn_fwd_rotate_keys followed by cgr_gqa_rope_attn_fwd_rotated is the
    forward with a workspace, split in two: the same bits (the one call runs
    the small-unit instances here when no window is set)."""
    w = W.custom("split", B=2, T=T, n_head=H, n_kv_head=KV, head_dim=d, causal=causal, rope_style=style,
                 seed=T + 7 * d)
    announce(f"rotate_keys + rotated vs one call: T={T} H={H} KV={KV} d={d} causal={causal} {style} W={win} "
             f"padded={padded}")
    x = to_dev(W.make_inputs(w), gpu)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    sl = torch.tensor([T // 3, T], dtype=torch.int32, device=gpu) if padded else None
    kw = dict(causal=causal, rope_style=style, window=win, seqlens=sl)
    o1 = torch.full_like(x["q"], 7.0)
    l1 = torch.full((2, H, T), 7.0, device=gpu)
    cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, out=o1, lse=l1, **kw)
    ws = torch.empty(cgr.cgr_attn_fwd_workspace_size(2, T, KV, d), dtype=torch.uint8, device=gpu)
    cgr.attn_fwd_rotate_keys(x["k"], cos, sin, ws, rope_style=style, seqlens=sl)
    o2 = torch.full_like(x["q"], 7.0)
    l2 = torch.full((2, H, T), 7.0, device=gpu)
    cgr.gqa_rope_attn_fwd_rotated(x["q"], x["k"], x["v"], cos, sin, ws, out=o2, lse=l2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("qk", ["f16", "bf16"])
def test_rotated_calls_share_one_workspace(gpu, qk):
    """The causal attention over once-rotated keys hands its lightest query
    blocks out from a counter at the workspace's end: the key rotation zeroes
    it and each call leaves it at zero. Starting from a workspace of 0xFF
    bytes, one rotation then three attention calls in a row give the one
    call's bits every time; then a smaller batch in the same workspace."""
    H, KV, d = 8, 2, 128
    big, small = (2, 1000), (1, 333)
    n = max(cgr.cgr_attn_fwd_workspace_size(B, T, KV, d) for B, T in (big, small))
    ws = torch.full((n,), 255, dtype=torch.uint8, device=gpu)
    for B, T in (big, small):
        w = W.custom("shared_ws", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, seed=T)
        announce(f"rotated calls on one workspace: B={B} T={T} qk={qk}")
        x = to_dev(W.make_inputs(w), gpu)
        cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
        kw = dict(causal=True, rope_style=w.rope_style, qk_operand=qk)
        ref_o, ref_l = cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, **kw)
        cgr.attn_fwd_rotate_keys(x["k"], cos, sin, ws, rope_style=w.rope_style, qk_operand=qk)
        for _ in range(3):
            o = torch.full_like(x["q"], 7.0)
            l = torch.full((B, H, T), 7.0, device=gpu)
            cgr.gqa_rope_attn_fwd_rotated(x["q"], x["k"], x["v"], cos, sin, ws, out=o, lse=l, **kw)
            torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("qk", ["f16", "bf16"])
@pytest.mark.parametrize("causal,style", [(True, "interleaved"), (False, "half"), (True, "half")])
def test_small_grid_units_give_the_same_bits(gpu, d, qk, causal, style):
    """A call whose default grid leaves compute units idle runs 4-wave units
    with keys rotated per tile; the split entries always run the default
    8-wave units on once-rotated keys. Every row's arithmetic is the same, so
    the bits are too (ragged T, a padded entry)."""
    B, T, H, KV = 2, 203, 6, 2
    assert default_grid(B, T, H, KV, d) < compute_units(gpu)
    w = W.custom("smallgrid", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, causal=causal, rope_style=style,
                 seed=d + (qk == "bf16"))
    announce(f"small-grid units vs split entries: d={d} qk={qk} causal={causal} {style}")
    x = to_dev(W.make_inputs(w), gpu)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    sl = torch.tensor([T, 150], dtype=torch.int32, device=gpu)
    kw = dict(causal=causal, rope_style=style, qk_operand=qk, seqlens=sl)
    o1 = torch.full_like(x["q"], 7.0)
    l1 = torch.full((B, H, T), 7.0, device=gpu)
    ws1 = torch.full((cgr.cgr_attn_fwd_workspace_size(B, T, KV, d),), 5, dtype=torch.uint8, device=gpu)
    cgr.gqa_rope_attn_fwd(x["q"], x["k"], x["v"], cos, sin, out=o1, lse=l1, workspace=ws1, **kw)
    ws2 = torch.empty_like(ws1)
    cgr.attn_fwd_rotate_keys(x["k"], cos, sin, ws2, rope_style=style, qk_operand=qk, seqlens=sl)
    o2 = torch.full_like(x["q"], 7.0)
    l2 = torch.full((B, H, T), 7.0, device=gpu)
    cgr.gqa_rope_attn_fwd_rotated(x["q"], x["k"], x["v"], cos, sin, ws2, out=o2, lse=l2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # The small-grid call leaves the workspace it was given untouched.
    assert bool((ws1 == 5).all())


PACKED_PREROT = [
    # lengths, H, KV, d, causal, style, window
    ([5, 1, 0, 130, 64, 257, 1], 4, 1, 128, True, "interleaved", 0),
    ([0, 300, 17], 6, 2, 64, False, "half", 0),
    ([129, 128, 127, 2], 4, 4, 32, True, "interleaved", 0),
    ([700, 0, 0, 33, 1000], 8, 2, 128, True, "half", 100),
    ([300, 65, 64, 63], 4, 2, 256, True, "interleaved", 0),
]


@pytest.mark.parametrize("lengths,H,KV,d,causal,style,win", PACKED_PREROT,
                         ids=[f"p{i}" for i in range(len(PACKED_PREROT))])
def test_packed_pre_rotated_keys_give_the_same_bits(gpu, lengths, H, KV, d, causal, style, win):
    """A packed batch with the keys rotated once into the workspace (tile
    images per sequence, empty sequences owning none) gives the bits of the
    per-tile rotation, and both match the oracle."""
    announce(f"packed pre-rotated keys lengths={lengths} H={H} KV={KV} d={d} causal={causal} {style} W={win}")
    x = packed_inputs(lengths, H, KV, d, "bf16", seed=sum(lengths) + d)
    xd = to_dev(x, gpu)
    ms = max(max(lengths), 1)
    cos, sin = cgr.rope_tables(ms, d, 5e5, device=gpu)
    args = (xd["q"], xd["k"], xd["v"], xd["cu_seqlens"], ms, cos, sin)
    kw = dict(causal=causal, rope_style=style, window=win)
    o1, l1 = cgr.gqa_rope_attn_fwd_varlen(*args, rotate_keys_once=False, **kw)
    o2, l2 = cgr.gqa_rope_attn_fwd_varlen(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if sum(lengths):
        ro, rl = oracle.attention_varlen(x["q"], x["k"], x["v"], x["cu_seqlens"].numpy(), causal=causal,
                                         base=5e5, style=style, window=win)
        assert_close("packed pre-rotated", f64(o2), ro, f64(l2), rl, "bf16")


@pytest.mark.parametrize("rotate_keys_once", [True, False], ids=["rotated_once", "per_tile"])
def test_packed_batch_of_many_short_sequences(gpu, rotate_keys_once):
    """1300 sequences of 0 to 70 tokens (the schedule handles 512 sequences per
    round; empty sequences leave unowned image slots between their
    neighbours'): against the oracle, and the two key paths bit for bit."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 71, 1300)]
    lengths[100:110] = [0] * 10
    lengths[-1] = 0
    announce(f"packed batch of {len(lengths)} short sequences, {sum(lengths)} tokens, "
             f"rotate_keys_once={rotate_keys_once}")
    x = packed_inputs(lengths, 4, 1, 64, "bf16", seed=78)
    xd = to_dev(x, gpu)
    ms = max(lengths)
    cos, sin = cgr.rope_tables(ms, 64, 1e4, device=gpu)
    args = (xd["q"], xd["k"], xd["v"], xd["cu_seqlens"], ms, cos, sin)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(*args, rotate_keys_once=rotate_keys_once)
    o2, l2 = cgr.gqa_rope_attn_fwd_varlen(*args, rotate_keys_once=not rotate_keys_once)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    ro, rl = oracle.attention_varlen(x["q"], x["k"], x["v"], x["cu_seqlens"].numpy(), causal=True, base=1e4)
    assert_close("many short sequences", f64(o), ro, f64(lse), rl, "bf16")


def test_longest_sequence_the_offsets_allow(gpu):
    """T = 120000 with 32 query heads of 128 (one sequence of 0.98 GB of q, byte
    offsets up to 2^31 within a sequence): sampled rows, the last rows of every
    K/V group among them, against the oracle. The host check rejects T past
    130815 for this width (tests/test_abi.py)."""
    w = W.custom("longest", B=1, T=120000, n_head=32, n_kv_head=8, head_dim=128, base=500000.0, seed=29)
    announce(f"{w.name}: T={w.T}, sampled rows")
    x = W.make_inputs(w)
    o, lse = run_gpu(w, to_dev(x, gpu), gpu)
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(29)
    ts = [0, 63, 64, 65535, 65536, 119935, 119936, 119999] + [int(t) for t in rng.integers(0, w.T, 12)]
    rows = [(0, t, int(rng.integers(0, 32))) for t in ts] + [(0, 119999, h) for h in range(0, 32, 4)]
    ro, rl = oracle.attention_rows(x["q"], x["k"], x["v"], rows, causal=True, base=w.base)
    go = np.stack([o[b, t, h] for (b, t, h) in rows])
    gl = np.array([lse[b, h, t] for (b, t, h) in rows])
    assert_close(w.name + " (sampled)", go, ro, gl, rl, "bf16")


HEAD_PACKED = [
    # d, H, KV, style, causal, window: units of 32 rows x 8 heads (G = 8) and of
    # 64 rows x 4 heads (G = 4), whose waves rotate the same positions of
    # several heads
    (32, 8, 1, "interleaved", True, 0),
    (32, 8, 2, "half", True, 0),
    (64, 8, 1, "half", True, 0),
    (64, 8, 2, "interleaved", False, 0),
    (128, 8, 1, "interleaved", True, 0),
    (128, 8, 2, "half", True, 0),
    (128, 8, 1, "half", False, 0),
    (128, 8, 2, "interleaved", True, 50),
    (64, 8, 1, "interleaved", True, 33),
]


@pytest.mark.parametrize("d,H,KV,style,causal,window", HEAD_PACKED,
                         ids=[f"d{e[0]}-G{e[1] // e[2]}-{e[3]}-c{int(e[4])}-w{e[5]}" for e in HEAD_PACKED])
def test_head_packed_units(gpu, d, H, KV, style, causal, window):
    """Units whose waves cover several heads of one row block: a dense batch
    with a ragged tail (the small-grid units) and a packed batch with empty and
    one-token sequences, element by element against the oracle."""
    announce(f"head-packed units d={d} H={H} KV={KV} {style} causal={causal} window={window}")
    w = W.custom("head_packed", B=2, T=300, n_head=H, n_kv_head=KV, head_dim=d, dtype="bf16", causal=causal,
                 rope_style=style, base=1e4, seed=d + H + 7 * KV + window)
    x = W.make_inputs(w)
    xd = to_dev(x, gpu)
    cos, sin = cgr.rope_tables(w.T, d, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin, causal=causal, rope_style=style,
                                   window=window)
    ro, rl = oracle.attention_dense(x["q"], x["k"], x["v"], causal=causal, base=w.base, style=style,
                                    window=window)
    assert_close("head-packed dense", f64(o), ro, f64(lse), rl, "bf16")
    lengths = [5, 0, 130, 64, 1, 97]
    xp = packed_inputs(lengths, H, KV, d, "bf16", seed=d * 3 + KV)
    xpd = to_dev(xp, gpu)
    cosp, sinp = cgr.rope_tables(max(lengths), d, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(xpd["q"], xpd["k"], xpd["v"], xpd["cu_seqlens"], max(lengths), cosp,
                                          sinp, causal=causal, rope_style=style, window=window)
    ro, rl = oracle.attention_varlen(xp["q"], xp["k"], xp["v"], xp["cu_seqlens"].numpy(), causal=causal,
                                     base=w.base, style=style, window=window)
    assert_close("head-packed packed", f64(o), ro, f64(lse), rl, "bf16")
