"""GPU tests of the f16 Q.K^T operand's range: inputs whose rotated keys, or
rotated queries times scale*log2(e), reach f16's limit (|x| >= 65520 rounds
to infinity) must still match the float64 oracle, never come out as NaN or
infinity. The path finds such units (out-of-range keys arrive as NaN from the
once-rotation, out-of-range queries are checked where they are staged, keys
rotated per tile are checked there) and recomputes their scores from bf16
hi + lo parts of the rotated operands.

Bars: O against the oracle at the bf16 bar (2e-2 max abs, 5e-3 median
relative). The LSE of rows that see a key of magnitude ~1e5 is itself ~1e4 in
size, so it is held to the per-element bar derived from the formats
(tests/error_bounds.py) for f16 operands, which bounds the wide path too (its
operands keep 16 significant bits against f16's 11)."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.error_bounds import BF16, F16, attention_sigma, bar, check_within
from tests.gpu_cases import TOL, announce, errors, f64

pytestmark = pytest.mark.gpu


def big_keys(x, rows, value=6.0e4):
    """Keys of the given rows get +-value on their first four features (every K/V head)."""
    k = x["k"].float().clone()
    for r in rows:
        k[..., r, :, 0:4] = torch.tensor([value, -value, value, -value])
    x["k"] = k.to(torch.bfloat16)
    return x


def check(name, x, o, lse, causal, base, window=0, scale=None, cu=None):
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{name}: non-finite output"
    if cu is None:
        ro, rl = oracle.attention_dense(x["q"], x["k"], x["v"], causal=causal, base=base, window=window,
                                        scale=scale)
    else:
        ro, rl = oracle.attention_varlen(x["q"], x["k"], x["v"], cu, causal=causal, base=base, window=window,
                                         scale=scale)
    mx, med = errors(o, ro)
    print(f"{name}: O max abs {mx:.3e}, median rel {med:.3e}", flush=True)
    assert mx <= TOL["bf16"]["max_abs"] and med <= TOL["bf16"]["med_rel"], (mx, med)
    # LSE per element against the f16-format bar, sequence by sequence.
    seqs = [(0, x["q"].shape[1], b) for b in range(x["q"].shape[0])] if cu is None else \
        [(int(cu[s]), int(cu[s + 1]), None) for s in range(len(cu) - 1)]
    H, d = x["q"].shape[-2], x["q"].shape[-1]
    KV = x["k"].shape[-2]
    c = np.log2(np.e) * (scale if scale is not None else 1.0 / np.sqrt(d))
    for (a, e, b) in seqs:
        Ls = e - a
        if Ls == 0:
            continue
        pos = np.arange(Ls)
        qq = x["q"][b] if b is not None else x["q"][a:e]
        kk = x["k"][b] if b is not None else x["k"][a:e]
        vv = f64(x["v"][b] if b is not None else x["v"][a:e])
        qr = oracle.apply_rope(qq, pos, base)
        kr = oracle.apply_rope(kk, pos, base)
        vis = np.tril(np.ones((Ls, Ls), dtype=bool)) if causal else np.ones((Ls, Ls), dtype=bool)
        if window:
            vis &= ~np.tril(np.ones((Ls, Ls), dtype=bool), -window)
        for h in range(H):
            kv = h // (H // KV)
            _, _, _, sl = attention_sigma(qr[:, h] * c, kr[:, kv], vv[:, kv], vis, qfmt=F16, kfmt=F16, pfmt=BF16)
            got = lse[b, h] if b is not None else lse[h, a:e]
            ref = rl[b, h] if b is not None else rl[h, a:e]
            check_within(f"{name} LSE seq@{a} h{h}", got, ref, bar(sl, ref, z=8, out_u=2.0 ** -23, slack=2e-2))


@pytest.mark.parametrize("workspace", [True, False], ids=["rotated_once", "per_tile"])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 50)], ids=["causal", "nomask", "window50"])
def test_keys_beyond_the_f16_range(gpu, workspace, causal, window):
    w = W.custom("range_k", B=2, T=300, n_head=4, n_kv_head=2, head_dim=128, base=1e4, causal=causal, seed=40)
    announce(f"keys near 6e4: workspace={workspace} causal={causal} window={window}")
    x = big_keys(W.make_inputs(w), [37, 150, 299])
    xd = {n: x[n].to(gpu) for n in ("q", "k", "v")}
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin, causal=causal, window=window,
                                   workspace=None if workspace else False)
    torch.cuda.synchronize()
    check("big keys", x, o, lse, causal, w.base, window=window)


def test_queries_beyond_the_f16_range_with_unit_scale(gpu):
    """q * scale * log2(e) past 65520: queries of ~7e4 with softmax_scale = 1."""
    w = W.custom("range_q", B=1, T=200, n_head=4, n_kv_head=1, head_dim=64, base=1e4, seed=41)
    announce("queries near 7e4, softmax_scale 1")
    x = W.make_inputs(w)
    q = x["q"].float().clone()
    q[0, 120, 2, 0:2] = torch.tensor([7.0e4, -7.0e4])
    q[0, 5, 0, 10] = 7.0e4
    x["q"] = q.to(torch.bfloat16)
    xd = {n: x[n].to(gpu) for n in ("q", "k", "v")}
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin, softmax_scale=1.0)
    torch.cuda.synchronize()
    check("big queries", x, o, lse, True, w.base, scale=1.0)


@pytest.mark.parametrize("rotate_keys_once", [True, False])
def test_packed_batch_keys_beyond_the_f16_range(gpu, rotate_keys_once):
    lengths = [120, 0, 300, 65]
    announce(f"packed batch, keys near 6e4, rotate_keys_once={rotate_keys_once}")
    g = torch.Generator("cpu").manual_seed(42)
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = dict(q=torch.randn((total, 8, 128), generator=g).to(torch.bfloat16),
             k=torch.randn((total, 2, 128), generator=g), v=torch.randn((total, 2, 128), generator=g).to(torch.bfloat16))
    for r in (3, 130, 419, 470):
        x["k"][r, :, 0:4] = torch.tensor([6.0e4, -6.0e4, 6.0e4, -6.0e4])
    x["k"] = x["k"].to(torch.bfloat16)
    xd = {n: x[n].to(gpu) for n in ("q", "k", "v")}
    cos, sin = cgr.rope_tables(300, 128, 1e4, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd_varlen(xd["q"], xd["k"], xd["v"], torch.from_numpy(cu).to(gpu), 300, cos, sin,
                                          rotate_keys_once=rotate_keys_once)
    torch.cuda.synchronize()
    check("packed big keys", x, o, lse, True, 1e4, cu=cu)


def test_in_range_inputs_keep_their_bits(gpu):
    """The guard only reroutes out-of-range units: a batch where one entry has
    huge keys gives the other entry the bits it gets on its own."""
    w = W.custom("range_iso", B=2, T=256, n_head=4, n_kv_head=2, head_dim=128, base=1e4, seed=43)
    announce("in-range entry unchanged beside an out-of-range one")
    x = W.make_inputs(w)
    k = x["k"].float().clone()
    k[1, 77, :, 0:4] = torch.tensor([6.0e4, -6.0e4, 6.0e4, -6.0e4])
    x["k"] = k.to(torch.bfloat16)
    xd = {n: x[n].to(gpu) for n in ("q", "k", "v")}
    cos, sin = cgr.rope_tables(w.T, w.head_dim, w.base, device=gpu)
    o, lse = cgr.gqa_rope_attn_fwd(xd["q"], xd["k"], xd["v"], cos, sin)
    o0, l0 = cgr.gqa_rope_attn_fwd(xd["q"][:1].contiguous(), xd["k"][:1].contiguous(), xd["v"][:1].contiguous(),
                                   cos, sin)
    torch.cuda.synchronize()
    assert torch.equal(o[:1], o0) and torch.equal(lse[:1], l0)
    check("batch with one big entry", x, o, lse, True, w.base)
