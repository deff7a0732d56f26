"""GPU parity of the fp8-operand forward (cgr_gqa_rope_attn_fwd_fp8) through the
C-ABI against the float64 oracle: the exact attention of the dequantized
inputs (e4m3 codes x descale), on the same seeded inputs.

Bar against the oracle, per element, derived from the formats alone
(tests/error_bounds.py): the path rounds the rotated q and k and the
probabilities p to e4m3 (unit round-off 2^-4, subnormal floor 2^-10) and O to
bf16. Eight standard deviations of the first-order error those roundings
cause, plus the bf16 rounding of O and 1e-3 of slack. The subnormal floors
use the scalings the header documents (q scaled into [1/4, 1/2) of its
range, k halved), nothing else of the kernel's structure. Keys with outliers
(0.5 % of entries x 20) get the same treatment: their large scores widen the
bar where, and only where, the roundings move them.

Every case is also held to a rounding model that mirrors the documented fp8
arithmetic step by step (tests/fp8_error_model.py: tile-0 row reference,
128-row blocks, fallback): a tighter consistency check. The kernel and that
model round at the same points and differ only where f32 and float64
evaluation fall on opposite sides of an e4m3 rounding boundary, which is
rare. Bar: at most 1 in 1000 outputs differ by more than 0.02, median
relative 5e-3, LSE 2e-2, and no output by more than max|v| / 8 (one flipped p
moves its weight by at most 1/16 of the row sum)."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.fp8_error_model import model_forward
from tests.gpu_cases import announce, errors, f64

pytestmark = pytest.mark.gpu

def check_model(name, o, mo, lse, ml, vmax):
    d = np.abs(o - mo)
    frac = float((d > 0.02).mean())
    _, med = errors(o, mo)
    lmx, _ = errors(lse, ml)
    msg = (f"{name} vs the rounding model: O max abs {d.max():.3e} (bound {vmax / 8:.3e}), share above 0.02 "
           f"{frac:.2e}, median rel {med:.3e}; LSE max abs {lmx:.3e}")
    print(msg, flush=True)
    assert frac <= 1e-3 and med <= 5e-3 and lmx <= 2e-2 and d.max() <= vmax / 8, msg


def check(name, x, w, o, lse, ro, rl, causal, style, rows=None):
    """O and LSE against the oracle within the format-derived bar. rows: None
    (every row of every batch entry and head) or a list of (b, t, h)."""
    from tests.error_bounds import E4M3, attention_sigma, bar, check_within
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{name}: non-finite output"
    T, d = o.shape[1], o.shape[3]
    H, KV = o.shape[2], x["k64"].shape[2]
    c = np.log2(np.e) / np.sqrt(d)
    vis = np.tril(np.ones((T, T), dtype=bool)) if causal else np.ones((T, T), dtype=bool)
    # Absolute floors in the units of qs and kt: e4m3 subnormals (2^-10) of q
    # scaled by at least 1/4 and of k halved, in units of the code values.
    a_q = 2.0 ** -8 * x["q_descale"] * c
    a_k = 2.0 ** -9 * x["k_descale"]
    want = {}
    for (b, t, h) in ([(b, t, h) for b in range(o.shape[0]) for h in range(H) for t in [None]] if rows is None
                      else rows):
        want.setdefault((b, h), []).append(t)
    worst = 0.0
    for (b, h), ts in want.items():
        kv = h // (H // KV)
        pos = np.arange(T)
        qs = oracle.apply_rope(x["q64"][b, :, h], pos, w.base, style) * c
        kt = oracle.apply_rope(x["k64"][b, :, kv], pos, w.base, style)
        sel = None if ts == [None] else np.array(ts)
        _, _, so, sl = attention_sigma(qs, kt, x["v64"][b, :, kv], vis, qfmt=E4M3, kfmt=E4M3, pfmt=E4M3,
                                       a_q=a_q, a_k=a_k, rows=sel)
        tt = slice(None) if sel is None else sel
        worst = max(worst, check_within(f"{name} b{b} h{h} O", o[b, tt, h], ro[b, tt, h],
                                        bar(so, ro[b, tt, h], z=8, out_u=2.0 ** -9, slack=1e-3)))
        worst = max(worst, check_within(f"{name} b{b} h{h} LSE", lse[b, h, tt], rl[b, h, tt],
                                        bar(sl, rl[b, h, tt], z=8, out_u=0.0, slack=1e-3)))
    mx, med = errors(o if rows is None else np.stack([o[b, t, h] for (b, t, h) in rows]),
                     ro if rows is None else np.stack([ro[b, t, h] for (b, t, h) in rows]))
    print(f"{name}: O max abs {mx:.3e}, median rel {med:.3e}; largest error / bar {worst:.3f}", flush=True)


def model(w, x, causal, style):
    q8, k8, v8 = (x[n].to(torch.float64).numpy() for n in ("q", "k", "v"))
    out = [model_forward(q8[b], k8[b], v8[b], x["q_descale"], x["k_descale"], x["v_descale"], base=w.base,
                         style=style, causal=causal) for b in range(w.B)]
    return np.stack([o for o, _ in out]), np.stack([l for _, l in out])


def run(w, x, dev, causal=True, style="interleaved"):
    cos, sin = cgr.rope_tables(w.T, 128, w.base, device=dev)
    return cgr.gqa_rope_attn_fwd_fp8(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["q_descale"],
                                     x["k_descale"], x["v_descale"], cos, sin, causal=causal, rope_style=style)


# (B, T, H, KV, causal, style, outliers): one tile, ragged tails over the
# 64-key tile and 256-row unit, MHA/GQA/MQA, no mask, both pairings, T = 1,
# and keys with 0.5 % outliers x 20 (scores far above the first tile's, the
# rescaling path).
CASES = [
    (1, 64, 4, 2, True, "interleaved", False),
    (2, 256, 6, 2, True, "half", False),
    (1, 77, 14, 2, True, "interleaved", True),
    (1, 1000, 4, 1, True, "interleaved", False),
    (1, 300, 4, 2, False, "interleaved", False),
    (3, 1, 2, 1, True, "interleaved", False),
    (1, 129, 8, 8, True, "half", False),
    (1, 700, 8, 2, True, "interleaved", True),
]


@pytest.mark.parametrize("B,T,H,KV,causal,style,outl", CASES,
                         ids=[f"B{c[0]}_T{c[1]}_H{c[2]}_KV{c[3]}_{'causal' if c[4] else 'nomask'}_{c[5]}"
                              f"{'_outliers' if c[6] else ''}" for c in CASES])
def test_fp8_dense(gpu, B, T, H, KV, causal, style, outl):
    w = W.custom(f"fp8_T{T}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=128, base=5e5, dtype="f32",
                 seed=600 + T + H, outlier_frac=0.005 if outl else 0.0, outlier_factor=20.0 if outl else 1.0)
    announce(f"fp8 forward {w.name} B{B} H{H} KV{KV} causal={causal} {style} outliers={outl}")
    x = W.make_fp8_inputs(w)
    o, lse = run(w, x, gpu, causal, style)
    o, lse = f64(o), f64(lse)
    ro, rl = oracle.attention_dense(x["q64"], x["k64"], x["v64"], causal=causal, base=w.base, style=style)
    mo, ml = model(w, x, causal, style)
    check_model(w.name, o, mo, lse, ml, float(np.abs(x["v64"]).max()))
    check(w.name + " vs the oracle", x, w, o, lse, ro, rl, causal, style)


def test_fp8_row0_is_v0(gpu):
    """Causal row 0 sees only key 0: p = 1 is exact in e4m3, so O = v_0 up to the
    final bf16 rounding and the LSE is the one score."""
    w = W.custom("fp8_row0", B=1, T=100, n_head=4, n_kv_head=2, head_dim=128, base=1e4, dtype="f32", seed=9)
    x = W.make_fp8_inputs(w)
    o, _ = run(w, x, gpu)
    v0 = x["v64"][0, 0]
    got = f64(o)[0, 0]
    for h in range(4):
        assert np.abs(got[h] - v0[h // 2]).max() <= 2.0 ** -8 * np.abs(v0).max() + 1e-6


def test_fp8_is_deterministic(gpu):
    w = W.custom("fp8_det", B=1, T=600, n_head=8, n_kv_head=2, head_dim=128, base=1e4, dtype="f32", seed=10)
    x = W.make_fp8_inputs(w)
    o1, l1 = run(w, x, gpu)
    o2, l2 = run(w, x, gpu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_long_context_full_size_sampled(gpu):
    """The fp8 long-context workload in the benchmark's launch configuration, sampled rows."""
    w = W.get("fp8_long_context_T8192_H32_KV8_d128")
    announce(f"{w.name}: full-size run, sampled rows")
    x = W.make_fp8_inputs(w)
    o, lse = run(w, x, gpu)
    o, lse = f64(o), f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(12)
    ts = [0, 1, 63, 64, 255, 256, 4095, 8127, 8128, 8191] + [int(t) for t in rng.integers(0, w.T, 40)]
    rows = [(0, t, int(rng.integers(0, w.n_head))) for t in ts] + [(0, 8191, h) for h in range(0, 32, 3)]
    ro, rl = oracle.attention_rows(x["q64"], x["k64"], x["v64"], rows, causal=True, base=w.base)
    big_o = np.full_like(o, np.nan)
    big_l = np.full_like(lse, np.nan)
    for i, (b, t, h) in enumerate(rows):
        big_o[b, t, h] = ro[i]
        big_l[b, h, t] = rl[i]
    check(w.name + " (sampled)", x, w, o, lse, big_o, big_l, True, "interleaved", rows=rows)


# Right-padded batches (valid lengths per entry): (B, T, H, KV, causal,
# style, lengths): an empty entry, one-token and full entries, lengths at and
# around the 64-key tile and the 128-row unit, both masks and pairings.
PADDED = [
    (3, 300, 4, 2, True, "interleaved", [300, 129, 0]),
    (2, 256, 8, 1, False, "half", [1, 200]),
    (4, 130, 6, 3, True, "half", [64, 65, 127, 130]),
]


def entry(x, b, L):
    """Entry b's first L tokens as a batch of one (codes, descales, dequantized values)."""
    xb = {n: x[n][b:b + 1, :L].contiguous() for n in ("q", "k", "v")}
    xb.update({n + "64": x[n + "64"][b:b + 1, :L] for n in ("q", "k", "v")})
    xb.update({n + "_descale": x[n + "_descale"] for n in ("q", "k", "v")})
    return xb


@pytest.mark.parametrize("B,T,H,KV,causal,style,lengths", PADDED,
                         ids=[f"B{c[0]}_T{c[1]}_H{c[2]}_KV{c[3]}_{'causal' if c[4] else 'nomask'}_{c[5]}"
                              for c in PADDED])
def test_fp8_padded(gpu, B, T, H, KV, causal, style, lengths):
    """Every valid row of every entry against the oracle of that entry's first L
    tokens (the format-derived bar) and the rounding model; the padding rows of
    o and lse keep what they held; each entry gives the same bits as the
    unpadded call on its first L tokens alone."""
    w = W.custom(f"fp8_pad_T{T}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=128, base=5e5, dtype="f32",
                 seed=700 + T + H)
    announce(f"fp8 padded forward {w.name} B{B} H{H} KV{KV} causal={causal} {style} lengths={lengths}")
    x = W.make_fp8_inputs(w)
    cos, sin = cgr.rope_tables(T, 128, w.base, device=gpu)
    out = torch.full((B, T, H, 128), float("nan"), dtype=torch.bfloat16, device=gpu)
    lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device=gpu)
    seqlens = torch.tensor(lengths, dtype=torch.int32, device=gpu)
    cgr.gqa_rope_attn_fwd_fp8(x["q"].to(gpu), x["k"].to(gpu), x["v"].to(gpu), x["q_descale"], x["k_descale"],
                              x["v_descale"], cos, sin, causal=causal, rope_style=style, out=out, lse=lse,
                              seqlens=seqlens)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        assert torch.isnan(out[b, L:]).all() and torch.isnan(lse[b, :, L:]).all(), f"entry {b}: padding rows written"
        if L == 0:
            continue
        xb = entry(x, b, L)
        wb = W.custom(w.name, B=1, T=L, n_head=H, n_kv_head=KV, head_dim=128, base=w.base, dtype="f32")
        o_b, l_b = f64(out[b:b + 1, :L]), f64(lse[b:b + 1, :, :L])
        ro, rl = oracle.attention_dense(xb["q64"], xb["k64"], xb["v64"], causal=causal, base=w.base, style=style)
        mo, ml = model(wb, xb, causal, style)
        check_model(f"{w.name} entry {b} (L={L})", o_b, mo, l_b, ml, float(np.abs(xb["v64"]).max()))
        check(f"{w.name} entry {b} (L={L}) vs the oracle", xb, wb, o_b, l_b, ro, rl, causal, style)
        od, ld = cgr.gqa_rope_attn_fwd_fp8(xb["q"].to(gpu), xb["k"].to(gpu), xb["v"].to(gpu), x["q_descale"],
                                           x["k_descale"], x["v_descale"], cos, sin, causal=causal,
                                           rope_style=style)
        assert torch.equal(out[b:b + 1, :L], od) and torch.equal(lse[b:b + 1, :, :L], ld), f"entry {b}: bits"
