"""GPU parity of the dense forward with right padding (per-entry valid
lengths, `seqlens`) through the C-ABI against the float64 oracle's
`attention_padded` on the same seeded inputs.

Rows at or past an entry's length must be left exactly as they were (the
output and LSE buffers are filled with a marker first); the valid rows meet
the forward's bars (bf16: max abs 2e-2 and median relative 5e-3 on O, max abs
2e-2 on the LSE; f32: 1e-4)."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
import workloads as W
from tests.gpu_cases import announce, assert_close, f64

pytestmark = pytest.mark.gpu

MARK = 7.0

# (T, H, KV, d, io, causal, style, lengths, window, workspace): empty and
# one-token entries, lengths inside, at and across the 256-row unit and 64-key
# tile edges, full-length entries, no mask, a window, with and without the
# once-rotated keys, every head_dim, f32 and bf16.
CASES = [
    (300, 8, 2, 128, "bf16", True, "interleaved", [300, 0, 1, 257, 64], 0, True),
    (300, 8, 2, 128, "bf16", True, "interleaved", [299, 256, 65], 0, False),
    (200, 4, 4, 64, "bf16", False, "half", [200, 13, 129], 0, True),
    (129, 4, 2, 32, "f32", True, "interleaved", [129, 33, 2, 0], 0, False),
    (100, 4, 1, 64, "f32", False, "half", [7, 100], 0, False),
    (700, 6, 3, 64, "bf16", True, "interleaved", [700, 600, 513], 100, True),
    (1024, 16, 4, 128, "bf16", True, "half", [1000, 1024, 31], 0, True),
]


@pytest.mark.parametrize("T,H,KV,d,io,causal,style,lens,win,ws", CASES,
                         ids=[f"T{c[0]}_H{c[1]}_KV{c[2]}_d{c[3]}_{c[4]}_{'causal' if c[5] else 'nomask'}_{c[6]}_"
                              f"W{c[8]}_{'ws' if c[9] else 'nows'}_lens{'-'.join(map(str, c[7]))}" for c in CASES])
def test_padded_forward(gpu, T, H, KV, d, io, causal, style, lens, win, ws):
    B = len(lens)
    w = W.custom(f"pad_T{T}", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, dtype=io, rope_style=style,
                 causal=causal, seed=300 + T + sum(lens))
    announce(f"padded forward {w.name} B{B} H{H} KV{KV} d{d} {io} causal={causal} {style} W={win} "
             f"workspace={ws} lens={lens}")
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    q, k, v = (x[n].to(gpu) for n in ("q", "k", "v"))
    o = torch.full_like(q, MARK)
    lse = torch.full((B, H, T), MARK, dtype=torch.float32, device=gpu)
    sl = torch.tensor(lens, dtype=torch.int32, device=gpu)
    cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, causal=causal, rope_style=style, window=win, out=o, lse=lse,
                          seqlens=sl, workspace=None if ws else False)
    ro, rl = oracle.attention_padded(x["q"], x["k"], x["v"], lens, causal=causal, base=w.base, style=style,
                                     window=win)
    go, gl = f64(o), f64(lse)
    for b, n in enumerate(lens):
        assert (go[b, n:] == MARK).all(), f"entry {b}: a padding row of o was written"
        assert (gl[b, :, n:] == MARK).all(), f"entry {b}: a padding row of lse was written"
    valid_o = np.concatenate([go[b, :n].reshape(-1) for b, n in enumerate(lens)])
    ref_o = np.concatenate([ro[b, :n].reshape(-1) for b, n in enumerate(lens)])
    valid_l = np.concatenate([gl[b, :, :n].reshape(-1) for b, n in enumerate(lens)])
    ref_l = np.concatenate([rl[b, :, :n].reshape(-1) for b, n in enumerate(lens)])
    assert_close(w.name, valid_o, ref_o, valid_l, ref_l, io)


def test_padding_at_full_length_is_the_dense_call(gpu):
    """seqlens = T everywhere gives the same bits as no seqlens."""
    w = W.custom("pad_full", B=2, T=500, n_head=8, n_kv_head=2, head_dim=128, seed=17)
    x = W.make_inputs(w)
    cos, sin = cgr.rope_tables(500, 128, w.base, device=gpu)
    q, k, v = (x[n].to(gpu) for n in ("q", "k", "v"))
    o1, l1 = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin)
    o2, l2 = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, seqlens=torch.tensor([500, 500], dtype=torch.int32,
                                                                            device=gpu))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
