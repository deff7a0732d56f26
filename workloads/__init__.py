"""Seeded synthetic inputs for causal GQA + RoPE attention.

This module only draws random tensors and names shapes. It holds none of the
attention or RoPE arithmetic, so both the float64 oracle (``oracle/``) and the
HIP path (``causal_gqa_rope_amd``) can take their inputs from here without
sharing any of the method's code.

Shapes follow the workloads the pages describe:

* "Attention from Scratch", section "Attention, the math": n_head query heads
  share n_kv_groups K/V heads; tensors are laid out [B, T, heads, head_dim]
  after the projection view.
* "The Transformer Block & the Model", section "Scaling nano to ~80M": the
  nanollama3 config (6 heads, 3 KV groups, theta 500000, block_size 256,
  n_embd 384, so head_dim 64).
* "kohakutt" (PyPI page), Highlights and the tt-xla comparison table: flash
  attention over MHA/GQA/MQA, causal masks and packed variable-length batches;
  a Qwen2.5-0.5B 77-token prefill.

Draw recipe (every workload): ``torch.Generator('cpu').manual_seed(seed)``;
for packed batches the sequence lengths are drawn first with
``torch.randint(lo, hi + 1, (num_seqs,))``; then ``torch.randn`` in float32 in
the order Q, K, V; optional K outliers (``torch.rand(K.shape) < frac`` scaled by
``factor``); finally one cast to the I/O dtype. Consumers upcast the cast values,
so every side sees bit-identical inputs.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "PARITY_EXTRAS",
    "get",
    "make_inputs",
    "varlen_lengths",
    "make_dout",
    "visible_pairs",
    "algorithmic_flops",
    "algorithmic_flops_bwd",
    "DecodeWorkload",
    "DECODE_WORKLOADS",
    "make_decode_inputs",
    "decode_bytes",
    "QkvWorkload",
    "QKV_WORKLOADS",
    "WIDE_WORKLOADS",
    "FP8_WORKLOADS",
    "quantize_fp8",
    "make_fp8_inputs",
    "padded_lengths",
    "make_qkv_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload.

    ``lengths is None`` means a dense [B, T, H, d] batch; otherwise a packed
    batch of ``num_seqs`` sequences whose lengths are drawn uniformly from
    ``[len_lo, len_hi]`` (inclusive) by the workload's seed.
    """

    name: str
    B: int
    T: int
    n_head: int
    n_kv_head: int
    head_dim: int
    base: float
    dtype: str  # "f32" or "bf16": the I/O dtype
    seed: int
    causal: bool = True
    rope_style: str = "interleaved"  # "interleaved" pairs (2i, 2i+1); "half" pairs (i, i + d/2)
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0
    num_seqs: int = 0  # > 0 marks a packed variable-length batch
    len_lo: int = 0
    len_hi: int = 0

    @property
    def varlen(self) -> bool:
        return self.num_seqs > 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the measurements are quoted on (sizes as named).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_T64_H4_KV2_d32", B=1, T=64, n_head=4, n_kv_head=2, head_dim=32,
                 base=10000.0, dtype="f32", seed=0),
        Workload("nanollama3_train_B8_T256_H6_KV2_d64", B=8, T=256, n_head=6, n_kv_head=2,
                 head_dim=64, base=10000.0, dtype="bf16", seed=1),
        Workload("qwen05b_prefill_T77_H14_KV2_d64_koutliers", B=1, T=77, n_head=14, n_kv_head=2,
                 head_dim=64, base=1e6, dtype="bf16", seed=2, outlier_frac=0.005,
                 outlier_factor=20.0),
        Workload("long_context_T8192_H32_KV8_d128", B=1, T=8192, n_head=32, n_kv_head=8,
                 head_dim=128, base=500000.0, dtype="bf16", seed=3),
        Workload("varlen_mqa_32seqs_16to2048_H16_KV1_d128", B=1, T=0, n_head=16, n_kv_head=1,
                 head_dim=128, base=10000.0, dtype="bf16", seed=4, num_seqs=32, len_lo=16,
                 len_hi=2048),
    ]
}

# Extra parity cases (never bench lines).
PARITY_EXTRAS = {
    w.name: w
    for w in [
        # The pages' own nanollama3 attention: 6 heads, 3 KV groups, theta 500000, T 256.
        Workload("nanollama3_pages_B8_T256_H6_KV3_d64", B=8, T=256, n_head=6, n_kv_head=3,
                 head_dim=64, base=500000.0, dtype="bf16", seed=11),
        # rotate_half pairing on the three small workloads.
        WORKLOADS["tiny_fp32_T64_H4_KV2_d32"].replace(
            name="tiny_fp32_T64_H4_KV2_d32_half", rope_style="half"),
        WORKLOADS["nanollama3_train_B8_T256_H6_KV2_d64"].replace(
            name="nanollama3_train_B8_T256_H6_KV2_d64_half", rope_style="half"),
        WORKLOADS["qwen05b_prefill_T77_H14_KV2_d64_koutliers"].replace(
            name="qwen05b_prefill_T77_H14_KV2_d64_koutliers_half", rope_style="half"),
        # No mask.
        WORKLOADS["nanollama3_train_B8_T256_H6_KV2_d64"].replace(
            name="nanollama3_train_B8_T256_H6_KV2_d64_nomask", causal=False),
    ]
}


# fp8 operands: the long-context workload with its q, k, v quantized per
# tensor to e4m3 (make_fp8_inputs); a bench line against the fp8 peak.
FP8_WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp8_long_context_T8192_H32_KV8_d128", B=1, T=8192, n_head=32, n_kv_head=8, head_dim=128,
                 base=500000.0, dtype="f32", seed=3),
    ]
}

# head_dim 256: the long-context workload's width (n_head * head_dim = 4096)
# in half as many, twice as wide heads (a parity case and its own bench line).
WIDE_WORKLOADS = {
    w.name: w
    for w in [
        Workload("long_context_T8192_H16_KV8_d256", B=1, T=8192, n_head=16, n_kv_head=8, head_dim=256,
                 base=500000.0, dtype="bf16", seed=5),
    ]
}


def get(name: str) -> Workload:
    for table in (WORKLOADS, PARITY_EXTRAS, WIDE_WORKLOADS, FP8_WORKLOADS):
        if name in table:
            return table[name]
    raise KeyError(name)


def varlen_lengths(w: Workload, gen: Optional[torch.Generator] = None) -> torch.Tensor:
    """Sequence lengths of a packed workload (int64, CPU), drawn first from the seed."""
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(w.seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.num_seqs,), generator=gen)


def _io_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload) -> dict:
    """Draw the seeded CPU tensors of a workload.

    Returns a dict with ``q``, ``k``, ``v`` in the I/O dtype and, for packed
    batches, ``cu_seqlens`` (int32, [num_seqs + 1]), ``lengths`` and
    ``max_seqlen``. Dense tensors are [B, T, H, d] / [B, T, KV, d]; packed ones
    are [total, H, d] / [total, KV, d].
    """
    gen = torch.Generator("cpu").manual_seed(w.seed)
    out = {}
    if w.varlen:
        lengths = varlen_lengths(w, gen)
        total = int(lengths.sum())
        cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(lengths, 0).to(torch.int32)
        qshape = (total, w.n_head, w.head_dim)
        kshape = (total, w.n_kv_head, w.head_dim)
        out.update(cu_seqlens=cu, lengths=lengths, max_seqlen=int(lengths.max()),
                   total_tokens=total)
    else:
        qshape = (w.B, w.T, w.n_head, w.head_dim)
        kshape = (w.B, w.T, w.n_kv_head, w.head_dim)
    q = torch.randn(qshape, generator=gen, dtype=torch.float32)
    k = torch.randn(kshape, generator=gen, dtype=torch.float32)
    v = torch.randn(kshape, generator=gen, dtype=torch.float32)
    if w.outlier_frac > 0.0:
        sel = torch.rand(kshape, generator=gen) < w.outlier_frac
        k = torch.where(sel, k * w.outlier_factor, k)
    dt = _io_dtype(w.dtype)
    out.update(q=q.to(dt), k=k.to(dt), v=v.to(dt))
    return out


def quantize_fp8(x: torch.Tensor):
    """Per-tensor e4m3 quantization of a float tensor: descale = amax / 448
    (rounded to float32), codes = x / descale rounded to the nearest e4m3
    (torch's conversion). Returns (codes as torch.float8_e4m3fn, descale)."""
    amax = float(x.abs().max())
    descale = float(torch.tensor(amax / 448.0 if amax > 0 else 1.0, dtype=torch.float32))
    return (x.to(torch.float32) / descale).to(torch.float8_e4m3fn), descale


def make_fp8_inputs(w: Workload) -> dict:
    """The workload's q, k, v drawn as for make_inputs (float32, same seed and
    order), then quantized per tensor to e4m3 (quantize_fp8). Returns q, k, v
    (torch.float8_e4m3fn, CPU), their descales, and the dequantized float64
    numpy arrays q64, k64, v64 that the exact attention is taken of."""
    x = make_inputs(dataclasses.replace(w, dtype="f32"))
    out = {}
    for n in ("q", "k", "v"):
        codes, ds = quantize_fp8(x[n])
        out[n] = codes
        out[n + "_descale"] = ds
        out[n + "64"] = codes.to(torch.float64).numpy() * ds
    return out


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with explicit fields (used by edge-case parity tests)."""
    defaults = dict(B=1, T=1, n_head=1, n_kv_head=1, head_dim=64, base=10000.0, dtype="bf16",
                    seed=0)
    defaults.update(kw)
    return Workload(name, **defaults)


def padded_lengths(B: int, lo: int, hi: int, seed: int) -> list:
    """Valid lengths of a right-padded dense batch: B draws, uniform in [lo, hi]
    (inclusive), from a generator of its own seed."""
    gen = torch.Generator("cpu").manual_seed(seed + 7919)
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=gen)]


def visible_pairs(L: int, causal: bool, window: int = 0) -> int:
    """Allowed (query, key) pairs of one sequence of length L: L(L+1)/2 causal,
    L^2 unmasked; with a sliding window W, row i sees min(i + 1, W) keys."""
    L = int(L)
    if not causal:
        return L * L
    if window <= 0 or window >= L:
        return L * (L + 1) // 2
    return window * (window + 1) // 2 + (L - window) * window


def algorithmic_flops(n_head: int, head_dim: int, lengths, causal: bool, window: int = 0) -> int:
    """FLOPs credited to one forward: 4*d per allowed (query, key) pair per query head.

    2*d for the score dot product and 2*d for the weighted sum of V.
    Exponentials, RoPE and rescaling are not counted.
    """
    return 4 * head_dim * n_head * sum(visible_pairs(L, causal, window) for L in lengths)


# Seed offset of the upstream gradient dL/dO, so it is a stream of its own and
# the workload's q, k, v stay what they are without it.
DOUT_SEED_OFFSET = 1_000_003


def make_dout(w: Workload, like: torch.Tensor) -> torch.Tensor:
    """dL/dO for a workload: N(0,1) iid in the I/O dtype, q's shape, from seed + 1000003."""
    gen = torch.Generator("cpu").manual_seed(w.seed + DOUT_SEED_OFFSET)
    return torch.randn(tuple(like.shape), generator=gen, dtype=torch.float32).to(_io_dtype(w.dtype))


def algorithmic_flops_bwd(n_head: int, head_dim: int, lengths, causal: bool, window: int = 0) -> int:
    """FLOPs credited to one backward: 10*d per allowed (query, key) pair per query head.

    Five products of 2*d each per pair: the recomputed scores q.k, dO.v, and
    the three gradient sums dv += p dO, dk += ds q, dq += ds k (2.5 times the
    forward's count). The recomputation that splitting dq from dk/dv costs is
    not credited.
    """
    return algorithmic_flops(n_head, head_dim, lengths, causal, window) // 4 * 10


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """New queries against a KV cache: B sequences with cache lengths drawn
    uniformly from [len_lo, len_hi] (inclusive) by the seed, the Tq newest
    tokens of each as queries; the cache has room for `capacity` tokens."""

    name: str
    B: int
    Tq: int
    capacity: int
    n_head: int
    n_kv_head: int
    head_dim: int
    base: float
    seed: int
    len_lo: int
    len_hi: int
    rope_style: str = "interleaved"

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        # One serving step of the long-context model's attention: 16 sequences,
        # one new token each, caches of 4096 to 8192 tokens.
        DecodeWorkload("decode_B16_Tq1_cache4096to8192_H32_KV8_d128", B=16, Tq=1, capacity=8192,
                       n_head=32, n_kv_head=8, head_dim=128, base=500000.0, seed=20, len_lo=4096,
                       len_hi=8192),
    ]
}


def make_decode_inputs(w: DecodeWorkload) -> dict:
    """Seeded CPU tensors: cache lengths first (int32 [B]), then q [B, Tq, H, d] and the
    un-rotated k, v caches [B, capacity, KV, d], all N(0,1), cast once to bf16."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    lens = torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=gen).to(torch.int32)
    q = torch.randn((w.B, w.Tq, w.n_head, w.head_dim), generator=gen, dtype=torch.float32)
    k = torch.randn((w.B, w.capacity, w.n_kv_head, w.head_dim), generator=gen, dtype=torch.float32)
    v = torch.randn((w.B, w.capacity, w.n_kv_head, w.head_dim), generator=gen, dtype=torch.float32)
    return dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16), cache_seqlens=lens,
                max_seqlen=int(lens.max()))


def decode_bytes(w: DecodeWorkload, lens) -> int:
    """Bytes one decode call must move at least: the used K and V cache rows
    (bf16), the queries in, the outputs out (bf16) and their log-sum-exp (f32)."""
    cache = sum(int(L) for L in lens) * w.n_kv_head * w.head_dim * 2 * 2
    qo = 2 * w.B * w.Tq * w.n_head * w.head_dim * 2
    return cache + qo + w.B * w.n_head * w.Tq * 4


@dataclasses.dataclass(frozen=True)
class QkvWorkload:
    """The block's pre-attention step: RMSNorm, q/k/v projections, RoPE, for
    B sequences of T tokens of width n_embd (positions 0 .. T-1 in each)."""

    name: str
    B: int
    T: int
    n_embd: int
    n_head: int
    n_kv_head: int
    head_dim: int
    base: float
    seed: int
    eps: float = 1e-6
    rope_style: str = "interleaved"

    def replace(self, **kw) -> "QkvWorkload":
        return dataclasses.replace(self, **kw)


QKV_WORKLOADS = {
    w.name: w
    for w in [
        # The long-context model (n_embd = n_head * head_dim) over one 8192-token sequence.
        QkvWorkload("qkv_long_context_T8192_C4096_H32_KV8_d128", B=1, T=8192, n_embd=4096, n_head=32,
                    n_kv_head=8, head_dim=128, base=500000.0, seed=30),
        # The pages' nanollama3 block: n_embd 384, 6 heads, 3 KV groups, theta 500000, B8 x T256.
        QkvWorkload("qkv_nanollama3_B8_T256_C384_H6_KV3_d64", B=8, T=256, n_embd=384, n_head=6,
                    n_kv_head=3, head_dim=64, base=500000.0, seed=31),
    ]
}


def make_qkv_inputs(w: QkvWorkload) -> dict:
    """Seeded CPU tensors in bf16: x [N, C] ~ N(0,1); norm_weight [C] ~ 1 + 0.1 N(0,1);
    w_qkv [(H + 2 KV) d, C] ~ N(0,1) / sqrt(C); positions int32 [N] = t mod T."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    N, C = w.B * w.T, w.n_embd
    O = (w.n_head + 2 * w.n_kv_head) * w.head_dim
    x = torch.randn((N, C), generator=gen)
    g = 1.0 + 0.1 * torch.randn((C,), generator=gen)
    W = torch.randn((O, C), generator=gen) / (C ** 0.5)
    pos = (torch.arange(N) % w.T).to(torch.int32)
    return dict(x=x.to(torch.bfloat16), norm_weight=g.to(torch.bfloat16), w_qkv=W.to(torch.bfloat16),
                positions=pos)
