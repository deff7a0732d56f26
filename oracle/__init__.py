"""Float64 CPU oracle for the fused causal GQA + RoPE attention forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code with it; the product path fails when its extension is missing.

What it computes is the plain definition, written out with numpy in float64,
one (batch, head) at a time, with the full T x T score matrix materialised:

1. RoPE tables ("Embeddings & the Residual Stream", section "Positional
   information: RoPE"): inv_freq[i] = base^(-2i/d) for i < d/2, and the angle
   at position p is p * inv_freq[i].
2. Rotation of Q and K only, never V (same section; "Attention from Scratch",
   section "Attention, the math", step "Rotate"). Two pairings: "interleaved"
   rotates the adjacent pairs (2i, 2i+1), as the RoPE prose describes;
   "half" rotates (i, i + d/2), the x*cos + rotate_half(x)*sin form of the
   printed helper. See ``apply_rope``.
3. GQA sharing ("Attention, the math", step "Share"): query head h reads K/V
   head h // (n_head / n_kv_head), the repeat_interleave order.
4. Scores q.k * scale with scale = 1/sqrt(d) unless given (step "Score").
5. Causal mask: key j > query i gets -inf (the lower-triangular mask buffer and
   step "Mask + softmax"); or no mask.
6. Softmax over keys with the max shifted out, and the weighted sum of V
   (steps "Mask + softmax" and "Gather"). The forward also returns the natural
   log-sum-exp of each row's scaled, masked scores (not on the pages; it is
   what the row's softmax denominator is, in log form).

The backward (``attention_dense_bwd``, ``attention_varlen_bwd``) is the chain
rule applied to that definition, op by op in reverse ("Train It & Run for
Real", section "Coming from CUDA: where's .backward()?": backprop is the
chain rule through every op, RoPE and attention included): from dL/dO it
returns dL/dq, dL/dk, dL/dv of the un-rotated inputs.

Decode against a KV cache (``attention_decode``): the new queries of a
sequence are its last positions, so the causal mask aligns them with the end
of the cache ("Attention from Scratch", section "Attention, the math": GQA
shares each K/V head among several query heads so that the cache of keys and
values kept for generation shrinks by that factor).

The neighbours of attention in the block (``rmsnorm``, ``rmsnorm_qkv_rope``):
pre-norm RMSNorm ("The Transformer Block & the Model", section "RMSNorm:
normalizing before every sub-layer": x / sqrt(mean(x^2) + eps) * weight), then
the bias-free q, k, v projections and RoPE on q and k ("Attention from
Scratch", "Attention, the math": project, then rotate).

Packed variable-length batches (the kohakutt page, Highlights: "packed
variable-length batches") are the concatenation of independent sequences:
positions restart at 0 in every sequence and the mask never crosses a
sequence boundary.

Every function here is pinned by ``tests/test_oracle_pins.py`` to results the
pages and the mathematics fix (closed forms, invariants, a library routine on
a special case, brute force on tiny inputs).
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "rope_inv_freq",
    "rope_tables",
    "apply_rope",
    "attention_dense",
    "attention_varlen",
    "attention_rows",
    "apply_rope_transpose",
    "attention_dense_bwd",
    "attention_varlen_bwd",
    "attention_bwd_group",
    "attention_decode",
    "rmsnorm",
    "rmsnorm_qkv_rope",
]


def _f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        # bf16 has no numpy dtype: go through float32, which holds every bf16 value exactly.
        x = x.float().numpy() if str(x.dtype) in ("torch.bfloat16", "torch.float16") else x.numpy()
    return np.asarray(x, dtype=np.float64)


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """inv_freq[i] = base^(-2i/head_dim), i < head_dim/2.

    "Embeddings & the Residual Stream", section "Positional information: RoPE":
    the angle shrinks with the feature index through this power of the fixed
    base (theta).
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even: RoPE rotates feature pairs")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope_tables(max_pos: int, head_dim: int, base: float):
    """cos and sin of angle(p, i) = p * inv_freq[i], each [max_pos, head_dim/2] float64.

    Same section as ``rope_inv_freq``. The page duplicates the half table to
    full width for its rotate_half form; both pairings here index the half
    table by pair number instead, which carries the same numbers.
    """
    pos = np.arange(max_pos, dtype=np.float64)
    ang = np.outer(pos, rope_inv_freq(head_dim, base))
    return np.cos(ang), np.sin(ang)


def apply_rope(x, positions, base: float, style: str = "interleaved") -> np.ndarray:
    """Rotate the last dim of x ([T, ..., d]) at the given positions ([T]).

    Pair i (partners a_i, b_i) turns by angle(p, i):
        y[a_i] = x[a_i] cos - x[b_i] sin,  y[b_i] = x[a_i] sin + x[b_i] cos.
    "interleaved": (a_i, b_i) = (2i, 2i+1), "each adjacent pair of features"
    in the RoPE prose. "half": (a_i, b_i) = (i, i + d/2), which is exactly
    x*cos + rotate_half(x)*sin with rotate_half(x) = (-x2, x1) and the
    duplicated half table ("Embeddings & the Residual Stream", printed
    rotate_half / apply_rope).
    """
    x = _f64(x)
    d = x.shape[-1]
    pos = np.asarray(positions, dtype=np.float64)
    ang = np.outer(pos, rope_inv_freq(d, base))  # [T, d/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    y = np.empty_like(x)
    if style == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = a * s + b * c
    elif style == "half":
        a, b = x[..., : d // 2], x[..., d // 2:]
        y[..., : d // 2] = a * c - b * s
        y[..., d // 2:] = a * s + b * c
    else:
        raise ValueError(f"unknown rope style {style!r}")
    return y


def _hidden(qpos, kpos, causal: bool, window: int) -> np.ndarray:
    """[len(qpos), len(kpos)]: True where the query at position qpos[i] may not
    see the key at kpos[j] -- a later key (causal), or, with window W > 0, a
    key W or more positions back (sliding window: 0 <= i - j < W is visible)."""
    qp = np.asarray(qpos)[:, None]
    kp = np.asarray(kpos)[None, :]
    hide = np.zeros((qp.shape[0], kp.shape[1]), dtype=bool)
    if causal:
        hide |= kp > qp
    if window > 0:
        hide |= qp - kp >= window
    return hide


def _check_window(causal: bool, window: int):
    if window < 0:
        raise ValueError("window must be >= 0 (0: no window)")
    if window > 0 and not causal:
        raise ValueError("a sliding window needs the causal mask")


def _one_sequence(q, k, v, causal: bool, scale: float, base: float, style: str, window: int = 0):
    """Attention for one sequence. q [L, H, d], k/v [L, KV, d] float64.

    Returns O [L, H, d] and lse [H, L]. The score matrix of every head is
    materialised in full ("Attention, the math": scores, masked_fill, softmax,
    weights @ v).
    """
    L, H, d = q.shape
    KV = k.shape[1]
    G = H // KV
    pos = np.arange(L)
    qr = apply_rope(q, pos, base, style)
    kr = apply_rope(k, pos, base, style)
    O = np.empty((L, H, d), dtype=np.float64)
    lse = np.empty((H, L), dtype=np.float64)
    if L == 0:
        return O, lse
    hidden = _hidden(pos, pos, causal, window)
    for h in range(H):
        kv = h // G  # repeat_interleave: heads of one group are adjacent
        S = (qr[:, h, :] @ kr[:, kv, :].T) * scale
        S[hidden] = -np.inf
        m = S.max(axis=1)
        e = np.exp(S - m[:, None])
        den = e.sum(axis=1)
        lse[h] = m + np.log(den)
        P = e / den[:, None]
        O[:, h, :] = P @ v[:, kv, :]
    return O, lse


def _check_heads(n_head: int, n_kv_head: int):
    if n_kv_head < 1 or n_head % n_kv_head:
        raise ValueError("n_head must be divisible by n_kv_head")


def attention_dense(q, k, v, *, causal: bool = True, base: float = 10000.0,
                    style: str = "interleaved", scale: Optional[float] = None, window: int = 0):
    """Dense batch: q [B,T,H,d], k/v [B,T,KV,d]. Returns O [B,T,H,d], lse [B,H,T] (float64).

    window W > 0 (with the causal mask) keeps only keys 0 <= i - j < W."""
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, d = q.shape
    _check_heads(H, k.shape[2])
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        O[b], lse[b] = _one_sequence(q[b], k[b], v[b], causal, scale, base, style, window)
    return O, lse


def attention_padded(q, k, v, seqlens, *, causal: bool = True, base: float = 10000.0,
                     style: str = "interleaved", scale: Optional[float] = None, window: int = 0):
    """Dense batch with right padding (a padding mask; "masks" in the Kohaku-TT
    feature list): entry b holds seqlens[b] tokens followed by padding. The
    padding keys are hidden from every query, so the first seqlens[b] rows are
    the attention of that prefix on its own, positions from 0; the padding rows
    have no output and are NaN here. Returns O [B,T,H,d], lse [B,H,T]."""
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, d = q.shape
    _check_heads(H, k.shape[2])
    lens = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    if len(lens) != B or any(n < 0 or n > T for n in lens):
        raise ValueError("seqlens must hold B values in [0, T]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.full_like(q, np.nan)
    lse = np.full((B, H, T), np.nan, dtype=np.float64)
    for b, n in enumerate(lens):
        if n > 0:
            O[b, :n], lse[b, :, :n] = _one_sequence(q[b, :n], k[b, :n], v[b, :n], causal, scale, base, style,
                                                    window)
    return O, lse


def attention_varlen(q, k, v, cu_seqlens, *, causal: bool = True, base: float = 10000.0,
                     style: str = "interleaved", scale: Optional[float] = None, window: int = 0):
    """Packed batch: q [total,H,d], k/v [total,KV,d], cu_seqlens [n+1].

    Each sequence s occupies tokens cu[s]..cu[s+1]-1 and is attended to on its
    own, positions restarting at 0. Returns O [total,H,d], lse [H,total].
    """
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    total, H, d = q.shape
    _check_heads(H, k.shape[1])
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.empty_like(q)
    lse = np.empty((H, total), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        O[a:b], lse[:, a:b] = _one_sequence(q[a:b], k[a:b], v[a:b], causal, scale, base, style, window)
    return O, lse


def attention_rows(q, k, v, rows: Sequence, *, causal: bool = True, base: float = 10000.0,
                   style: str = "interleaved", scale: Optional[float] = None,
                   cu_seqlens=None, window: int = 0):
    """O and lse of selected output rows only, one row at a time.

    ``rows`` lists (b, t, h) for a dense batch (q [B,T,H,d]) or (s, t, h) for a
    packed one (t local to sequence s, q [total,H,d] with ``cu_seqlens``).
    Row (t, h) needs the rotated query at position t and every rotated key of
    its sequence that the mask allows; nothing else is computed, so sampled
    checks at full size stay cheap. Returns (O [n, d], lse [n]) float64.
    """
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if cu_seqlens is None:
        H, KV = q.shape[2], k.shape[2]
    else:
        H, KV = q.shape[1], k.shape[1]
        cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    _check_heads(H, KV)
    G = H // KV
    outs, lses = [], []
    for (b, t, h) in rows:
        if cu_seqlens is None:
            L = q.shape[1]
            qrow = q[b, t, h]
            keys, vals = k[b, :, h // G], v[b, :, h // G]
        else:
            a = cu[b]
            L = cu[b + 1] - a
            qrow = q[a + t, h]
            keys, vals = k[a:a + L, h // G], v[a:a + L, h // G]
        n = t + 1 if causal else L
        lo = max(0, t - window + 1) if window > 0 else 0
        qr = apply_rope(qrow[None, :], [t], base, style)[0]
        kr = apply_rope(keys[lo:n], np.arange(lo, n), base, style)
        s = (kr @ qr) * scale
        m = s.max()
        e = np.exp(s - m)
        den = e.sum()
        outs.append((e / den) @ vals[lo:n])
        lses.append(m + math.log(den))
    return np.array(outs).reshape(len(rows), d), np.array(lses)


# ----------------------------------------------------------------------------- backward

def apply_rope_transpose(g, positions, base: float, style: str = "interleaved") -> np.ndarray:
    """The transpose of the rotation of ``apply_rope``, applied to g ([T, ..., d]).

    The chain rule through y = R(p) x gives dL/dx = R(p)^T dL/dy. Pair i
    (partners a_i, b_i) turns back by angle(p, i):
        x[a_i] = g[a_i] cos + g[b_i] sin,  x[b_i] = -g[a_i] sin + g[b_i] cos.
    """
    g = _f64(g)
    d = g.shape[-1]
    pos = np.asarray(positions, dtype=np.float64)
    ang = np.outer(pos, rope_inv_freq(d, base))
    shape = (g.shape[0],) + (1,) * (g.ndim - 2) + (d // 2,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x = np.empty_like(g)
    if style == "interleaved":
        a, b = g[..., 0::2], g[..., 1::2]
        x[..., 0::2] = a * c + b * s
        x[..., 1::2] = -a * s + b * c
    elif style == "half":
        a, b = g[..., : d // 2], g[..., d // 2:]
        x[..., : d // 2] = a * c + b * s
        x[..., d // 2:] = -a * s + b * c
    else:
        raise ValueError(f"unknown rope style {style!r}")
    return x


def _one_sequence_bwd(q, k, v, dout, causal: bool, scale: float, base: float, style: str,
                      window: int = 0):
    """Gradients for one sequence: q, dout [L, H, d], k/v [L, KV, d] float64.

    Reverse of ``_one_sequence``, op by op, for every head:
        O = P V                  ->  dV += P^T dO,  dP = dO V^T
        P = softmax_j(S)         ->  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
        S = scale * Qr Kr^T      ->  dQr = scale dS Kr,  dKr += scale dS^T Qr
        Qr = R Q, Kr = R K       ->  dQ = R^T dQr,  dK = R^T dKr
    The heads of one K/V group add their contributions to that group's dK and
    dV. Masked entries have P = 0 and so dS = 0.
    """
    L, H, d = q.shape
    KV = k.shape[1]
    G = H // KV
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if L == 0:
        return dq, dk, dv
    pos = np.arange(L)
    qr = apply_rope(q, pos, base, style)
    kr = apply_rope(k, pos, base, style)
    dqr = np.zeros_like(q)
    dkr = np.zeros_like(k)
    hidden = _hidden(pos, pos, causal, window)
    for h in range(H):
        kv = h // G
        S = (qr[:, h, :] @ kr[:, kv, :].T) * scale
        S[hidden] = -np.inf
        e = np.exp(S - S.max(axis=1)[:, None])
        P = e / e.sum(axis=1)[:, None]
        dv[:, kv, :] += P.T @ dout[:, h, :]
        dP = dout[:, h, :] @ v[:, kv, :].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dqr[:, h, :] = (dS @ kr[:, kv, :]) * scale
        dkr[:, kv, :] += (dS.T @ qr[:, h, :]) * scale
    dq = apply_rope_transpose(dqr, pos, base, style)
    dk = apply_rope_transpose(dkr, pos, base, style)
    return dq, dk, dv


def attention_dense_bwd(q, k, v, dout, *, causal: bool = True, base: float = 10000.0,
                        style: str = "interleaved", scale: Optional[float] = None, window: int = 0):
    """Dense batch backward: q/dout [B,T,H,d], k/v [B,T,KV,d] -> dq, dk, dv (float64, same shapes)."""
    _check_window(causal, window)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, H, d = q.shape
    _check_heads(H, k.shape[2])
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        dq[b], dk[b], dv[b] = _one_sequence_bwd(q[b], k[b], v[b], dout[b], causal, scale, base, style,
                                                window)
    return dq, dk, dv


def attention_varlen_bwd(q, k, v, dout, cu_seqlens, *, causal: bool = True, base: float = 10000.0,
                         style: str = "interleaved", scale: Optional[float] = None, window: int = 0):
    """Packed batch backward: q/dout [total,H,d], k/v [total,KV,d], cu_seqlens [n+1]; each sequence
    on its own, positions restarting at 0. Returns dq, dk, dv (float64, same shapes)."""
    _check_window(causal, window)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    total, H, d = q.shape
    _check_heads(H, k.shape[1])
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        dq[a:b], dk[a:b], dv[a:b] = _one_sequence_bwd(q[a:b], k[a:b], v[a:b], dout[a:b], causal, scale,
                                                      base, style, window)
    return dq, dk, dv


def attention_bwd_group(q, k, v, dout, b: int, kv: int, *, causal: bool = True, base: float = 10000.0,
                        style: str = "interleaved", scale: Optional[float] = None, rows_per_block: int = 512,
                        window: int = 0):
    """Gradients that involve one K/V head of one dense batch entry, for long sequences.

    Same arithmetic as ``_one_sequence_bwd`` restricted to batch entry b, K/V
    head kv and its query heads, with the score matrix built a block of query
    rows at a time (every row whole, so each row's softmax is exact) to bound
    memory. Under the causal mask a block of rows ending at r1 only needs keys
    below r1, and with a window W only keys from r0 - W + 1 on: the others
    have weight exactly 0.
    Returns dq [T, G, d] (the group's query heads, in order), dk [T, d], dv [T, d].
    """
    _check_window(causal, window)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, H, d = q.shape
    KV = k.shape[2]
    _check_heads(H, KV)
    G = H // KV
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    pos = np.arange(T)
    kr = apply_rope(k[b, :, kv], pos, base, style)
    vv = v[b, :, kv]
    dqr = np.zeros((T, G, d))
    dkr = np.zeros((T, d))
    dv = np.zeros((T, d))
    for g in range(G):
        h = kv * G + g
        qr = apply_rope(q[b, :, h], pos, base, style)
        do = dout[b, :, h]
        for r0 in range(0, T, rows_per_block):
            r1 = min(T, r0 + rows_per_block)
            n = r1 if causal else T
            lo = max(0, r0 - window + 1) if window > 0 else 0
            S = (qr[r0:r1] @ kr[lo:n].T) * scale
            S[_hidden(np.arange(r0, r1), np.arange(lo, n), causal, window)] = -np.inf
            e = np.exp(S - S.max(axis=1)[:, None])
            P = e / e.sum(axis=1)[:, None]
            dv[lo:n] += P.T @ do[r0:r1]
            dP = do[r0:r1] @ vv[lo:n].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dqr[r0:r1, g] = (dS @ kr[lo:n]) * scale
            dkr[lo:n] += (dS.T @ qr[r0:r1]) * scale
    dq = apply_rope_transpose(dqr, pos, base, style)
    dk = apply_rope_transpose(dkr, pos, base, style)
    return dq, dk, dv


def attention_decode(q, k, v, cache_seqlens, *, base: float = 10000.0, style: str = "interleaved",
                     scale: Optional[float] = None, window: int = 0):
    """New queries against a KV cache.

    q [B, Tq, H, d]: the Tq newest tokens of each sequence; k, v [B, S, KV, d]:
    the cache, un-rotated, of which batch entry b uses rows 0 .. L_b - 1 with
    L_b = cache_seqlens[b] >= Tq (the new tokens' own keys are its last Tq
    rows). Query i of entry b sits at position L_b - Tq + i and sees the keys
    at positions j <= L_b - Tq + i (the causal mask aligned with the end of the
    cache); with window W > 0 only keys 0 <= position - j < W. Returns
    O [B, Tq, H, d] and lse [B, H, Tq] (float64).
    """
    _check_window(True, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Tq, H, d = q.shape
    KV = k.shape[2]
    _check_heads(H, KV)
    G = H // KV
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    O = np.empty_like(q)
    lse = np.empty((B, H, Tq), dtype=np.float64)
    for b in range(B):
        L = lens[b]
        if not (Tq <= L <= k.shape[1]):
            raise ValueError(f"cache length {L} of entry {b} must lie in [Tq, S]")
        qpos = np.arange(L - Tq, L)
        qr = apply_rope(q[b], qpos, base, style)
        kr = apply_rope(k[b, :L], np.arange(L), base, style)
        hidden = _hidden(qpos, np.arange(L), True, window)
        for h in range(H):
            kv = h // G
            S = (qr[:, h, :] @ kr[:, kv, :].T) * scale
            S[hidden] = -np.inf
            m = S.max(axis=1)
            e = np.exp(S - m[:, None])
            den = e.sum(axis=1)
            lse[b, h] = m + np.log(den)
            O[b, :, h, :] = (e / den[:, None]) @ v[b, :L, kv, :]
    return O, lse


def rmsnorm(x, weight, eps: float) -> np.ndarray:
    """x [..., C] -> x / sqrt(mean(x^2 over C) + eps) * weight (float64)."""
    x = _f64(x)
    w = _f64(weight)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rmsnorm_qkv_rope(x, norm_weight, eps: float, w_qkv, positions, n_head: int, n_kv_head: int,
                     *, base: float = 10000.0, style: str = "interleaved", rotate_q: bool = True,
                     rotate_k: bool = True):
    """The block's pre-attention steps for N tokens: xn = rmsnorm(x), then
    q = xn W_q^T, k = xn W_k^T, v = xn W_v^T (no bias), and RoPE on q and/or k
    at each token's position.

    x [N, C]; w_qkv [(n_head + 2 n_kv_head) * d, C]: the rows of W_q, then W_k,
    then W_v (nn.Linear's [out, in] layout); positions [N].
    Returns q [N, n_head, d], k [N, n_kv_head, d], v [N, n_kv_head, d] (float64).
    """
    x = _f64(x)
    W = _f64(w_qkv)
    N = x.shape[0]
    d = W.shape[0] // (n_head + 2 * n_kv_head)
    if d * (n_head + 2 * n_kv_head) != W.shape[0]:
        raise ValueError("w_qkv rows must be (n_head + 2 n_kv_head) * head_dim")
    y = rmsnorm(x, norm_weight, eps) @ W.T
    q = y[:, : n_head * d].reshape(N, n_head, d)
    k = y[:, n_head * d:(n_head + n_kv_head) * d].reshape(N, n_kv_head, d)
    v = y[:, (n_head + n_kv_head) * d:].reshape(N, n_kv_head, d)
    if rotate_q:
        q = apply_rope(q, positions, base, style)
    if rotate_k:
        k = apply_rope(k, positions, base, style)
    return q, k, v
