"""A rounding model of the fp8-operand forward, used to derive its test bar.

Not the oracle: the oracle is the exact attention of the dequantized inputs
(`oracle.attention_dense` on codes x descale). This model takes the same
steps as the fp8 arithmetic the library documents, in float64 numpy, rounding
where that arithmetic rounds, so its distance to the oracle shows how far
e4m3 operands alone move the result:
  * q and k rotated at their positions (in e4m3 units), q times gamma in
    [1/4, 1/2), k halved, both rounded to e4m3;
  * scores in log2 units = (rounded q . rounded k) times the remaining power
    of two; the row reference m is the row's max over the first 64 keys;
  * p = 2^(s - m) rounded to e4m3 for the P.V product, the row sum over the
    unrounded p; O = (P V codes) * v_descale / row sum;
  * rows go in blocks of 128 (the library's work unit): if some p of a
    block would leave e4m3's range (above 464, which rounds to NaN), the block
    is redone as the classic online softmax over 64-key tiles: the running
    max is updated per tile, p = 2^(s - running max) is rounded, and O and
    the row sum are rescaled by 2^(old max - new max).
It shares nothing with the HIP path; e4m3 rounding is torch's conversion."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def e4m3(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def model_forward(q8, k8, v8, q_ds, k_ds, v_ds, *, base, style="interleaved", causal=True, tile=64, block=128):
    """q8 [T,H,d], k8/v8 [T,KV,d] float64 e4m3 code values -> O [T,H,d], lse [H,T]."""
    T, H, d = q8.shape
    G = H // k8.shape[1]
    pos = np.arange(T)
    qr = oracle.apply_rope(q8, pos, base, style)
    kr = oracle.apply_rope(k8, pos, base, style)
    c = q_ds * 2.0 * k_ds / math.sqrt(d) * math.log2(math.e)
    f, e = math.frexp(c)
    qt, kt = e4m3(qr * (f / 2)), e4m3(kr / 2)
    O = np.empty((T, H, d))
    L = np.empty((H, T))
    for h in range(H):
        vh = v8[:, h // G]
        Sh = (qt[:, h] @ kt[:, h // G].T) * 2.0 ** (e + 1)
        if causal:
            Sh[np.triu_indices(T, 1)] = -np.inf
        for r0 in range(0, T, block):
            rows = slice(r0, min(r0 + block, T))
            S = Sh[rows]
            m = S[:, :tile].max(axis=1, keepdims=True)
            if (S - m).max() <= math.log2(464.0):  # above 464, e4m3 rounds to NaN
                p = np.exp2(S - m)
                O[rows, h] = (e4m3(p) @ vh) * v_ds / p.sum(axis=1)[:, None]
                L[h, rows] = math.log(2.0) * (m[:, 0] + np.log2(p.sum(axis=1)))
                continue
            n = S.shape[0]
            m_run = np.full((n, 1), -np.inf)
            acc = np.zeros((n, d))
            lsum = np.zeros((n, 1))
            for j0 in range(0, T, tile):
                St = S[:, j0:j0 + tile]
                m_new = np.maximum(m_run, St.max(axis=1, keepdims=True))
                alpha = np.exp2(m_run - m_new)
                p = np.exp2(St - m_new)
                acc = acc * alpha + e4m3(p) @ vh[j0:j0 + tile]
                lsum = lsum * alpha + p.sum(axis=1, keepdims=True)
                m_run = m_new
            O[rows, h] = acc * v_ds / lsum
            L[h, rows] = math.log(2.0) * (m_run[:, 0] + np.log2(lsum[:, 0]))
    return O, L
