"""Error bars derived from number formats: a first-order model of how the
roundings a format imposes move the attention output.

Test infrastructure (not the oracle, and it shares nothing with the HIP path).
It is written from the definition of attention ("Attention from Scratch",
section "Attention, the math": scores, softmax over keys, weighted sum of V)
and from the formats alone: it knows which values a path rounds and to what
type, not how the path tiles or orders its work.

Model. Scores are in log2 units, s_ij = qs_i . kt_j with qs = rotated q times
scale * log2(e) and kt = rotated k, so p_ij = 2^(s_ij - m_i) and
P_ij = p_ij / sum_j p_ij. A path that rounds qs, kt and p to some formats
replaces each value x by x + e, the e independent with mean 0 and variance
(u^2 x^2 + a^2) / 3 -- the variance of a rounding error spread uniformly over
+-(u |x| + a), with u the format's unit round-off and a half the spacing of
its subnormals. The p are taken against the exact row max (p <= 1): a path
whose reference is below the row max has larger p and so no larger
subnormal error. To first order:

  dO_i = ln2 sum_j P_ij (v_j - O_i) ds_ij + sum_j dp_ij w_ij / l_i,
  ds_ij = sum_k (dqs_ik kt_jk + qs_ik dkt_jk),
  dlse_i = ln2 sum_j P_ij ds_ij + sum_j dp_ij / l_i,

with w_ij = v_j - O_i when the row sum adds the rounded p and w_ij = v_j when
it adds the unrounded ones (the larger variance of the two is taken, so the
bar does not depend on that choice). The variance of each output element
follows by summing the independent terms; the q term keeps its correlation
across keys:
  Var(dO_id) = ln2^2 [ sum_k Var(dqs_ik) A_ikd^2
                       + sum_j P_ij^2 (v_jd - O_id)^2 sum_k qs_ik^2 Var(dkt_jk) ]
               + sum_j Var(dp_ij) w_ijd^2 / l_i^2,
  A_ikd = sum_j P_ij (v_jd - O_id) kt_jk.

A bar built from it is Z standard deviations per element plus the rounding of
the output itself (see ``bar``). ``tests/test_error_bounds.py`` pins the model
to Monte Carlo runs of random roundings of exactly this kind.
"""

from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)

# Unit round-off and half the subnormal spacing of the formats the paths use.
F16 = dict(u=2.0 ** -11, a=2.0 ** -25)
BF16 = dict(u=2.0 ** -9, a=2.0 ** -134)
E4M3 = dict(u=2.0 ** -4, a=2.0 ** -10)


def attention_sigma(qs, kt, v, visible, *, qfmt, kfmt, pfmt, a_q=None, a_k=None, rows=None, psum="max"):
    """One sequence and head: qs [L, d] (log2 units), kt [L, d], v [L, d] float64,
    visible [L, L] bool (every row sees at least one key).

    qfmt/kfmt/pfmt: dicts with u (unit round-off) and a (half the subnormal
    spacing, in the rounded value's own units); a_q / a_k override the
    absolute floor of qs / kt in their units (for paths that scale an operand
    before rounding it). rows: optional row indices (all rows if None).
    psum: "rounded" / "unrounded" (the row sum adds the rounded / the exact p)
    or "max" (the larger variance of the two, per element).

    Returns (O [n, d], lse [n] natural log, sigma_O [n, d], sigma_lse [n]).
    """
    qs, kt, v = (np.asarray(x, np.float64) for x in (qs, kt, v))
    rows = np.arange(qs.shape[0]) if rows is None else np.asarray(rows)
    q = qs[rows]
    S = q @ kt.T
    S[~visible[rows]] = -np.inf
    m = S.max(axis=1)
    p = np.exp2(S - m[:, None])
    l = p.sum(axis=1)
    P = p / l[:, None]
    O = P @ v
    lse = LN2 * (m + np.log2(l))

    aq = qfmt["a"] if a_q is None else a_q
    ak = kfmt["a"] if a_k is None else a_k
    Vq = (qfmt["u"] ** 2 * q ** 2 + aq ** 2) / 3.0          # [n, d]
    Vk = (kfmt["u"] ** 2 * kt ** 2 + ak ** 2) / 3.0         # [L, d]
    Vp = np.where(visible[rows], (pfmt["u"] ** 2 * p ** 2 + pfmt["a"] ** 2) / 3.0, 0.0)  # [n, L]

    # Query-operand term: A_ikd = sum_j P_ij kt_jk v_jd - O_id (P kt)_ik.
    Pk = P @ kt                                               # [n, d]
    term_q = np.empty_like(O)
    for r in range(q.shape[0]):
        A = kt.T @ (P[r][:, None] * v) - np.outer(Pk[r], O[r])   # [d, d]: A_r,k,d
        term_q[r] = Vq[r] @ (A ** 2)
    # Key-operand term: sum_j P_ij^2 W_ij (v_jd - O_id)^2, W_ij = sum_k qs_ik^2 Var(dkt_jk).
    PW = P ** 2 * ((q ** 2) @ Vk.T)
    term_k = PW @ (v ** 2) - 2.0 * O * (PW @ v) + O ** 2 * PW.sum(axis=1)[:, None]
    var_o = LN2 ** 2 * (term_q + term_k)
    # Probability term: the larger of the two row-sum forms.
    Vl = Vp / l[:, None] ** 2
    centred = Vl @ (v ** 2) - 2.0 * O * (Vl @ v) + O ** 2 * Vl.sum(axis=1)[:, None]
    plain = Vl @ (v ** 2)
    var_o = var_o + {"rounded": centred, "unrounded": plain}.get(psum, np.maximum(centred, plain))

    var_l = LN2 ** 2 * (np.einsum("ik,ik->i", Vq, Pk ** 2) + (P ** 2 * ((q ** 2) @ Vk.T)).sum(axis=1))
    if psum != "unrounded":
        var_l = var_l + Vl.sum(axis=1)
    return O, lse, np.sqrt(np.maximum(var_o, 0.0)), np.sqrt(np.maximum(var_l, 0.0))


def bar(sigma, ref, *, z, out_u, slack):
    """Per-element bar: z standard deviations, plus the output's own rounding
    (out_u |ref|, out_u the output format's unit round-off) and an absolute
    slack for what the first-order model leaves out (f32 accumulation)."""
    return z * sigma + out_u * np.abs(ref) + slack


def check_within(name, got, ref, b):
    """Every element within its bar; returns the largest ratio |got - ref| / bar."""
    got, ref, b = (np.asarray(x, np.float64) for x in (got, ref, b))
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    r = np.abs(got - ref) / b
    worst = float(r.max()) if r.size else 0.0
    msg = f"{name}: largest error / bar {worst:.3f} (max abs {float(np.abs(got - ref).max()):.3e})"
    print(msg, flush=True)
    assert worst <= 1.0, msg
    return worst
