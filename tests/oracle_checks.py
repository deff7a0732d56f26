"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each ``check_*`` raises AssertionError when the oracle disagrees with an
independent statement of the same fact: a closed form, an invariant, a
special case that reduces to a library routine, or brute force on tiny inputs.
``test_oracle_pins.py`` runs every check on the oracle as it is, and runs them
again on copies of the oracle with a planted mistake to show that each
plausible mistake fails at least one check.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle

RNG = np.random.default_rng


# ----------------------------------------------------------------------------- RoPE

def check_inv_freq_closed_forms():
    # i = 0 never rotates slower than one radian per position, whatever the base.
    for base in (10000.0, 500000.0, 1e6):
        for d in (2, 8, 64, 128):
            assert oracle.rope_inv_freq(d, base)[0] == 1.0
    # i = d/4 sits halfway through the exponent range: base^(-1/2).
    assert abs(oracle.rope_inv_freq(64, 10000.0)[16] - 0.01) < 1e-15
    assert abs(oracle.rope_inv_freq(128, 1e6)[32] - 0.001) < 1e-16
    # The last pair's frequency is base^(-(d-2)/d): for d = 4, base^(-1/2).
    assert abs(oracle.rope_inv_freq(4, 10000.0)[1] - 0.01) < 1e-15
    f = oracle.rope_inv_freq(128, 500000.0)
    assert f.shape == (64,) and np.all(np.diff(f) < 0), "angle must shrink with feature index"


def check_tables_closed_forms():
    cos, sin = oracle.rope_tables(301, 64, 10000.0)
    assert cos.shape == (301, 32) and sin.shape == (301, 32)
    # Position 0: no rotation at all.
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    # i = 0 turns one radian per position; i = d/4 turns 0.01 rad per position.
    assert abs(cos[300, 0] - math.cos(300.0)) < 1e-12 and abs(sin[300, 0] - math.sin(300.0)) < 1e-12
    assert abs(cos[100, 16] - math.cos(1.0)) < 1e-13 and abs(sin[100, 16] - math.sin(1.0)) < 1e-13
    assert abs(cos[157, 16] - math.cos(1.57)) < 1e-13


def check_rope_d2_is_plane_rotation():
    # With d = 2 both pairings are the single pair (0, 1) and inv_freq = 1, so the
    # rotation at position p is the textbook 2x2 rotation matrix by p radians.
    x = RNG(1).standard_normal((7, 3, 2))
    pos = np.arange(7) * 3 + 1
    for style in ("interleaved", "half"):
        y = oracle.apply_rope(x, pos, 10000.0, style)
        for t, p in enumerate(pos):
            R = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
            assert np.allclose(y[t], x[t] @ R.T, atol=1e-13, rtol=0)


def check_rope_interleaved_complex_form():
    # Interleaved RoPE is multiplication of z_i = x[2i] + 1j*x[2i+1] by exp(1j*p*f_i).
    d, T = 16, 9
    x = RNG(2).standard_normal((T, 2, d))
    pos = np.arange(T) * 37
    f = 10000.0 ** (-np.arange(0, d, 2) / d)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = z * np.exp(1j * np.outer(pos, f))[:, None, :]
    y = oracle.apply_rope(x, pos, 10000.0, "interleaved")
    assert np.allclose(y[..., 0::2], w.real, atol=1e-12, rtol=0)
    assert np.allclose(y[..., 1::2], w.imag, atol=1e-12, rtol=0)


def check_rope_half_matches_rotate_half_form():
    # The printed helper: duplicate the half-width angle table to full width and
    # compute x*cos + rotate_half(x)*sin with rotate_half(x) = (-x2, x1).
    d, T = 12, 11
    x = RNG(3).standard_normal((T, 3, d))
    pos = np.arange(T)
    f = 500000.0 ** (-np.arange(0, d, 2) / d)
    ang = np.outer(pos, f)
    full = np.concatenate([ang, ang], axis=-1)[:, None, :]
    rot_half = np.concatenate([-x[..., d // 2:], x[..., : d // 2]], axis=-1)
    want = x * np.cos(full) + rot_half * np.sin(full)
    got = oracle.apply_rope(x, pos, 500000.0, "half")
    assert np.allclose(got, want, atol=1e-12, rtol=0)


def check_rope_norm_and_identity():
    d = 64
    x = RNG(4).standard_normal((300, 2, d))
    pos = np.arange(300)
    for style, (ia, ib) in (("interleaved", (np.arange(0, d, 2), np.arange(1, d, 2))),
                            ("half", (np.arange(d // 2), np.arange(d // 2, d)))):
        y = oracle.apply_rope(x, pos, 10000.0, style)
        n0 = x[..., ia] ** 2 + x[..., ib] ** 2
        n1 = y[..., ia] ** 2 + y[..., ib] ** 2
        assert np.allclose(n0, n1, atol=1e-12, rtol=1e-12), "each pair keeps its length"
        assert np.array_equal(y[0], x[0]), "position 0 is the identity"
        assert not np.allclose(y[5], x[5]), "later positions rotate"


def check_rope_relative():
    # (R(m) q) . (R(n) k) depends only on n - m.
    d = 32
    rng = RNG(5)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for style in ("interleaved", "half"):
        def dot(m, n):
            qr = oracle.apply_rope(q[None, :], [m], 10000.0, style)[0]
            kr = oracle.apply_rope(k[None, :], [n], 10000.0, style)[0]
            return float(qr @ kr)
        for (m, n, c) in ((3, 10, 100), (0, 0, 4000), (77, 5, 8191), (1000, 999, 17)):
            assert abs(dot(m, n) - dot(m + c, n + c)) < 1e-9
            # and equals q . R(n - m) k
            kr = oracle.apply_rope(k[None, :], [n - m], 10000.0, style)[0]
            assert abs(dot(m, n) - float(q @ kr)) < 1e-9


def deinterleave(x):
    """Permute the last dim so interleaved pair i (2i, 2i+1) lands on (i, i + d/2)."""
    return np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1)


def check_rope_styles_related_by_permutation():
    rng = RNG(6)
    q = rng.standard_normal((2, 20, 4, 16))
    k = rng.standard_normal((2, 20, 2, 16))
    v = rng.standard_normal((2, 20, 2, 16))
    o_int, l_int = oracle.attention_dense(q, k, v, base=10000.0, style="interleaved")
    o_half, l_half = oracle.attention_dense(deinterleave(q), deinterleave(k), v, base=10000.0,
                                            style="half")
    assert np.allclose(o_int, o_half, atol=1e-12) and np.allclose(l_int, l_half, atol=1e-12)
    o_bad, _ = oracle.attention_dense(q, k, v, base=10000.0, style="half")
    assert not np.allclose(o_int, o_bad, atol=1e-3), "the pairing must matter"


# ------------------------------------------------------------------------ attention

def brute_force(q, k, v, causal, base, style, scale=None, window=0):
    """Scalar loops over Python floats: rotate, share, score, mask, softmax, gather.

    Follows the six steps of "Attention from Scratch", section "Attention, the
    math", for one batch entry at a time, with no vectorisation and no
    max-shift (the inputs are small enough that exp cannot overflow).
    q [B][T][H][d], k/v [B][T][KV][d] nested lists.
    """
    B, T, H, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    KV = len(k[0][0])
    G = H // KV
    sc = 1.0 / math.sqrt(d) if scale is None else scale

    def rot(x, p):
        y = list(x)
        for i in range(d // 2):
            ang = p * base ** (-(2.0 * i) / d)
            a, b = (2 * i, 2 * i + 1) if style == "interleaved" else (i, i + d // 2)
            y[a] = x[a] * math.cos(ang) - x[b] * math.sin(ang)
            y[b] = x[a] * math.sin(ang) + x[b] * math.cos(ang)
        return y

    O = [[[[0.0] * d for _ in range(H)] for _ in range(T)] for _ in range(B)]
    L = [[[0.0] * T for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(T):
                qi = rot(q[b][i][h], i)
                w = []
                for j in range(T):
                    if (causal and j > i) or (window > 0 and i - j >= window):
                        w.append(0.0)
                        continue
                    kj = rot(k[b][j][g], j)
                    w.append(math.exp(sc * sum(qi[c] * kj[c] for c in range(d))))
                z = sum(w)
                L[b][h][i] = math.log(z)
                for c in range(d):
                    O[b][i][h][c] = sum(w[j] * v[b][j][g][c] for j in range(T)) / z
    return np.array(O), np.array(L)


def check_brute_force():
    rng = RNG(7)
    for (B, T, H, KV, d, causal, style, base) in (
            (2, 9, 4, 2, 8, True, "interleaved", 10000.0),
            (1, 12, 4, 2, 8, False, "interleaved", 500000.0),
            (1, 10, 3, 1, 6, True, "half", 1e6),
            (2, 7, 2, 2, 4, False, "half", 10000.0)):
        q = rng.standard_normal((B, T, H, d))
        k = rng.standard_normal((B, T, KV, d))
        v = rng.standard_normal((B, T, KV, d))
        o_ref, l_ref = brute_force(q.tolist(), k.tolist(), v.tolist(), causal, base, style)
        o, lse = oracle.attention_dense(q, k, v, causal=causal, base=base, style=style)
        assert np.allclose(o, o_ref, atol=1e-12, rtol=0), (B, T, H, KV, d, causal, style)
        assert np.allclose(lse, l_ref, atol=1e-12, rtol=0)


def check_library_sdpa():
    # After rotation, the rest is scaled-dot-product attention: cross-check the
    # score/mask/softmax/gather part against torch's float64 CPU routine (GQA
    # sharing through enable_gqa), and the log-sum-exp against scipy's.
    from scipy.special import logsumexp
    rng = RNG(8)
    B, T, H, KV, d = 2, 33, 6, 2, 16
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, KV, d))
    v = rng.standard_normal((B, T, KV, d))
    for causal in (True, False):
        o, lse = oracle.attention_dense(q, k, v, causal=causal, base=10000.0)
        pos = np.arange(T)
        qr = np.stack([oracle.apply_rope(q[b], pos, 10000.0) for b in range(B)])
        kr = np.stack([oracle.apply_rope(k[b], pos, 10000.0) for b in range(B)])
        tq = torch.from_numpy(qr).permute(0, 2, 1, 3)
        tk = torch.from_numpy(kr).permute(0, 2, 1, 3)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, enable_gqa=True).permute(0, 2, 1, 3).numpy()
        assert np.allclose(o, ref, atol=1e-12, rtol=0)
        for b in range(B):
            for h in range(H):
                S = qr[b, :, h] @ kr[b, :, h // (H // KV)].T / math.sqrt(d)
                if causal:
                    S = np.where(np.tril(np.ones((T, T), bool)), S, -np.inf)
                assert np.allclose(lse[b, h], logsumexp(S, axis=1), atol=1e-12, rtol=0)


def check_softmax_rows():
    # With V[j] = e_j (d >= T) the output rows are the softmax weights themselves:
    # rows sum to one, nothing above the diagonal, and P = exp(S - lse).
    T, d = 16, 16
    rng = RNG(9)
    q = rng.standard_normal((1, T, 2, d))
    k = rng.standard_normal((1, T, 1, d))
    v = np.eye(T, d)[None, :, None, :]
    for causal in (True, False):
        o, lse = oracle.attention_dense(q, k, v, causal=causal, base=10000.0)
        P = o[0]  # [T, H, d]
        assert np.allclose(P.sum(axis=-1), 1.0, atol=1e-14)
        if causal:
            assert np.all(P[np.triu_indices(T, 1)[0], :, np.triu_indices(T, 1)[1]] == 0.0)
        pos = np.arange(T)
        qr = oracle.apply_rope(q[0], pos, 10000.0)
        kr = oracle.apply_rope(k[0], pos, 10000.0)
        for h in range(2):
            S = qr[:, h] @ kr[:, 0].T / math.sqrt(d)
            want = np.exp(S - lse[0, h][:, None])
            if causal:
                want = np.tril(want)
            assert np.allclose(P[:, h, :], want, atol=1e-14)


def check_causal_row0():
    rng = RNG(10)
    q = rng.standard_normal((3, 25, 8, 32))
    k = rng.standard_normal((3, 25, 2, 32))
    v = rng.standard_normal((3, 25, 2, 32))
    o, lse = oracle.attention_dense(q, k, v, causal=True, base=500000.0)
    for h in range(8):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // 4]), "row 0 sees only key 0 of its KV head"
        want = np.einsum("bd,bd->b", q[:, 0, h], k[:, 0, h // 4]) / math.sqrt(32)
        assert np.allclose(lse[:, h, 0], want, atol=1e-13, rtol=0)


def check_gqa_is_mha_with_repeat_interleave():
    rng = RNG(11)
    G = 3
    q = rng.standard_normal((2, 19, 6, 8))
    k = rng.standard_normal((2, 19, 2, 8))
    v = rng.standard_normal((2, 19, 2, 8))
    o, lse = oracle.attention_dense(q, k, v, base=10000.0)
    o2, l2 = oracle.attention_dense(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2),
                                    base=10000.0)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def check_zero_query_closed_form():
    # q = 0: every allowed score is 0, so row i averages the values it may see
    # and its log-sum-exp is ln(#allowed keys), whatever the rotation.
    rng = RNG(12)
    T = 40
    k = rng.standard_normal((1, T, 2, 16))
    v = rng.standard_normal((1, T, 2, 16))
    q = np.zeros((1, T, 4, 16))
    o, lse = oracle.attention_dense(q, k, v, causal=True, base=10000.0)
    for h in range(4):
        cm = np.cumsum(v[0, :, h // 2], axis=0) / np.arange(1, T + 1)[:, None]
        assert np.allclose(o[0, :, h], cm, atol=1e-14)
        assert np.allclose(lse[0, h], np.log(np.arange(1, T + 1)), atol=1e-14)
    o, lse = oracle.attention_dense(q, k, v, causal=False, base=10000.0)
    assert np.allclose(o[0, :, 3], np.broadcast_to(v[0, :, 1].mean(axis=0), (T, 16)), atol=1e-14)
    assert np.allclose(lse, math.log(T), atol=1e-14)


def check_single_token():
    rng = RNG(13)
    q = rng.standard_normal((4, 1, 2, 8))
    k = rng.standard_normal((4, 1, 1, 8))
    v = rng.standard_normal((4, 1, 1, 8))
    for causal in (True, False):
        o, lse = oracle.attention_dense(q, k, v, causal=causal, base=10000.0, scale=0.25)
        assert np.array_equal(o[:, 0, 0], v[:, 0, 0]) and np.array_equal(o[:, 0, 1], v[:, 0, 0])
        assert np.allclose(lse[:, 1, 0], 0.25 * np.einsum("bd,bd->b", q[:, 0, 1], k[:, 0, 0]),
                           atol=1e-14)


def check_scale_argument():
    rng = RNG(14)
    q = rng.standard_normal((1, 12, 2, 16))
    k = rng.standard_normal((1, 12, 2, 16))
    v = rng.standard_normal((1, 12, 2, 16))
    a = oracle.attention_dense(q, k, v, base=10000.0)
    b = oracle.attention_dense(q, k, v, base=10000.0, scale=0.25)
    assert np.allclose(a[0], b[0], atol=1e-14) and np.allclose(a[1], b[1], atol=1e-14)
    c = oracle.attention_dense(q, k, v, base=10000.0, scale=0.7)
    d = oracle.attention_dense(q * 0.7 * 4.0, k, v, base=10000.0)
    assert np.allclose(c[0], d[0], atol=1e-12) and np.allclose(c[1], d[1], atol=1e-12)


def check_varlen_is_concat_of_dense():
    rng = RNG(15)
    lengths = [5, 1, 0, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((total, 4, 8))
    k = rng.standard_normal((total, 1, 8))
    v = rng.standard_normal((total, 1, 8))
    for causal in (True, False):
        o, lse = oracle.attention_varlen(q, k, v, cu, causal=causal, base=10000.0, style="half")
        for s, L in enumerate(lengths):
            a = int(cu[s])
            if L == 0:
                continue
            od, ld = oracle.attention_dense(q[None, a:a + L], k[None, a:a + L], v[None, a:a + L],
                                            causal=causal, base=10000.0, style="half")
            assert np.array_equal(o[a:a + L], od[0]) and np.array_equal(lse[:, a:a + L], ld[0])
        # One brute-force sequence pins the packed indexing directly.
        a, L = int(cu[3]), lengths[3]
        ob, lb = brute_force(q[None, a:a + L].tolist(), k[None, a:a + L].tolist(),
                             v[None, a:a + L].tolist(), causal, 10000.0, "half")
        assert np.allclose(o[a:a + L], ob[0], atol=1e-12) and np.allclose(lse[:, a:a + L], lb[0],
                                                                          atol=1e-12)


def check_rows_match_full():
    rng = RNG(16)
    q = rng.standard_normal((2, 30, 4, 16))
    k = rng.standard_normal((2, 30, 2, 16))
    v = rng.standard_normal((2, 30, 2, 16))
    rows = [(0, 0, 0), (1, 29, 3), (0, 17, 2), (1, 5, 1)]
    for causal in (True, False):
        o, lse = oracle.attention_dense(q, k, v, causal=causal, base=10000.0)
        ro, rl = oracle.attention_rows(q, k, v, rows, causal=causal, base=10000.0)
        for n, (b, t, h) in enumerate(rows):
            assert np.allclose(ro[n], o[b, t, h], atol=1e-13) and abs(rl[n] - lse[b, h, t]) < 1e-13
    lengths = [3, 11, 6]
    cu = np.array([0, 3, 14, 20], dtype=np.int32)
    q2, k2, v2 = q[0, :20], k[0, :20], v[0, :20]
    o, lse = oracle.attention_varlen(q2, k2, v2, cu, base=10000.0)
    rows = [(0, 2, 1), (1, 10, 0), (2, 0, 3), (1, 4, 2)]
    ro, rl = oracle.attention_rows(q2, k2, v2, rows, base=10000.0, cu_seqlens=cu)
    for n, (s, t, h) in enumerate(rows):
        tok = int(cu[s]) + t
        assert np.allclose(ro[n], o[tok, h], atol=1e-13) and abs(rl[n] - lse[h, tok]) < 1e-13
    assert lengths == [3, 11, 6]


# ------------------------------------------------------------------------ backward
#
# The gradients are pinned to finite differences of the (already pinned) forward,
# to torch's float64 autograd through its own scaled-dot-product attention, and to
# identities that any correct gradient of this function satisfies.

def check_rope_transpose_inverts_rotation():
    # R(p) is orthogonal: its transpose undoes it, and <R x, y> = <x, R^T y>.
    rng = RNG(30)
    pos = np.array([0, 1, 7, 300, 4095])
    for style in ("interleaved", "half"):
        for d in (2, 8, 64):
            x = rng.standard_normal((5, 3, d))
            y = rng.standard_normal((5, 3, d))
            rx = oracle.apply_rope(x, pos, 10000.0, style)
            assert np.allclose(oracle.apply_rope_transpose(rx, pos, 10000.0, style), x, atol=1e-12)
            lhs = np.sum(rx * y)
            rhs = np.sum(x * oracle.apply_rope_transpose(y, pos, 10000.0, style))
            assert abs(lhs - rhs) < 1e-11


def check_bwd_finite_differences():
    # Central differences of L = sum(O * W) with respect to every entry of q, k, v.
    rng = RNG(31)
    B, T, H, KV, d = 1, 6, 4, 2, 4
    eps = 1e-5
    for causal, style, base in ((True, "interleaved", 10000.0), (False, "interleaved", 500000.0),
                                (True, "half", 10000.0), (False, "half", 1e6)):
        q = rng.standard_normal((B, T, H, d))
        k = rng.standard_normal((B, T, KV, d))
        v = rng.standard_normal((B, T, KV, d))
        W = rng.standard_normal((B, T, H, d))

        def loss(q_, k_, v_):
            o, _ = oracle.attention_dense(q_, k_, v_, causal=causal, base=base, style=style)
            return float(np.sum(o * W))

        dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=causal, base=base, style=style)
        for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[which]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[which]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(fd - g[idx]) < 1e-7, (which, idx, causal, style, fd, g[idx])


def check_bwd_torch_autograd():
    # torch's float64 autograd through a rotation written as a complex product
    # (pair (a, b) is the complex number a + ib, turned by e^{i angle}) and
    # torch's scaled_dot_product_attention with GQA sharing.
    rng = RNG(32)
    B, T, H, KV, d = 2, 23, 6, 2, 16
    for causal, style, base in ((True, "interleaved", 10000.0), (False, "half", 500000.0)):
        q = rng.standard_normal((B, T, H, d))
        k = rng.standard_normal((B, T, KV, d))
        v = rng.standard_normal((B, T, KV, d))
        W = rng.standard_normal((B, T, H, d))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        ang = torch.outer(torch.arange(T, dtype=torch.float64),
                          base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d))
        turn = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

        def rot(x):
            if style == "interleaved":
                z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
                return torch.view_as_real(z * turn).reshape(x.shape)
            z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * turn
            return torch.cat([z.real, z.imag], dim=-1)

        o = torch.nn.functional.scaled_dot_product_attention(
            rot(tq).transpose(1, 2), rot(tk).transpose(1, 2), tv.transpose(1, 2),
            is_causal=causal, enable_gqa=True).transpose(1, 2)
        (o * torch.from_numpy(W)).sum().backward()
        dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=causal, base=base, style=style)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


def check_bwd_gqa_is_mha_summed():
    # A K/V head shared by G query heads gets the sum of the gradients that G
    # private copies of it would get; dq does not change.
    rng = RNG(33)
    G = 3
    q = rng.standard_normal((2, 15, 6, 8))
    k = rng.standard_normal((2, 15, 2, 8))
    v = rng.standard_normal((2, 15, 2, 8))
    W = rng.standard_normal((2, 15, 6, 8))
    dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W)
    dq2, dk2, dv2 = oracle.attention_dense_bwd(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), W)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(2, 15, 2, G, 8).sum(axis=3), atol=1e-13)
    assert np.allclose(dv, dv2.reshape(2, 15, 2, G, 8).sum(axis=3), atol=1e-13)


def check_bwd_invariants():
    rng = RNG(34)
    B, T, H, KV, d = 2, 21, 4, 2, 8
    G = H // KV
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, KV, d))
    v = rng.standard_normal((B, T, KV, d))
    W = rng.standard_normal((B, T, H, d))
    for causal in (True, False):
        dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=causal)
        for g in range(KV):
            hs = slice(g * G, (g + 1) * G)
            # O(q * c, k / c) = O(q, k): the derivative in c at c = 1 is
            # <dq, q> - <dk, k> = 0, per K/V group and per sequence.
            for b in range(B):
                assert abs(np.sum(dq[b, :, hs] * q[b, :, hs]) - np.sum(dk[b, :, g] * k[b, :, g])) < 1e-11
            # Every output row is a convex combination of value rows, so adding a
            # constant vector to every value row adds it to every output row:
            # sum over tokens of dv = sum over tokens and the group's heads of dO.
            assert np.allclose(dv[:, :, g].sum(axis=1), W[:, :, hs].sum(axis=(1, 2)), atol=1e-12)


def check_bwd_closed_forms():
    rng = RNG(35)
    T = 30
    k = rng.standard_normal((1, T, 2, 16))
    v = rng.standard_normal((1, T, 2, 16))
    W = rng.standard_normal((1, T, 4, 16))
    # q = 0: all allowed scores are 0, so P is uniform over the allowed keys.
    # Then dk = 0 (every dS_ij multiplies a zero query), and key j of group g
    # receives sum over i >= j and the group's heads of dO_i / (i + 1).
    q = np.zeros((1, T, 4, 16))
    dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=True)
    assert np.array_equal(dk, np.zeros_like(dk))
    for g in range(2):
        w = W[0, :, 2 * g:2 * g + 2].sum(axis=1) / np.arange(1, T + 1)[:, None]
        expect = np.cumsum(w[::-1], axis=0)[::-1]
        assert np.allclose(dv[0, :, g], expect, atol=1e-13)
    # Without the mask and q = 0, every key gets the mean of the group's dO.
    dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=False)
    assert np.allclose(dv[0, :, 1], np.broadcast_to(W[0, :, 2:].sum(axis=1).mean(axis=0), (T, 16)),
                       atol=1e-13)
    # Row 0 under the mask sees only key 0: P = 1, so dS = 0 and query 0 gets no gradient.
    q = rng.standard_normal((1, T, 4, 16))
    dq, _, _ = oracle.attention_dense_bwd(q, k, v, W, causal=True)
    assert np.all(dq[0, 0] == 0.0)
    # One token: O = v, so dq = dk = 0 and dv is the sum of the group's dO.
    q1, k1, v1, W1 = q[:, :1], k[:, :1], v[:, :1], W[:, :1]
    for causal in (True, False):
        dq, dk, dv = oracle.attention_dense_bwd(q1, k1, v1, W1, causal=causal)
        assert np.all(dq == 0.0) and np.all(dk == 0.0)
        assert np.allclose(dv[0, 0], W1[0, 0].reshape(2, 2, 16).sum(axis=1), atol=1e-15)


def check_bwd_varlen_is_concat_of_dense():
    rng = RNG(36)
    lengths = [5, 1, 0, 13, 8]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((total, 4, 8))
    k = rng.standard_normal((total, 2, 8))
    v = rng.standard_normal((total, 2, 8))
    W = rng.standard_normal((total, 4, 8))
    for causal, style in ((True, "interleaved"), (False, "half")):
        dq, dk, dv = oracle.attention_varlen_bwd(q, k, v, W, cu, causal=causal, style=style)
        for s, L in enumerate(lengths):
            a = int(cu[s])
            if L == 0:
                continue
            r = oracle.attention_dense_bwd(q[None, a:a + L], k[None, a:a + L], v[None, a:a + L],
                                           W[None, a:a + L], causal=causal, style=style)
            assert np.array_equal(dq[a:a + L], r[0][0]) and np.array_equal(dk[a:a + L], r[1][0])
            assert np.array_equal(dv[a:a + L], r[2][0])


def check_bwd_group_matches_full():
    # The blocked one-group backward is the full backward restricted to that group.
    rng = RNG(37)
    q = rng.standard_normal((2, 45, 6, 8))
    k = rng.standard_normal((2, 45, 2, 8))
    v = rng.standard_normal((2, 45, 2, 8))
    W = rng.standard_normal((2, 45, 6, 8))
    for causal, style in ((True, "interleaved"), (False, "half")):
        dq, dk, dv = oracle.attention_dense_bwd(q, k, v, W, causal=causal, style=style)
        for b, kv in ((0, 1), (1, 0)):
            gq, gk, gv = oracle.attention_bwd_group(q, k, v, W, b, kv, causal=causal, style=style,
                                                    rows_per_block=16)
            assert np.allclose(gq, dq[b, :, 3 * kv:3 * kv + 3], atol=1e-12)
            assert np.allclose(gk, dk[b, :, kv], atol=1e-12) and np.allclose(gv, dv[b, :, kv], atol=1e-12)


# -------------------------------------------------------------------------- decode

def check_decode_is_the_end_of_the_causal_forward():
    # The Tq new queries of a sequence of length L are rows L-Tq .. L-1 of the
    # causal forward over its first L tokens, whatever sits in the query rows
    # before them and in the cache rows past L.
    rng = RNG(40)
    B, S, H, KV, d, Tq = 3, 40, 6, 2, 8, 3
    lens = [3, 17, 40]
    q = rng.standard_normal((B, Tq, H, d))
    k = rng.standard_normal((B, S, KV, d))
    v = rng.standard_normal((B, S, KV, d))
    for style, base in (("interleaved", 10000.0), ("half", 500000.0)):
        o, lse = oracle.attention_decode(q, k, v, lens, base=base, style=style)
        for b, L in enumerate(lens):
            qf = rng.standard_normal((1, L, H, d))
            qf[0, L - Tq:] = q[b]
            of, lf = oracle.attention_dense(qf, k[None, b, :L], v[None, b, :L], causal=True, base=base,
                                            style=style)
            assert np.allclose(o[b], of[0, L - Tq:], atol=1e-12)
            assert np.allclose(lse[b], lf[0, :, L - Tq:], atol=1e-12)
    # brute force on one entry
    ob, lb = brute_force(np.concatenate([np.zeros((1, lens[1] - Tq, H, d)), q[1:2]], axis=1).tolist(),
                         k[1:2, :lens[1]].tolist(), v[1:2, :lens[1]].tolist(), True, 10000.0, "interleaved")
    o, lse = oracle.attention_decode(q, k, v, lens, base=10000.0)
    assert np.allclose(o[1], ob[0, lens[1] - Tq:], atol=1e-12) and np.allclose(lse[1], lb[0, :, lens[1] - Tq:], atol=1e-12)


def check_decode_special_cases():
    rng = RNG(41)
    B, S, H, KV, d = 2, 16, 4, 1, 8
    q = rng.standard_normal((B, 1, H, d))
    k = rng.standard_normal((B, S, KV, d))
    v = rng.standard_normal((B, S, KV, d))
    # A cache of one token: every head returns that token's value, lse = its score.
    o, lse = oracle.attention_decode(q, k, v, [1, 1])
    assert np.array_equal(o[:, 0, 2], v[:, 0, 0])
    assert np.allclose(lse[:, 3, 0], np.einsum("bd,bd->b", q[:, 0, 3], k[:, 0, 0]) / math.sqrt(d), atol=1e-14)
    # Cache rows past the length do not matter.
    k2, v2 = k.copy(), v.copy()
    k2[:, 9:] = 1e3
    v2[:, 9:] = np.nan
    a = oracle.attention_decode(q, k, v, [9, 5])
    b = oracle.attention_decode(q, k2, v2, [9, 5])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # Tq = L is the whole causal forward.
    q3 = rng.standard_normal((1, 12, H, d))
    o3, l3 = oracle.attention_decode(q3, k[:1], v[:1], [12])
    od, ld = oracle.attention_dense(q3, k[:1, :12], v[:1, :12], causal=True)
    assert np.allclose(o3, od, atol=1e-13) and np.allclose(l3, ld, atol=1e-13)
    # q = 0: the one new query averages every cached value.
    o4, l4 = oracle.attention_decode(np.zeros((B, 1, H, d)), k, v, [16, 7])
    assert np.allclose(o4[1, 0, 0], v[1, :7, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(l4[1], math.log(7), atol=1e-14)


# ------------------------------------------------------------------ sliding window

def check_window_is_causal_attention_on_a_slice():
    # With a window W, row i sees keys i-W+1 .. i. RoPE scores depend on i - j
    # only, so row i equals the last row of plain causal attention over the
    # tokens i-W+1 .. i with positions restarting at 0.
    rng = RNG(50)
    T, H, KV, d = 40, 4, 2, 8
    q = rng.standard_normal((1, T, H, d))
    k = rng.standard_normal((1, T, KV, d))
    v = rng.standard_normal((1, T, KV, d))
    for W, style in ((7, "interleaved"), (16, "half"), (1, "interleaved")):
        o, lse = oracle.attention_dense(q, k, v, causal=True, base=10000.0, style=style, window=W)
        for i in (0, 3, W - 1, W, 25, T - 1):
            if i >= T:
                continue
            a = max(0, i - W + 1)
            os_, ls = oracle.attention_dense(q[:, a:i + 1], k[:, a:i + 1], v[:, a:i + 1], causal=True,
                                             base=10000.0, style=style)
            assert np.allclose(o[0, i], os_[0, -1], atol=1e-9) and np.allclose(lse[0, :, i], ls[0, :, -1], atol=1e-9)


def check_window_special_cases():
    rng = RNG(51)
    T = 24
    q = rng.standard_normal((2, T, 4, 8))
    k = rng.standard_normal((2, T, 1, 8))
    v = rng.standard_normal((2, T, 1, 8))
    a = oracle.attention_dense(q, k, v, causal=True)
    b = oracle.attention_dense(q, k, v, causal=True, window=T)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # W = 1: each row sees itself only.
    o, lse = oracle.attention_dense(q, k, v, causal=True, window=1, base=10000.0)
    assert np.array_equal(o[:, :, 2], v[:, :, 0])
    qr = oracle.apply_rope(q[0, :, 3], np.arange(T), 10000.0)
    kr = oracle.apply_rope(k[0, :, 0], np.arange(T), 10000.0)
    assert np.allclose(lse[0, 3], np.einsum("td,td->t", qr, kr) / math.sqrt(8), atol=1e-12)
    # brute force
    ob, lb = brute_force(q[:1, :12].tolist(), k[:1, :12].tolist(), v[:1, :12].tolist(), True, 500000.0,
                         "half", window=5)
    o5, l5 = oracle.attention_dense(q[:1, :12], k[:1, :12], v[:1, :12], causal=True, base=500000.0,
                                    style="half", window=5)
    assert np.allclose(o5, ob, atol=1e-12) and np.allclose(l5, lb, atol=1e-12)
    # sampled rows, packed batch, decode
    rows = [(0, 0, 0), (1, 23, 3), (0, 9, 1), (1, 4, 2)]
    o9, l9 = oracle.attention_dense(q, k, v, causal=True, window=9)
    ro, rl = oracle.attention_rows(q, k, v, rows, causal=True, window=9)
    for n, (bb, t, h) in enumerate(rows):
        assert np.allclose(ro[n], o9[bb, t, h], atol=1e-13) and abs(rl[n] - l9[bb, h, t]) < 1e-13
    cu = np.array([0, 10, 10, 24], dtype=np.int32)
    ov, lv = oracle.attention_varlen(q[0], k[0], v[0], cu, causal=True, window=4)
    for s0, s1 in ((0, 10), (10, 24)):
        od, ld = oracle.attention_dense(q[None, 0, s0:s1], k[None, 0, s0:s1], v[None, 0, s0:s1], causal=True,
                                        window=4)
        assert np.array_equal(ov[s0:s1], od[0]) and np.array_equal(lv[:, s0:s1], ld[0])
    Tq = 3
    od, ld = oracle.attention_decode(q[:, T - Tq:], k, v, [T, T], window=6)
    ow, lw = oracle.attention_dense(q, k, v, causal=True, window=6)
    assert np.allclose(od, ow[:, T - Tq:], atol=1e-12) and np.allclose(ld, lw[:, :, T - Tq:], atol=1e-12)


def check_window_backward():
    # Finite differences of sum(O * W) through the windowed forward, and the
    # blocked one-group backward against the full one.
    rng = RNG(52)
    B, T, H, KV, d, Wn = 1, 9, 2, 1, 4, 3
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, KV, d))
    v = rng.standard_normal((B, T, KV, d))
    Wt = rng.standard_normal((B, T, H, d))
    eps = 1e-5
    dq, dk, dv = oracle.attention_dense_bwd(q, k, v, Wt, causal=True, window=Wn)
    for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in list(np.ndindex(*x.shape))[::3]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": lambda y: (y, k, v), "k": lambda y: (q, y, v), "v": lambda y: (q, k, y)}[which]
            fp = np.sum(oracle.attention_dense(*args(xp), causal=True, window=Wn)[0] * Wt)
            fm = np.sum(oracle.attention_dense(*args(xm), causal=True, window=Wn)[0] * Wt)
            assert abs((fp - fm) / (2 * eps) - g[idx]) < 1e-7, (which, idx)
    q2 = rng.standard_normal((1, 37, 4, 8))
    k2 = rng.standard_normal((1, 37, 2, 8))
    v2 = rng.standard_normal((1, 37, 2, 8))
    W2 = rng.standard_normal((1, 37, 4, 8))
    fq, fk, fv = oracle.attention_dense_bwd(q2, k2, v2, W2, causal=True, window=10)
    gq, gk, gv = oracle.attention_bwd_group(q2, k2, v2, W2, 0, 1, causal=True, window=10, rows_per_block=8)
    assert np.allclose(gq, fq[0, :, 2:4], atol=1e-12) and np.allclose(gk, fk[0, :, 1], atol=1e-12)
    assert np.allclose(gv, fv[0, :, 1], atol=1e-12)


# ----------------------------------------------------------- RMSNorm + QKV + RoPE

def check_rmsnorm_closed_forms():
    rng = RNG(60)
    x = rng.standard_normal((7, 48)) * 3.0
    # weight 1, eps 0: every row has root-mean-square exactly 1.
    y = oracle.rmsnorm(x, np.ones(48), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    # Scale invariance (eps 0) and the weight as a per-feature factor.
    assert np.allclose(oracle.rmsnorm(5.0 * x, np.ones(48), 0.0), y, atol=1e-13)
    w = rng.standard_normal(48)
    assert np.allclose(oracle.rmsnorm(x, w, 0.0), y * w, atol=1e-13)
    # eps: mean(y^2) = m / (m + eps) for m = mean(x^2).
    m = np.mean(x * x, axis=1)
    ye = oracle.rmsnorm(x, np.ones(48), 0.5)
    assert np.allclose(np.mean(ye * ye, axis=1), m / (m + 0.5), atol=1e-13)
    # A constant row c: x / |c| (eps 0).
    assert np.allclose(oracle.rmsnorm(np.full((1, 8), -3.0), np.ones(8), 0.0), -1.0, atol=1e-15)
    # Against torch's own RMSNorm.
    tn = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-6), tn.numpy(), atol=1e-12)


def check_rmsnorm_qkv_rope_structure():
    rng = RNG(61)
    N, H, KV, d = 9, 4, 2, 8
    C = H * d
    x = rng.standard_normal((N, C))
    pos = rng.integers(0, 100, N)
    # Identity projections (W_q = I, W_k = W_v = the first KV*d rows of I),
    # weight 1, eps 0: q is RoPE of the unit-RMS row itself.
    W = np.concatenate([np.eye(C), np.eye(C)[: KV * d], np.eye(C)[: KV * d]])
    q, k, v = oracle.rmsnorm_qkv_rope(x, np.ones(C), 0.0, W, pos, H, KV, base=10000.0)
    xn = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    assert np.allclose(q, oracle.apply_rope(xn.reshape(N, H, d), pos, 10000.0), atol=1e-13)
    assert np.allclose(v, xn[:, : KV * d].reshape(N, KV, d), atol=1e-14)
    assert np.allclose(k, oracle.apply_rope(xn[:, : KV * d].reshape(N, KV, d), pos, 10000.0), atol=1e-13)
    # Random weights: each output is the normalised row times its slice of W,
    # rotated (or not) as asked; positions 0 leave q, k unrotated.
    W = rng.standard_normal(((H + 2 * KV) * d, 24))
    x2 = rng.standard_normal((N, 24))
    g = rng.standard_normal(24)
    q, k, v = oracle.rmsnorm_qkv_rope(x2, g, 1e-6, W, np.zeros(N, int), H, KV, style="half")
    xn2 = x2 / np.sqrt(np.mean(x2 * x2, axis=1, keepdims=True) + 1e-6) * g
    for n in range(N):
        for h in range(H):
            assert np.allclose(q[n, h], W[h * d:(h + 1) * d] @ xn2[n], atol=1e-12)
        for j in range(KV):
            assert np.allclose(k[n, j], W[(H + j) * d:(H + j + 1) * d] @ xn2[n], atol=1e-12)
            assert np.allclose(v[n, j], W[(H + KV + j) * d:(H + KV + j + 1) * d] @ xn2[n], atol=1e-12)
    q2, k2, _ = oracle.rmsnorm_qkv_rope(x2, g, 1e-6, W, pos, H, KV, style="half", rotate_q=False)
    assert np.allclose(k2, oracle.apply_rope(k, pos, 10000.0, "half"), atol=1e-12)
    assert np.allclose(q2, q, atol=1e-13)


def check_padding_mask():
    """Right-padded dense batches: the valid rows against scalar brute force on
    each entry's prefix and against torch's SDPA with an explicit key mask
    (after float64 RoPE); the padding tokens' values change nothing; padding
    rows are NaN (no output); full lengths give the dense result."""
    import torch
    rng = RNG(67)
    B, T, H, KV, d = 4, 11, 4, 2, 8
    lens = [11, 5, 1, 0]
    for causal, style in ((True, "interleaved"), (False, "half")):
        q = rng.standard_normal((B, T, H, d))
        k = rng.standard_normal((B, T, KV, d))
        v = rng.standard_normal((B, T, KV, d))
        o, lse = oracle.attention_padded(q, k, v, lens, causal=causal, base=1e4, style=style)
        for b, n in enumerate(lens):
            assert np.isnan(o[b, n:]).all() and np.isnan(lse[b, :, n:]).all()
            if n == 0:
                continue
            ob, lb = brute_force(q[b:b + 1, :n].tolist(), k[b:b + 1, :n].tolist(), v[b:b + 1, :n].tolist(),
                                 causal, 1e4, style)
            assert np.allclose(o[b, :n], ob[0], atol=1e-12, rtol=0)
            assert np.allclose(lse[b, :, :n], lb[0], atol=1e-12, rtol=0)
            # SDPA over all T keys with the padding keys (and the future) masked out.
            pos = np.arange(T)
            qr = torch.from_numpy(oracle.apply_rope(q[b], pos, 1e4, style)).permute(1, 0, 2)
            kr = torch.from_numpy(oracle.apply_rope(k[b], pos, 1e4, style)).permute(1, 0, 2)
            vv = torch.from_numpy(v[b]).permute(1, 0, 2)
            kr = kr.repeat_interleave(H // KV, 0)
            vv = vv.repeat_interleave(H // KV, 0)
            allow = torch.arange(T)[None, :] < n
            if causal:
                allow = allow & (torch.arange(T)[None, :] <= torch.arange(T)[:, None])
            ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, attn_mask=allow)
            assert np.allclose(o[b, :n], ref.permute(1, 0, 2).numpy()[:n], atol=1e-12, rtol=0)
        # The padding tokens carry no information.
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for b, n in enumerate(lens):
            q2[b, n:] = 1e3 * rng.standard_normal(q2[b, n:].shape)
            k2[b, n:] = 1e3 * rng.standard_normal(k2[b, n:].shape)
            v2[b, n:] = 1e3 * rng.standard_normal(v2[b, n:].shape)
        o2, l2 = oracle.attention_padded(q2, k2, v2, lens, causal=causal, base=1e4, style=style)
        assert np.array_equal(np.isnan(o2), np.isnan(o)) and np.allclose(o2, o, atol=0, rtol=0, equal_nan=True)
        assert np.allclose(l2, lse, atol=0, rtol=0, equal_nan=True)
        of, lf = oracle.attention_padded(q, k, v, [T] * B, causal=causal, base=1e4, style=style)
        od, ld = oracle.attention_dense(q, k, v, causal=causal, base=1e4, style=style)
        assert np.array_equal(of, od) and np.array_equal(lf, ld)


ALL_CHECKS = [
    check_inv_freq_closed_forms,
    check_tables_closed_forms,
    check_rope_d2_is_plane_rotation,
    check_rope_interleaved_complex_form,
    check_rope_half_matches_rotate_half_form,
    check_rope_norm_and_identity,
    check_rope_relative,
    check_rope_styles_related_by_permutation,
    check_brute_force,
    check_library_sdpa,
    check_softmax_rows,
    check_causal_row0,
    check_gqa_is_mha_with_repeat_interleave,
    check_zero_query_closed_form,
    check_single_token,
    check_scale_argument,
    check_varlen_is_concat_of_dense,
    check_rows_match_full,
    check_rope_transpose_inverts_rotation,
    check_bwd_finite_differences,
    check_bwd_torch_autograd,
    check_bwd_gqa_is_mha_summed,
    check_bwd_invariants,
    check_bwd_closed_forms,
    check_bwd_varlen_is_concat_of_dense,
    check_bwd_group_matches_full,
    check_decode_is_the_end_of_the_causal_forward,
    check_decode_special_cases,
    check_window_is_causal_attention_on_a_slice,
    check_window_special_cases,
    check_window_backward,
    check_rmsnorm_closed_forms,
    check_rmsnorm_qkv_rope_structure,
    check_padding_mask,
]
