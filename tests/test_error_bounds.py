"""Pins of the format-derived error model (tests/error_bounds.py): its
standard deviations against Monte Carlo runs of random roundings of exactly
the kind it models, on small inputs, for each of its terms."""

import numpy as np
import pytest

from tests.error_bounds import attention_sigma

L, D = 24, 8


def inputs(seed, spread=1.5):
    rng = np.random.default_rng(seed)
    qs = rng.standard_normal((L, D)) * spread
    kt = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    vis = np.tril(np.ones((L, L), dtype=bool))
    return qs, kt, v, vis


def monte_carlo(qs, kt, v, vis, fq, fk, fp, psum, n=6000, seed=0):
    """Empirical std of O and lse when qs, kt and p take random rounding errors
    e ~ U(-(u|x| + a), u|x| + a), p taken against the exact row max."""
    rng = np.random.default_rng(seed)

    def perturb(x, f):
        h = f["u"] * np.abs(x) + f["a"]
        return x + h * rng.uniform(-1.0, 1.0, x.shape)

    outs, lses = [], []
    for _ in range(n):
        q2, k2 = perturb(qs, fq), perturb(kt, fk)
        S = q2 @ k2.T
        S[~vis] = -np.inf
        m = S.max(axis=1, keepdims=True)
        p = np.exp2(S - m)
        pr = np.where(vis, perturb(p, fp), 0.0)
        lsum = (pr if psum == "rounded" else p).sum(axis=1)
        outs.append((pr @ v) / lsum[:, None])
        lses.append(np.log(2.0) * (m[:, 0] + np.log2(lsum)))
    return np.std(outs, axis=0), np.std(lses, axis=0)


@pytest.mark.parametrize("which", ["q", "k", "p_rounded", "p_unrounded", "all"])
def test_sigma_matches_monte_carlo(which):
    qs, kt, v, vis = inputs(3)
    zero = dict(u=0.0, a=0.0)
    f = dict(u=2.0 ** -7, a=2.0 ** -12)
    fq = f if which in ("q", "all") else zero
    fk = f if which in ("k", "all") else zero
    fp = f if which.startswith("p") or which == "all" else zero
    psum = "unrounded" if which == "p_unrounded" else "rounded"
    _, _, so, sl = attention_sigma(qs, kt, v, vis, qfmt=fq, kfmt=fk, pfmt=fp, psum=psum)
    mo, ml = monte_carlo(qs, kt, v, vis, fq, fk, fp, psum)
    big = so > 0.2 * so.max()
    r = mo[big] / so[big]
    assert 0.9 < np.median(r) < 1.1 and r.min() > 0.75 and r.max() < 1.3, (which, np.median(r), r.min(), r.max())
    if which != "p_unrounded":
        bl = sl > 0.2 * sl.max()
        rl = ml[bl] / sl[bl]
        assert 0.85 < np.median(rl) < 1.15 and rl.min() > 0.7 and rl.max() < 1.35, (which, rl.min(), rl.max())
    else:
        assert np.allclose(sl, 0.0) and np.allclose(ml, 0.0, atol=1e-12)


def test_max_form_covers_both_row_sums():
    qs, kt, v, vis = inputs(5)
    f = dict(u=2.0 ** -5, a=2.0 ** -10)
    kw = dict(qfmt=f, kfmt=f, pfmt=f)
    _, _, s_max, _ = attention_sigma(qs, kt, v, vis, **kw)
    _, _, s_r, _ = attention_sigma(qs, kt, v, vis, psum="rounded", **kw)
    _, _, s_u, _ = attention_sigma(qs, kt, v, vis, psum="unrounded", **kw)
    assert (s_max >= s_r - 1e-15).all() and (s_max >= s_u - 1e-15).all()


def test_first_row_has_no_softmax_error():
    """Causal row 0 sees one key: P = 1 whatever the scores, so neither the
    operands nor a rounded p that the row sum also adds move its output."""
    qs, kt, v, vis = inputs(7)
    f = dict(u=2.0 ** -4, a=0.0)
    O, _, so, _ = attention_sigma(qs, kt, v, vis, qfmt=f, kfmt=f, pfmt=f, psum="rounded")
    assert np.allclose(O[0], v[0]) and np.allclose(so[0], 0.0, atol=1e-8 * so.max())
