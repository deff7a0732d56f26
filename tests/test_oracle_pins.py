"""The oracle against its pins, and planted mistakes against the pins (CPU only)."""

import importlib.util
import os
import types

import pytest

import oracle
from tests import oracle_checks

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()


# Each mutant is one plausible mistake, planted by editing the oracle's source
# text in memory: (what it breaks, text to find, replacement).
MUTANTS = [
    ("padding rows written as zeros", "O = np.full_like(q, np.nan)", "O = np.zeros_like(q)"),
    ("length-1 entries dropped", "        if n > 0:\n            O[b, :n]", "        if n > 1:\n            O[b, :n]"),
    ("padding keys visible", "_one_sequence(q[b, :n], k[b, :n], v[b, :n]",
     "_one_sequence(q[b], k[b], v[b]"),
    ("exponent -i/d", "-2.0 * i / head_dim", "-1.0 * i / head_dim"),
    ("base^(+2i/d)", "-2.0 * i / head_dim", "2.0 * i / head_dim"),
    ("rotation sign", "y[..., 0::2] = a * c - b * s", "y[..., 0::2] = a * c + b * s"),
    ("dropped sin term", "y[..., 1::2] = a * s + b * c", "y[..., 1::2] = b * c"),
    ("half pairing swapped", "y[..., d // 2:] = a * s + b * c", "y[..., d // 2:] = a * c + b * s"),
    ("GQA repeat instead of repeat_interleave", "kv = h // G  #", "kv = h % KV  #"),
    ("mask hides the diagonal", "hide |= kp > qp", "hide |= kp >= qp"),
    ("sliding window one key too wide", "hide |= qp - kp >= window", "hide |= qp - kp > window"),
    ("sliding window ignored", "    if window > 0:\n        hide |=", "    if window < 0:\n        hide |="),
    ("sampled row ignores the window", "lo = max(0, t - window + 1) if window > 0 else 0",
     "lo = 0"),
    ("no softmax scale", "S = (qr[:, h, :] @ kr[:, kv, :].T) * scale",
     "S = (qr[:, h, :] @ kr[:, kv, :].T)"),
    ("transposed P", "O[:, h, :] = P @ v[:, kv, :]", "O[:, h, :] = P.T @ v[:, kv, :]"),
    ("lse without max", "lse[h] = m + np.log(den)", "lse[h] = np.log(den)"),
    ("K not rotated", "kr = apply_rope(k, pos, base, style)", "kr = k"),
    ("positions do not restart per sequence",
     "O[a:b], lse[:, a:b] = _one_sequence(q[a:b], k[a:b], v[a:b], causal, scale, base, style, window)",
     "O[a:b], lse[:, a:b] = _one_sequence(q[:b], k[:b], v[:b], causal, scale, base, style, window)[0][a:b],"
     " _one_sequence(q[:b], k[:b], v[:b], causal, scale, base, style, window)[1][:, a:b]"),
    ("sampled row sees one key too few", "n = t + 1 if causal else L", "n = t if causal else L"),
    ("sampled row uses wrong KV head", "keys, vals = k[b, :, h // G], v[b, :, h // G]",
     "keys, vals = k[b, :, h % KV], v[b, :, h % KV]"),
    # Backward.
    ("softmax backward without the row-sum term",
     "dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP"),
    ("rotation transposed with the wrong sign", "x[..., 0::2] = a * c + b * s",
     "x[..., 0::2] = a * c - b * s"),
    ("half-pairing transpose with the wrong sign", "x[..., d // 2:] = -a * s + b * c",
     "x[..., d // 2:] = a * s + b * c"),
    ("dq without the softmax scale", "dqr[:, h, :] = (dS @ kr[:, kv, :]) * scale",
     "dqr[:, h, :] = dS @ kr[:, kv, :]"),
    ("dk from un-rotated queries", "dkr[:, kv, :] += (dS.T @ qr[:, h, :]) * scale",
     "dkr[:, kv, :] += (dS.T @ q[:, h, :]) * scale"),
    ("dk not accumulated over the group", "dkr[:, kv, :] += (dS.T @ qr[:, h, :]) * scale",
     "dkr[:, kv, :] = (dS.T @ qr[:, h, :]) * scale"),
    ("dv not accumulated over the group", "dv[:, kv, :] += P.T @ dout[:, h, :]",
     "dv[:, kv, :] = P.T @ dout[:, h, :]"),
    ("dv from P instead of its transpose", "dv[:, kv, :] += P.T @ dout[:, h, :]",
     "dv[:, kv, :] += P @ dout[:, h, :]"),
    ("dP against the wrong K/V head", "dP = dout[:, h, :] @ v[:, kv, :].T",
     "dP = dout[:, h, :] @ v[:, h % KV, :].T"),
    ("dq left rotated", "dq = apply_rope_transpose(dqr, pos, base, style)", "dq = dqr"),
    ("backward ignores the mask", "        S[hidden] = -np.inf\n        e = np.exp",
     "        e = np.exp"),
    ("group backward ignores the window", "lo = max(0, r0 - window + 1) if window > 0 else 0",
     "lo = max(0, r0 - window + 2) if window > 0 else 0"),
    ("group backward drops the last row", "r1 = min(T, r0 + rows_per_block)",
     "r1 = min(T - 1, r0 + rows_per_block)"),
    ("group backward sees one key too few", "            n = r1 if causal else T",
     "            n = r1 - 1 if causal else T"),
    ("decode queries at positions 0..Tq-1", "qpos = np.arange(L - Tq, L)", "qpos = np.arange(0, Tq)"),
    ("decode mask aligned with the start", "hidden = _hidden(qpos, np.arange(L), True, window)",
     "hidden = _hidden(np.arange(Tq), np.arange(L), True, window)"),
    ("decode keys unrotated", "kr = apply_rope(k[b, :L], np.arange(L), base, style)", "kr = k[b, :L]"),
    ("decode sees cache rows past the length", "O[b, :, h, :] = (e / den[:, None]) @ v[b, :L, kv, :]",
     "O[b, :, h, :] = (e / den[:, None]) @ v[b, :L, kv, :] + 0.0 * v[b, L - 1:L, kv, :].sum() + "
     "(v[b, L:, kv, :].sum() if L < v.shape[1] else 0.0)"),
    ("rmsnorm without the mean", "np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
     "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    ("rmsnorm eps outside the root", "np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
     "(np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    ("projection not transposed", "y = rmsnorm(x, norm_weight, eps) @ W.T",
     "y = rmsnorm(x, norm_weight, eps) @ W.reshape(W.shape[1], W.shape[0])"),
    ("k and v slices swapped", "k = y[:, n_head * d:(n_head + n_kv_head) * d].reshape(N, n_kv_head, d)",
     "k = y[:, (n_head + n_kv_head) * d:].reshape(N, n_kv_head, d)"),
    ("v rotated", "    return q, k, v\n", "    return q, k, apply_rope(v, positions, base, style)\n"),
    ("backward positions do not restart per sequence",
     "_one_sequence_bwd(q[a:b], k[a:b], v[a:b], dout[a:b], causal, scale,\n"
     "                                                      base, style, window)",
     "(lambda r: (r[0][a:], r[1][a:], r[2][a:]))(_one_sequence_bwd(q[:b], k[:b], v[:b], dout[:b],"
     " causal, scale, base, style, window))"),
]


def _load_mutant(find, repl):
    src = open(ORACLE_SRC).read()
    assert src.count(find) >= 1, f"mutation target vanished from the oracle: {find!r}"
    src = src.replace(find, repl)
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = types.ModuleType(spec.name)
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, find, repl, monkeypatch):
    mutant = _load_mutant(find, repl)
    monkeypatch.setattr(oracle_checks, "oracle", mutant)
    failed = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            with __import__("warnings").catch_warnings():
                __import__("warnings").simplefilter("ignore")
                check()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
