"""The fp8 inputs' format, pinned to its definition (CPU only).

The fp8 forward takes OCP e4m3 codes: 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits, subnormals at exponent 0, no infinities, 0x7f and 0xff
NaN, largest finite 448. The test inputs are quantized and the oracle's
inputs dequantized by torch's float8_e4m3fn conversion; this checks that
conversion against the definition for all 256 codes, and that quantization
rounds to the nearest code (ties to even)."""

import math

import numpy as np
import torch

import workloads as W


def decode(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_every_code_decodes_by_the_definition():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = np.array([decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(codes) == nan).all()
    assert np.array_equal(codes[~nan], ref[~nan])
    assert ref[~nan].max() == 448.0 and ref[0x01] == 2.0 ** -9


def test_quantization_rounds_to_nearest_even():
    finite = sorted({decode(c) for c in range(256) if not math.isnan(decode(c))})
    rng = np.random.default_rng(0)
    x = rng.uniform(-448, 448, 20000)
    got = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    grid = np.array(finite)
    idx = np.abs(grid[None, :] - x.astype(np.float32).astype(np.float64)[:, None]).argmin(axis=1)
    assert np.array_equal(np.abs(got - x), np.abs(grid[idx] - x)) or np.allclose(np.abs(got - x), np.abs(grid[idx] - x))


def test_quantize_fp8_uses_the_range():
    x = torch.linspace(-3.0, 5.0, 1001)
    codes, ds = W.quantize_fp8(x)
    back = codes.to(torch.float64) * ds
    assert float(codes.to(torch.float32).abs().max()) == 448.0
    assert torch.allclose(back, x.double(), rtol=2.0 ** -4, atol=2.0 ** -9 * ds)
