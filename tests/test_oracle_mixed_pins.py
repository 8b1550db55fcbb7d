"""Pins of the oracle's 16-bit-input product (CPU only).

The oracle reads bf16 and fp16 codes by the published formats and sums exact
fp64 products in ascending k, rounding once to fp32.  Each test fixes it to
something outside itself:

  * the decoders against numpy's float16 and torch's bfloat16 conversions
    over all 65536 codes, and against the formats' textbook constants
    (largest finite, smallest normal and subnormal, 1, -2, a third, pi);
  * the product against exact rational arithmetic (``fractions.Fraction``)
    on tiny inputs whose exponents keep every fp64 partial sum exact;
  * the product against exact integer matmul (numpy int64) for small
    integers, which both formats hold exactly;
  * the product against the fp32 oracle (itself pinned elsewhere) on the
    decoded values, which fp32 holds exactly, so the two must agree bit for
    bit (a transposed operand or a wrong index in either breaks this);
  * the seeded generator's rounding against torch's float32 -> bfloat16 and
    numpy's float32 -> float16 conversions.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make, make_mixed, to_code16

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _same(got: np.ndarray, want: np.ndarray) -> None:
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w)
    ok = ~nan_w
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))  # signed zeros


def test_f16_decode_all_codes_matches_numpy():
    _same(oracle.decode16(ALL, "f16"), ALL.view(np.float16).astype(np.float64))


def test_bf16_decode_all_codes_matches_torch():
    want = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    _same(oracle.decode16(ALL, "bf16"), want.numpy())


@pytest.mark.parametrize("fmt,code,value", [
    ("f16", 0x3C00, 1.0), ("f16", 0xC000, -2.0), ("f16", 0x7BFF, 65504.0),
    ("f16", 0x0400, 2.0 ** -14), ("f16", 0x0001, 2.0 ** -24),
    ("f16", 0x03FF, 1023 / 1024 * 2.0 ** -14), ("f16", 0x3555, 0.333251953125),
    ("f16", 0x7C00, float("inf")), ("f16", 0xFC00, float("-inf")),
    ("bf16", 0x3F80, 1.0), ("bf16", 0xC000, -2.0), ("bf16", 0x4049, 3.140625),
    ("bf16", 0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), ("bf16", 0x0080, 2.0 ** -126),
    ("bf16", 0x0001, 2.0 ** -133), ("bf16", 0x7F80, float("inf")),
])
def test_format_constants(fmt, code, value):
    assert oracle.decode16(np.array([code], np.uint16), fmt)[0] == value


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_nan_codes(fmt):
    code = 0x7E00 if fmt == "f16" else 0x7FC0
    assert np.isnan(oracle.decode16(np.array([code], np.uint16), fmt)[0])


def _narrow_codes(rng, shape, fmt):
    """Random finite codes with exponents within 2^-3..2^3, so every product
    and partial sum of a short dot product is exact in fp64."""
    sign = rng.integers(0, 2, shape).astype(np.uint32) << 15
    if fmt == "f16":
        exp = rng.integers(12, 19, shape).astype(np.uint32) << 10
        frac = rng.integers(0, 1 << 10, shape).astype(np.uint32)
    else:
        exp = rng.integers(124, 131, shape).astype(np.uint32) << 7
        frac = rng.integers(0, 1 << 7, shape).astype(np.uint32)
    return (sign | exp | frac).astype(np.uint16)


def _exact_values(codes, fmt):
    if fmt == "f16":
        return codes.view(np.float16).astype(np.float64)
    t = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (6, 2, 9), (4, 4, 1), (2, 7, 3)])
def test_product_against_exact_rationals(fmt, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a = _narrow_codes(rng, (M, K), fmt)
    b = _narrow_codes(rng, (K, N), fmt)
    av, bv = _exact_values(a, fmt), _exact_values(b, fmt)
    got = oracle.gemm_mixed(a, b, fmt)
    for i in range(M):
        for j in range(N):
            exact = sum((Fraction(av[i, k]) * Fraction(bv[k, j]) for k in range(K)), Fraction(0))
            assert got[i, j] == np.float32(float(exact)), (i, j)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_small_integers_exact(fmt):
    a32, b32 = make(33, 17, 65, "small_int", seed=9)
    a, b = to_code16(a32, fmt), to_code16(b32, fmt)
    want = a32.astype(np.int64) @ b32.astype(np.int64)
    assert np.array_equal(oracle.gemm_mixed(a, b, fmt), want.astype(np.float32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_agrees_with_fp32_oracle_on_decoded_values(fmt):
    a, b = make_mixed(37, 29, 41, "normal", seed=5, fmt=fmt)
    a32 = oracle.decode16(a, fmt).astype(np.float32)
    b32 = oracle.decode16(b, fmt).astype(np.float32)
    assert np.array_equal(oracle.gemm_mixed(a, b, fmt), oracle.gemm(a32, b32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_elems_agree_with_full_product(fmt):
    a, b = make_mixed(23, 31, 19, "uniform", seed=6, fmt=fmt)
    full = oracle.gemm_mixed(a, b, fmt)
    rng = np.random.default_rng(1)
    ii, jj = rng.integers(0, 23, 50), rng.integers(0, 31, 50)
    assert np.array_equal(oracle.gemm_mixed_elems(a, b, fmt, ii, jj), full[ii, jj])


def test_generator_rounding_matches_library_conversions():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        rng.uniform(-1, 1, 20000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-8, 3.0e38], np.float32)])
    want_bf = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_code16(x, "bf16"), want_bf)
    want_h = torch.from_numpy(x[np.abs(x) < 65504]).to(torch.float16).view(torch.int16)
    assert np.array_equal(to_code16(x[np.abs(x) < 65504], "f16"), want_h.numpy().view(np.uint16))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.decode16(np.zeros(2, np.uint16), "fp8")
    with pytest.raises(TypeError):
        oracle.gemm_mixed(np.zeros((2, 2), np.float32), np.zeros((2, 2), np.uint16), "f16")
    with pytest.raises(ValueError):
        oracle.gemm_mixed(np.zeros((2, 3), np.uint16), np.zeros((2, 2), np.uint16), "f16")
