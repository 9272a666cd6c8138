"""Arithmetic identities the HIP kernels are built on, checked on the host with numpy.

These are facts about IEEE fp32/fp64 arithmetic, not about the method: each test states one
identity a kernel uses in place of a more expensive operation, and checks it on many random and
adversarial operands (CPU only).
"""
import numpy as np
import pytest

F32 = np.float32


def _div_via_f64_reciprocal(x, s):
    """fl32(fl64(x * fl64(1 / s))): the prepass's replacement for the fp32 division x / s."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = np.float64(1.0) / s.astype(np.float64)
        return (x.astype(np.float64) * r).astype(F32)


def _div_f32(x, s):
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (x / s).astype(F32)


def _same(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32)) or np.all(
        (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b)))


def test_fp32_division_equals_rounded_fp64_reciprocal_product():
    rng = np.random.default_rng(20261203)
    n = 2_000_000
    # random significands and a wide exponent range (normal and subnormal operands)
    x = (rng.standard_normal(n) * 2.0 ** rng.integers(-140, 120, n)).astype(F32)
    s = np.abs(rng.standard_normal(n) * 2.0 ** rng.integers(-140, 120, n)).astype(F32)
    assert _same(_div_f32(x, s), _div_via_f64_reciprocal(x, s))


def test_division_identity_on_quantization_shaped_operands():
    # the operands the prepass actually divides: bf16 (or fp32 mean-shifted) values by
    # amax / 127 of their block, so quotients lie in [-127, 127] and many sit near half-integers
    rng = np.random.default_rng(7)
    for _ in range(20):
        blk = rng.standard_normal(1 << 16).astype(F32) * F32(rng.uniform(1e-3, 1e3))
        amax = np.max(np.abs(blk))
        scale = F32(amax / F32(127.0))
        s = np.full_like(blk, scale)
        a, b = _div_f32(blk, s), _div_via_f64_reciprocal(blk, s)
        assert _same(a, b)
        assert np.array_equal(np.rint(a), np.rint(b))


def test_division_identity_special_operands():
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38, 3.4e38,
                         1.0, -1.0, 127.0, 0.5, 1.5, 2.5], dtype=F32)
    x = np.repeat(specials, specials.size)
    s = np.abs(np.tile(specials, specials.size))
    assert _same(_div_f32(x, s), _div_via_f64_reciprocal(x, s))


def test_midpoint_quotients_cannot_occur():
    # exhaustive over small odd significands: x / s is never an exact fp32 midpoint, the one
    # case where a 2^-52-accurate product could round the other way
    a = np.arange(1, 1 << 12, 2, dtype=np.int64)
    for b in (3, 5, 7, 127, 255, (1 << 23) + 1, (1 << 24) - 1):
        q = a.astype(np.float64) / b
        assert _same(_div_f32(a.astype(F32), np.full(a.size, b, F32)),
                     _div_via_f64_reciprocal(a.astype(F32), np.full(a.size, b, F32)))
        assert np.all(np.isfinite(q))


@pytest.mark.parametrize("n", [0, 1, -1, 2_064_512, -2_064_512, (1 << 22) - 1, -(1 << 22)])
def test_biased_integer_reads_as_float(n):
    # the int8 attention starts its integer accumulator at bits(1.5 * 2^23); the final bits,
    # read as fp32, are 1.5 * 2^23 + n exactly for |n| < 2^22 (127 * 127 * 128 = 2_064_512)
    bias = np.array([12582912.0], dtype=F32)
    bits = bias.view(np.int32)[0] + np.int32(n)
    as_float = np.array([bits], dtype=np.int32).view(F32)[0]
    assert float(as_float) == 12582912.0 + n
    assert float(as_float - F32(12582912.0)) == float(n)


def test_biased_scores_order_as_signed_integers():
    # ... and the int8 row maximum compares those bit patterns as signed integers, with -inf
    # (a masked key) below every biased score
    n = np.array([-2_064_512, -5, 0, 7, 2_064_512], dtype=np.int64)
    f = (12582912.0 + n).astype(F32)
    allv = np.concatenate([f, np.array([-np.inf], F32)])
    ints = allv.view(np.int32)
    assert np.argmax(ints) == np.argmax(allv)
    assert ints[-1] < ints[:-1].min()
