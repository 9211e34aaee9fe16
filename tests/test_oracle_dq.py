"""Pins of the oracle's nested (double) quantization (CPU only).

"Bitsandbytes" (Transformers docs), section İç içe nicelleştirme: a second
quantization of the already quantized constants saves about 0.4 bit per
parameter.  The reading: centre the fp32 absmax on its exact mean (rounded once
to binary32) and quantize the differences with the dynamic 8-bit code in blocks
of 256.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def is_rn32(f, exact):
    f = np.float32(f)
    d = abs(Fraction(float(f)) - exact)
    for g in (np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
        dg = abs(Fraction(float(g)) - exact)
        if dg < d or (dg == d and (int(np.array(f).view(np.uint32)) & 1)):
            return False
    return True


def test_rn32_rational_is_nearest_even():
    rng = np.random.default_rng(21)
    for _ in range(3000):
        num = int(rng.integers(1, 2 ** 62)) * int(rng.integers(1, 2 ** 40))
        den = int(rng.integers(1, 2 ** 60))
        shift = int(rng.integers(-170, 120))
        if shift >= 0:
            num <<= shift
        else:
            den <<= -shift
        try:
            f = oracle.rn32_rational(num, den)
        except OverflowError:
            assert Fraction(num, den) > 3.4e38
            continue
        assert is_rn32(f, Fraction(num, den))
    # exact ties to even, and the subnormal range
    assert oracle.rn32_rational(2 ** 24 + 1, 2) == np.float32(2 ** 23)        # 2^23 + 0.5 -> even
    assert oracle.rn32_rational(2 ** 24 + 3, 2) == np.float32(2 ** 23 + 2)
    assert oracle.rn32_rational(1, 2 ** 150) == np.float32(0.0)               # half of 2^-149 -> 0 (even)
    assert oracle.rn32_rational(3, 2 ** 150) == np.float32(2.0 ** -148)


def test_exact_mean_pins():
    rng = np.random.default_rng(22)
    # a constant vector has itself as mean
    for v in (np.float32(0.0123), np.float32(3e-38), np.float32(1e30)):
        assert oracle.exact_mean_f32(np.full(1001, v, dtype=np.float32)) == v
    # against the exact rational mean, for values spread over many binades
    a = np.abs(rng.standard_normal(777) * np.exp(rng.uniform(-40, 40, 777))).astype(np.float32)
    exact = sum(Fraction(float(x)) for x in a) / a.size
    assert is_rn32(oracle.exact_mean_f32(a), exact)
    # math.fsum is the correctly rounded binary64 sum; for absmax-like values on
    # a common grid it is exact, and the mean is then fsum / n rounded once
    a = rng.uniform(0.01, 0.2, 100000).astype(np.float32)
    s = math.fsum(float(x) for x in a)
    exact_sum = sum(Fraction(float(x)) for x in a)
    assert Fraction(s) == exact_sum
    assert is_rn32(oracle.exact_mean_f32(a), Fraction(s) / a.size)


def test_exact_mean_independent_of_order():
    rng = np.random.default_rng(23)
    a = np.abs(rng.standard_normal(5000) * np.exp(rng.uniform(-60, 60, 5000))).astype(np.float32)
    m = oracle.exact_mean_f32(a)
    for _ in range(3):
        assert oracle.exact_mean_f32(rng.permutation(a)) == m


def test_dq_error_bound_and_structure():
    rng = np.random.default_rng(24)
    w = (rng.standard_normal(64 * 3000 + 40) * 0.02).astype(np.float32)
    codes, st = oracle.quantize(w, oracle.NF4, 64, double_quant=True)
    a = st["absmax_fp32"]
    assert st["c2"].size == a.size and st["absmax2"].size == (a.size + 255) // 256
    assert st["mu"] == oracle.exact_mean_f32(a)
    ahat = oracle.dq_decode(st["c2"], st["absmax2"], st["mu"])
    a2 = np.repeat(st["absmax2"], 256)[:a.size].astype(np.float64)
    bound = a2 * 0.00703126 + 2 * np.abs(np.spacing(ahat)).astype(np.float64)
    assert np.all(np.abs(a.astype(np.float64) - ahat.astype(np.float64)) <= bound)
    # a DQ'd dequantize equals a plain dequantize with the decoded absmax
    y1 = oracle.dequantize(codes, st, oracle.NF4, 64, w.size)
    y2 = oracle.dequantize_blockwise(codes, ahat, oracle.NF4, 64, w.size)
    assert np.array_equal(y1, y2)


def test_dq_decode_closed_form():
    cb = oracle.codebook(oracle.DYN8)
    c2 = np.array([127, 255, 0, 200], dtype=np.uint8)
    a2 = np.array([0.5], dtype=np.float32)
    mu = np.float32(0.1)
    got = oracle.dq_decode(c2, a2, mu, 256)
    want = ((cb[c2] * a2[0]).astype(np.float32) + mu).astype(np.float32)
    assert np.array_equal(got, want)
    assert got[0] == mu and got[1] == np.float32(np.float32(0.5) + mu)
