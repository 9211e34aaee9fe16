"""Pins of the oracle's codebooks against closed forms, invariants and an
independent library routine (CPU only).

The dynamic code, NF4 and FP4 are readings of the pages (the dynamic code of
the abstract quoted on "Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略",
section 2; NF4 of "Bitsandbytes", section Normal Float 4 (NF4); FP4 of
"Quantize 🤗 Transformers models", section FP4 quantization).  No table is
printed on the pages, so each is pinned to its defining construction computed
here by other means.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.stats

import oracle


def is_rn32(f, exact):
    """True if binary32 f is the round-to-nearest-even of the rational `exact`:
    no neighbour is closer, and on a tie the significand of f is even."""
    f = np.float32(f)
    d = abs(Fraction(float(f)) - exact)
    for g in (np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
        dg = abs(Fraction(float(g)) - exact)
        if dg < d:
            return False
        if dg == d and (int(np.array(f, dtype=np.float32).view(np.uint32)) & 1):
            return False
    return True


def dyn8_exact_positive():
    vals = []
    for e in range(7):
        for j in range(2 ** e):
            # 10^(e-6) * (1/10 + 9/10 * (j + 1/2) / 2^e)
            vals.append(Fraction(10) ** (e - 6) * (Fraction(1, 10) + Fraction(9, 10) * (j + Fraction(1, 2)) / 2 ** e))
    return vals


def test_dyn8_is_rounded_exact_construction():
    cb = oracle.codebook(oracle.DYN8)
    pos = dyn8_exact_positive()
    assert len(pos) == 127
    exact = [-v for v in reversed(pos)] + [Fraction(0)] + pos + [Fraction(1)]
    for f, ex in zip(cb, exact):
        assert is_rn32(f, ex), (f, ex)


def test_dyn8_invariants():
    cb = oracle.codebook(oracle.DYN8)
    assert cb.dtype == np.float32 and cb.size == 256
    assert np.all(np.diff(cb) > 0), "strictly ascending"
    assert cb[127] == 0.0 and cb[255] == 1.0
    for k in range(1, 128):
        assert cb[127 - k] == -cb[127 + k]
    assert cb[254] == np.float32(0.99296875)
    assert cb[128] == np.float32(5.5e-7)
    # decade counts 1, 2, 4, ..., 64 (plus the extra +1.0 in the top decade)
    pos = cb[128:255].astype(np.float64)
    counts = [int(np.sum((pos > 10.0 ** (e - 7)) & (pos < 10.0 ** (e - 6)))) for e in range(7)]
    assert counts == [1, 2, 4, 8, 16, 32, 64]
    # largest half-gap on [0.1, 1] is 0.9/64/2
    top = cb[(cb >= 0.1)].astype(np.float64)
    assert abs(np.max(np.diff(top)) / 2 - 0.00703125) < 1e-7   # binary32 rounding of the entries


def test_nf4_matches_scipy_quantiles():
    cb = oracle.codebook(oracle.NF4)
    delta = 0.5 * (1 / 30 + 1 / 32)
    P = 1 - delta
    pos = scipy.stats.norm.ppf(0.5 + (P - 0.5) * np.arange(1, 9) / 8)
    neg = -scipy.stats.norm.ppf(0.5 + (P - 0.5) * np.arange(1, 8) / 7)
    ref = np.sort(np.concatenate([neg, [0.0], pos]) / scipy.stats.norm.ppf(P))
    # scipy's ppf is accurate to ~1e-15 relative; the binary32 roundings agree
    assert np.array_equal(cb, ref.astype(np.float32))
    # no entry sits close enough to a binary32 tie for the two roundings to disagree
    f32 = ref.astype(np.float32).astype(np.float64)
    ulp = np.abs(np.spacing(ref.astype(np.float32))).astype(np.float64)
    nz = ref != 0
    assert np.all(np.abs(np.abs(ref[nz] - f32[nz]) - ulp[nz] / 2) > 1e-12 * np.abs(ref[nz]))


def test_nf4_invariants():
    cb = oracle.codebook(oracle.NF4)
    assert cb.size == 16 and np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[7] == 0.0 and cb[15] == 1.0
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8
    assert abs(cb[1] + 0.6961928) < 1e-6 and abs(cb[14] - 0.7229568) < 2e-6


def test_fp4_is_e2m1_over_six():
    cb = oracle.codebook(oracle.FP4)
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]     # E2M1 magnitudes by bit pattern
    for k, m in enumerate(e2m1):
        assert is_rn32(cb[k], Fraction(m) / 6)
        assert cb[8 + k] == (-cb[k] if k else 0.0)
    assert np.array(cb[8], dtype=np.float32).view(np.uint32) == 0, "code 8 decodes to +0.0"
    assert np.all(np.diff(cb[:8]) > 0)
