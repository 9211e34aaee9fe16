"""Brute-force pin of the oracle's nearest-code encoder (CPU only).

For every input the expected code is the argmin over ALL codebook entries of the
exact distance (Python fractions), a tie going to the entry of smaller
magnitude.  Inputs cover random values, every exact midpoint between adjacent
entries and its binary32 neighbours, every entry, +-0, +-1, and extremes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def brute(code, x):
    cb = oracle.codebook(code)
    if code == oracle.FP4:
        mags = [Fraction(float(c)) for c in cb[:8]]
        ax = abs(Fraction(float(x)))
        best = min(range(8), key=lambda k: (abs(ax - mags[k]), mags[k]))
        return (8 | best) if (x < 0 and best > 0) else best
    ent = [Fraction(float(c)) for c in cb]
    fx = Fraction(float(x))
    return min(range(len(ent)), key=lambda k: (abs(fx - ent[k]), abs(ent[k])))


def probe_inputs(code, rng, n_random):
    cb = oracle.codebook(code)
    vals = list(rng.uniform(-1, 1, n_random).astype(np.float32))
    vals += list((rng.standard_normal(n_random // 4) * 1e-4).astype(np.float32))
    srt = np.sort(cb[:8]) if code == oracle.FP4 else cb
    for a, b in zip(srt[:-1], srt[1:]):
        mid = np.float32((np.float64(a) + np.float64(b)) / 2)
        for v in (mid, np.nextafter(mid, np.float32(2)), np.nextafter(mid, np.float32(-2))):
            vals += [v, -v]
    vals += list(cb) + list(-cb)
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0),
             np.float32(1e-38), np.float32(-1e-38), np.float32(1e-45), np.float32(2.75e-7),
             np.float32(-2.75e-7)]
    x = np.array(vals, dtype=np.float32)
    return x[np.abs(x) <= 1]


@pytest.mark.parametrize("code,n_random", [(oracle.DYN8, 600), (oracle.NF4, 3000), (oracle.FP4, 3000)])
def test_encoder_matches_brute_force(code, n_random):
    rng = np.random.default_rng(1234 + code)
    x = probe_inputs(code, rng, n_random)
    got = oracle.encode(code, x)
    for xi, gi in zip(x, got):
        assert gi == brute(code, xi), (code, float(xi), int(gi))


def test_exact_midpoint_ties_go_toward_zero():
    """Every adjacent pair whose exact midpoint is a binary32 value: that value
    encodes to the entry of smaller magnitude, for both signs."""
    found = 0
    for code in (oracle.DYN8, oracle.NF4, oracle.FP4):
        cb = oracle.codebook(code)
        srt = np.sort(cb[:8]) if code == oracle.FP4 else cb
        for k in range(len(srt) - 1):
            mid = (np.float64(srt[k]) + np.float64(srt[k + 1])) / 2
            if np.float64(np.float32(mid)) != mid:
                continue
            found += 1
            x = np.array([mid], dtype=np.float32)
            got = int(oracle.encode(code, x)[0])
            small = k if abs(srt[k]) < abs(srt[k + 1]) else k + 1
            if code == oracle.FP4:
                want = small if mid >= 0 else (8 | small)
                assert got == (small if small == 0 else want)
            else:
                assert got == small
    assert found >= 5, "the tie rule must be exercised"
