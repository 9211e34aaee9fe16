"""Pins of the oracle's unsigned dynamic 8-bit code and of the 8-bit steps that
keep their never-negative state in it (CPU only).

Reading: the pages name only the signed dynamic code (abstract quoted on
"Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略", section 2); the
unsigned form spends the sign bit on one more fraction bit, so each of the same
seven decades holds twice as many linearly spaced magnitudes.  Pinned to its
defining construction (exact rationals), to its relation with the signed code,
to a brute-force nearest-entry search, and to the binary32 step."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle_codebooks import is_rn32
from test_oracle_encoder import brute


def udyn8_exact_positive():
    vals = []
    for e in range(7):
        for j in range(2 ** (e + 1)):
            # 10^(e-6) * (1/10 + 9/10 * (j + 1/2) / 2^(e+1))
            vals.append(Fraction(10) ** (e - 6) * (Fraction(1, 10) + Fraction(9, 10) * (j + Fraction(1, 2))
                                                   / 2 ** (e + 1)))
    return vals


def test_udyn8_is_rounded_exact_construction():
    cb = oracle.codebook(oracle.UDYN8)
    pos = udyn8_exact_positive()
    assert len(pos) == 254
    exact = [Fraction(0)] + pos + [Fraction(1)]
    assert cb.dtype == np.float32 and cb.size == 256
    for f, ex in zip(cb, exact):
        assert is_rn32(f, ex), (f, ex)


def test_udyn8_invariants():
    cb = oracle.codebook(oracle.UDYN8)
    assert np.all(np.diff(cb) > 0), "strictly ascending"
    assert cb[0] == 0.0 and cb[255] == 1.0
    assert cb[1] == np.float32(3.25e-7)                   # (4 + 9) / (4 * 10^7)
    assert cb[254] == np.float32(2551 / 2560)             # (256 + 18*127 + 9) / (256 * 10)
    # 2^(e+1) entries in decade e, [10^(e-7), 10^(e-6)), e = 0..6
    for e in range(7):
        lo, hi = 10.0 ** (e - 7), 10.0 ** (e - 6)
        assert np.sum((cb >= lo) & (cb < hi)) == 2 ** (e + 1)


def test_signed_magnitudes_are_midpoints_of_unsigned_pairs():
    """Each positive entry of the signed code is the midpoint of two adjacent
    unsigned entries (the unsigned code splits every bin of the signed one in
    two): exactly for the rationals, so within one ulp for the binary32
    values (half an ulp from each side's rounding)."""
    s = oracle.codebook(oracle.DYN8)[128:255].astype(np.float64)   # 127 magnitudes
    u = oracle.codebook(oracle.UDYN8)[1:255].astype(np.float64)    # 254 magnitudes
    mid = (u[0::2] + u[1::2]) / 2
    ulp = np.spacing(s.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(s - mid) <= ulp), np.max(np.abs(s - mid) / ulp)


def test_udyn8_encoder_matches_brute_force():
    cb = oracle.codebook(oracle.UDYN8)
    rng = np.random.default_rng(77)
    vals = list(rng.uniform(0, 1, 600).astype(np.float32))
    vals += list(np.abs(rng.standard_normal(200) * 1e-5).astype(np.float32))
    for a, b in zip(cb[:-1], cb[1:]):
        mid = np.float32((np.float64(a) + np.float64(b)) / 2)
        vals += [mid, np.nextafter(mid, np.float32(2)), np.nextafter(mid, np.float32(-2))]
    vals += list(cb) + [np.float32(0.0), np.float32(-0.0), np.float32(1e-45), np.float32(1.625e-7),
                        np.float32(-0.25)]                # a negative input takes the entry 0.0
    x = np.array(vals, dtype=np.float32)
    got = oracle.encode(oracle.UDYN8, x)
    for xi, gi in zip(x, got):
        assert gi == brute(oracle.UDYN8, xi), (float(xi), int(gi))


def test_unsigned_code_halves_the_worst_error_on_a_positive_state():
    """A v-like state (squares of normal gradients): block-wise round trips with
    both codes; relative to the block absmax the worst error is the code's
    largest half-gap, 0.00352 unsigned against 0.00703 signed, and the mean
    error drops too."""
    B = 2048
    v = (np.random.default_rng(5).standard_normal(B * 64) * 1e-3).astype(np.float32) ** 2
    err = {}
    for code in (oracle.DYN8, oracle.UDYN8):
        c, a = oracle.quantize_blockwise(v, code, B)
        y = oracle.dequantize_blockwise(c, a, code, B, v.size)
        err[code] = np.abs(y - v).reshape(-1, B) / a[:, None]
    cbu, cbs = oracle.codebook(oracle.UDYN8), oracle.codebook(oracle.DYN8)[127:]
    assert err[oracle.UDYN8].max() <= np.max(np.diff(cbu)) / 2 * (1 + 1e-6)
    assert err[oracle.DYN8].max() <= np.max(np.diff(cbs)) / 2 * (1 + 1e-6)
    assert np.max(np.diff(cbu)) / 2 < 0.0036 and np.max(np.diff(cbs)) / 2 > 0.0070
    assert err[oracle.UDYN8].mean() < 0.6 * err[oracle.DYN8].mean()


UV_KINDS = [(oracle.ADAMW, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)),
            (oracle.ADAM, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)),
            (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, eps=1e-8, wd=0.0)),
            (oracle.LAMB, dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, wd=0.01))]


def rnd(seed, n, scale):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


@pytest.mark.parametrize("kind,hp", UV_KINDS)
def test_8bit_step_with_unsigned_state_is_the_quantized_binary32_update(kind, hp):
    """One 8-bit step with the never-negative state in the unsigned code =
    decode every state with its code, the binary32 update, block-wise
    re-quantization with the same codes."""
    n, B = 2048 * 4 + 333, 2048
    two = oracle.OPTIMIZER_STATES[kind] == 2
    vs = 1 if kind == oracle.RMSPROP else 2                 # which state is never negative
    code = {1: oracle.UDYN8 if vs == 1 else oracle.DYN8, 2: oracle.UDYN8}
    p0, g = rnd(10 + kind, n, 0.02), rnd(20 + kind, n, 1e-3)
    s1 = rnd(30 + kind, n, 1e-3)
    s2 = np.abs(rnd(40 + kind, n, 1e-6))
    if vs == 1:
        s1 = np.abs(s1)
    c1, a1 = oracle.quantize_blockwise(s1, code[1], B)
    c2, a2 = oracle.quantize_blockwise(s2, code[2], B)
    d1 = oracle.dequantize_blockwise(c1, a1, code[1], B, n)
    d2 = oracle.dequantize_blockwise(c2, a2, code[2], B, n)
    step = 3
    p32, x1, x2 = p0.copy(), d1.copy(), d2.copy()
    oracle.optim32_step(kind, p32, g, x1, x2 if two else None, step=step, **hp)
    p8 = p0.copy()
    oracle.optim8bit_step(kind, p8, g, c1, a1, c2 if two else None, a2 if two else None, B, step=step,
                          vcode=oracle.UDYN8, **hp)
    assert np.array_equal(p8, p32)
    q1, qa1 = oracle.quantize_blockwise(x1, code[1], B)
    assert np.array_equal(c1, q1) and np.array_equal(a1, qa1)
    if two:
        q2, qa2 = oracle.quantize_blockwise(x2, code[2], B)
        assert np.array_equal(c2, q2) and np.array_equal(a2, qa2)


def test_unsigned_code_needs_a_never_negative_state():
    n, B = 100, 64
    p, g = rnd(1, n, 0.02), rnd(2, n, 1e-3)
    c, a = np.full(n, 127, np.uint8), np.zeros(2, np.float32)
    for kind, hp in [(oracle.LION, dict(lr=1e-4, beta1=0.9, beta2=0.99)),
                     (oracle.SGD, dict(lr=1e-2, beta1=0.9)),
                     (oracle.LARS, dict(lr=0.5, beta1=0.9, trust=1e-3))]:
        with pytest.raises(RuntimeError):
            oracle.optim8bit_step(kind, p.copy(), g, c.copy(), a.copy(), None, None, B, vcode=oracle.UDYN8, **hp)
    with pytest.raises(RuntimeError):
        oracle.optim8bit_step(oracle.ADAM, p.copy(), g, c.copy(), a.copy(), c.copy(), a.copy(), B, vcode=7,
                              lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
