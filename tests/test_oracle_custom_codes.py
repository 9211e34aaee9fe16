"""Pins of the oracle's user codes (CPU only): the linear 8-bit code, block-wise
quantization with any 256-entry code, and the estimated quantile code (the
pages list quantile, linear and dynamic 8-bit quantization and a fast quantile
estimation: "Py之bitsandbytes", section 1)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_linear_code_closed_form():
    cb = oracle.linear_codebook()
    want = np.array([float(Fraction(k, 127)) for k in range(-128, 128)], dtype=np.float32)   # one rounding
    assert np.array_equal(cb.view(np.uint32), want.view(np.uint32))
    assert cb[128] == 0.0 and cb[255] == 1.0 and cb[1] == -1.0
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    assert np.array_equal(cb[129:], -cb[127:0:-1])          # symmetric around 0 (entry 0 is -128/127)


def brute_nearest(cb, x):
    """argmin over all entries under exact rationals; ties toward the smaller
    magnitude, equal magnitudes to the upper entry."""
    fx = Fraction(float(x))
    best = 0
    for k in range(1, len(cb)):
        db, dk = abs(fx - Fraction(float(cb[best]))), abs(fx - Fraction(float(cb[k])))
        if dk < db or (dk == db and abs(float(cb[k])) <= abs(float(cb[best]))):
            best = k
    return best


@pytest.mark.parametrize("which", ["linear", "symmetric_no_zero", "quantile"])
def test_custom_encoder_equals_brute_force(which):
    rng = np.random.default_rng(3)
    if which == "linear":
        cb = oracle.linear_codebook()
    elif which == "symmetric_no_zero":                     # -a and a adjacent: the equal-magnitude tie
        half = np.sort(rng.uniform(0.001, 1.0, 128)).astype(np.float32)
        half[-1] = 1.0
        cb = np.concatenate([-half[::-1], half]).astype(np.float32)
    else:
        cb = oracle.estimate_quantiles(rng.standard_normal(20000).astype(np.float32))
    mids = [(float(cb[k]) + float(cb[k + 1])) / 2 for k in range(255)]
    xs = list(rng.uniform(-1, 1, 300)) + list(cb) + mids + [0.0, -0.0, 1.0, -1.0]
    xs += [np.nextafter(np.float32(m), np.float32(2)) for m in mids[::7]]
    xs += [np.nextafter(np.float32(m), np.float32(-2)) for m in mids[::7]]
    x = np.array([v for v in xs if abs(v) <= 1.0], dtype=np.float32)
    # one block of absmax 1.0 holding x (the block max is 1 or -1: n = x exactly)
    blk = np.concatenate([x, [1.0]]).astype(np.float32)
    codes, absmax = oracle.quantize_custom(blk, cb, blk.size)
    assert absmax[0] == 1.0
    for xi, c in zip(x, codes[:-1]):
        assert c == brute_nearest(cb, xi), (which, float(xi))


def test_custom_quantize_with_the_dynamic_table_equals_dynamic_quantize():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, 5000) * 0.02).astype(np.float32)
    cb = oracle.codebook(oracle.DYN8)
    for B in (64, 256, 2048):
        c1, a1 = oracle.quantize_custom(x, cb, B)
        c2, a2 = oracle.quantize_blockwise(x, oracle.DYN8, B)
        assert np.array_equal(c1, c2) and np.array_equal(a1, a2)
        y1 = oracle.dequantize_custom(c1, a1, cb, B, x.size)
        y2 = oracle.dequantize_blockwise(c2, a2, oracle.DYN8, B, x.size)
        assert np.array_equal(y1, y2)


def test_quantile_code_of_a_uniform_grid_closed_form():
    # every chunk holds a shuffled copy of 0, 1, ..., L-1 with L = 257 k: the
    # order statistic at floor(j L / 257) is j k, so q_i = (i + 1/2) k and the
    # normalized code is (i + 1/2) / 255.5, whatever the chunking
    k = 16
    L = 257 * k
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.permutation(L) for _ in range(5)]).astype(np.float32)
    want = np.array([(i + 0.5) / 255.5 for i in range(256)], dtype=np.float32)
    for chunk in (L, 2 * L):
        got = oracle.estimate_quantiles(x, chunk=chunk)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), chunk


def _chunk_stats(x, C):
    """Each chunk's order statistics s[floor(j L / 257)], j = 0..256, from
    numpy's sort (an independent library routine); -0 counts as +0."""
    x = np.where(x == 0, np.float32(0.0), x).astype(np.float32)
    out = []
    for lo in range(0, x.size, C):
        s = np.sort(x[lo:lo + C])
        L = s.size
        out.append([s[j * L // 257] for j in range(257)])
    return np.array(out, dtype=np.float32)


def _exact_means(E):
    """Exact rational mean of each column, rounded once to binary64 (CPython's
    int / int division is correctly rounded)."""
    nch = E.shape[0]
    A = []
    for j in range(E.shape[1]):
        s = sum((Fraction(float(v)) for v in E[:, j]), Fraction(0))
        A.append(s.numerator / (s.denominator * nch))
    return np.array(A, dtype=np.float64)


def _code_from_averages(A):
    q = [(A[i] + A[i + 1]) * 0.5 for i in range(256)]
    m = max(abs(v) for v in q)
    return np.array([np.float32(v / m) if m > 0 else np.float32(0.0) for v in q], dtype=np.float32)


def test_quantile_averages_are_exact_means_beyond_256_chunks():
    """601 chunks (the last ragged) of values spread over 2^-60 .. 2^60 with
    both signs, zeros and -0: every A_j equals the exact mean rounded once,
    while a plain binary64 sum in chunk order misses it for some j."""
    rng = np.random.default_rng(11)
    C = 257
    n = C * 600 + 100
    mag = np.ldexp(rng.uniform(1.0, 2.0, n), rng.integers(-60, 61, n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    x[rng.integers(0, n, 500)] = 0.0
    x[rng.integers(0, n, 500)] = -0.0
    E = _chunk_stats(x, C)
    assert E.shape[0] == 601
    want = _exact_means(E)
    got = oracle.quantile_averages(x, chunk=C)
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))
    naive = np.array([sum(float(v) for v in E[:, j]) / E.shape[0] for j in range(257)])
    assert np.any(naive != want), "the data must separate the exact mean from a plain sum"
    assert np.array_equal(oracle.estimate_quantiles(x, chunk=C).view(np.uint32),
                          _code_from_averages(want).view(np.uint32))


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_quantile_averages_of_16_bit_inputs(xdt):
    rng = np.random.default_rng(12)
    C = 300
    x32 = (rng.standard_t(3, C * 270 + 17) * 0.02).astype(np.float32)
    if xdt == "f16":
        h = x32.astype(np.float16)
        bits, dt, widened = h.view(np.uint16), oracle.F16, h.astype(np.float32)
    else:
        bits = oracle.f32_to_bf16_bits(x32)
        dt = oracle.BF16
        widened = (bits.astype(np.uint32) << 16).view(np.float32)
    want = _exact_means(_chunk_stats(widened, C))
    got = oracle.quantile_averages(bits, chunk=C, xdt=dt)
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


def test_quantile_average_rounding_and_order():
    C = 257
    one = np.full(C, 1.0, np.float32)
    # (1 + 2^-53) / 2 = 0.5 + 2^-54 lies halfway between 0.5 and its successor: to even, 0.5
    A = oracle.quantile_averages(np.concatenate([one, np.full(C, 2.0 ** -53, np.float32)]), chunk=C)
    assert np.all(A == 0.5)
    # (1 + 3 2^-53) / 2 = 0.5 + 1.5 ulp: halfway between 0.5 + 1 ulp (odd) and 0.5 + 2 ulp (even)
    A = oracle.quantile_averages(np.concatenate([one, np.full(C, 3 * 2.0 ** -53, np.float32)]), chunk=C)
    assert np.all(A == 0.5 + 2.0 ** -52)
    # 2^60, 2^-60, -2^60 in this chunk order: a running binary64 sum loses 2^-60
    big, tiny = np.float32(2.0 ** 60), np.float32(2.0 ** -60)
    x = np.concatenate([np.full(C, big), np.full(C, tiny), np.full(C, -big)]).astype(np.float32)
    A = oracle.quantile_averages(x, chunk=C)
    assert np.all(A == float(Fraction(2) ** -60 / 3))
    # means cancel exactly to zero: every entry of the code is then 0
    x = np.concatenate([np.full(C, big), np.full(C, -big)]).astype(np.float32)
    assert np.all(oracle.quantile_averages(x, chunk=C) == 0.0)
    assert np.all(oracle.estimate_quantiles(x, chunk=C) == 0.0)


def test_quantile_code_invariances():
    rng = np.random.default_rng(8)
    C = oracle.QUANTILE_CHUNK
    x = (rng.standard_normal(C * 6 + 1000) * 0.03).astype(np.float32)
    base = oracle.estimate_quantiles(x)
    assert np.all(np.diff(base.astype(np.float64)) >= 0) and np.max(np.abs(base)) == 1.0
    # order within a chunk does not matter
    xp = x.copy()
    for c in range(0, x.size, C):
        xp[c:c + C] = rng.permutation(xp[c:c + C])
    assert np.array_equal(oracle.estimate_quantiles(xp), base)
    # a power-of-two scale cancels in the normalization
    assert np.array_equal(oracle.estimate_quantiles((x * np.float32(8.0)).astype(np.float32)), base)
    # chunks are equal-weighted: two identical chunks give the one chunk's code
    one = x[:C]
    assert np.array_equal(oracle.estimate_quantiles(np.concatenate([one, one])), oracle.estimate_quantiles(one))


def test_quantile_code_of_a_normal_sample_tracks_normal_quantiles():
    """Statistical sanity (not a pin of the bits): on N(0,1) data the entries
    away from the extremes are proportional to the midpoints of the normal
    quantiles at j/257."""
    from scipy.stats import norm
    x = np.random.default_rng(9).standard_normal(4096 * 64).astype(np.float32)
    got = oracle.estimate_quantiles(x).astype(np.float64)
    q = norm.ppf(np.arange(1, 257) / 257.0)
    mid = (q[:-1] + q[1:]) / 2                              # entries 1..254
    inner = slice(8, 246)
    g = got[1:255][inner]
    m = mid[inner]
    scale = np.dot(g, m) / np.dot(m, m)
    assert np.max(np.abs(g - scale * m)) < 0.01


def test_zero_data_gives_the_zero_code_and_zero_blocks():
    cb = oracle.estimate_quantiles(np.zeros(5000, np.float32))
    assert np.all(cb == 0.0)
    codes, absmax = oracle.quantize_custom(np.zeros(100, np.float32), oracle.linear_codebook(), 64)
    assert np.all(codes == 128) and np.all(absmax == 0.0)
