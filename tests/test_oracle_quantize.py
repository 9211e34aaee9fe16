"""Pins of the oracle's block-wise quantize / dequantize (CPU only).

What the pages fix, and what is checked here:
  - blocks are quantized independently (abstract quoted on "Py之bitsandbytes",
    section 2; "bitsandbytes深度解析", section 核心量化原理与实现机制): permuting
    whole blocks permutes codes and absmax the same way;
  - each block is scaled by its own absmax: scaling x by 2^k leaves every code
    unchanged and scales the absmax by 2^k;
  - the nearest-code rule bounds the round-trip error by the local half-gap;
  - two 4-bit codes share a byte (0.5 byte per parameter, "bitsandbytes -
    Quantização de LLM", section Etapa 1).
Conversions to bfloat16 / float16 are pinned against torch / numpy.
"""
import numpy as np
import pytest
import torch

import oracle

CODES = [oracle.DYN8, oracle.NF4, oracle.FP4]
MAX_HALF_GAP = {oracle.DYN8: 0.00703126, oracle.NF4: 0.1519, oracle.FP4: 1 / 6 + 1e-7}


def student_t(rng, n, scale=0.02):
    return (rng.standard_t(3, n) * scale).astype(np.float32)


def unpack4(codes, n):
    hi = codes >> 4
    lo = codes & 15
    return np.stack([hi, lo], axis=1).reshape(-1)[:n]


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("B", [64, 256, 2048])
def test_block_permutation(code, B):
    rng = np.random.default_rng(7)
    nb = 12
    x = student_t(rng, nb * B)
    c, a = oracle.quantize_blockwise(x, code, B)
    perm = rng.permutation(nb)
    xp = x.reshape(nb, B)[perm].reshape(-1)
    cp, ap = oracle.quantize_blockwise(xp, code, B)
    per = B // 2 if code != oracle.DYN8 else B
    assert np.array_equal(ap, a[perm])
    assert np.array_equal(cp.reshape(nb, per), c.reshape(nb, per)[perm])


@pytest.mark.parametrize("code", CODES)
def test_power_of_two_scale_invariance(code):
    rng = np.random.default_rng(8)
    x = student_t(rng, 64 * 37 + 5)
    c, a = oracle.quantize_blockwise(x, code, 64)
    for k in (-20, -3, 5, 30):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        cs, as_ = oracle.quantize_blockwise(xs, code, 64)
        assert np.array_equal(cs, c)
        assert np.array_equal(as_, (a * np.float32(2.0 ** k)).astype(np.float32))


def test_negation_symmetry():
    rng = np.random.default_rng(9)
    x = student_t(rng, 256 * 20)
    # FP4: sign-magnitude, exact mirror
    c, _ = oracle.quantize_blockwise(x, oracle.FP4, 64)
    cn, _ = oracle.quantize_blockwise(-x, oracle.FP4, 64)
    e, en = unpack4(c, x.size), unpack4(cn, x.size)
    nz = (e & 7) != 0
    assert np.array_equal(en[nz], e[nz] ^ 8) and np.array_equal(en[~nz], e[~nz])
    # DYN8: index 127+k <-> 127-k, except +1.0 (index 255), whose mirror is index 0
    c, a = oracle.quantize_blockwise(x, oracle.DYN8, 256)
    cn, an = oracle.quantize_blockwise(-x, oracle.DYN8, 256)
    assert np.array_equal(a, an)
    c = c.astype(np.int64)
    want = np.where(c == 255, 0, 254 - c)
    want = np.where(c == 127, 127, want)
    got = cn.astype(np.int64)
    # an element that maps to 0 (-0.99296874) under negation came from a value near -1
    neg_top = (c == 0)
    assert np.array_equal(got[~neg_top], want[~neg_top])


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("B", [64, 512, 4096])
def test_round_trip_bound(code, B):
    rng = np.random.default_rng(10 + B)
    n = B * 9 + 17
    x = student_t(rng, n)
    x[B:2 * B] = 0.0                                   # an all-zero block
    codes, a = oracle.quantize_blockwise(x, code, B)
    y = oracle.dequantize_blockwise(codes, a, code, B, n)
    scale = np.repeat(a, B)[:n].astype(np.float64)
    err = np.abs(x.astype(np.float64) - y.astype(np.float64))
    bound = scale * (MAX_HALF_GAP[code] + 2.0 ** -24) + np.abs(np.spacing(y)).astype(np.float64)
    assert np.all(err <= bound)
    assert np.all(y[B:2 * B] == 0.0) and a[1] == 0.0


def test_positive_block_max_maps_to_one():
    rng = np.random.default_rng(11)
    x = np.abs(student_t(rng, 2048 * 4))
    c, a = oracle.quantize_blockwise(x, oracle.DYN8, 2048)
    for b in range(4):
        blk = x[b * 2048:(b + 1) * 2048]
        i = int(np.argmax(blk))
        assert c[b * 2048 + i] == 255 and a[b] == blk[i]


@pytest.mark.parametrize("code", CODES)
def test_idempotence(code):
    rng = np.random.default_rng(12)
    n = 64 * 50
    x = student_t(rng, n)
    B = 64
    if code == oracle.DYN8:
        # idempotent when every block's largest magnitude is positive
        xb = x.reshape(-1, B)
        i = np.argmax(np.abs(xb), axis=1)
        xb[np.arange(xb.shape[0]), i] = np.abs(xb[np.arange(xb.shape[0]), i])
        x = xb.reshape(-1)
    c1, a1 = oracle.quantize_blockwise(x, code, B)
    y = oracle.dequantize_blockwise(c1, a1, code, B, n)
    c2, a2 = oracle.quantize_blockwise(y, code, B)
    assert np.array_equal(c1, c2) and np.array_equal(a1, a2)


def test_odd_length_4bit_padding_and_nibble_order():
    x = np.array([1.0, -1.0, 0.0], dtype=np.float32)
    c, a = oracle.quantize_blockwise(x, oracle.NF4, 64)
    assert a[0] == 1.0
    assert c.size == 2
    assert c[0] == (15 << 4) | 0       # element 0 -> high nibble (+1 = index 15), element 1 -> low (-1 = 0)
    assert c[1] == (7 << 4)            # element 2 -> 0.0 = index 7; padding nibble 0


@pytest.mark.parametrize("code", CODES)
def test_dequantize_closed_form(code):
    rng = np.random.default_rng(13)
    n = 1000
    K = 256 if code == oracle.DYN8 else 16
    cidx = rng.integers(0, K, n).astype(np.uint8)
    packed = cidx if code == oracle.DYN8 else ((cidx[0::2] << 4) | cidx[1::2]).astype(np.uint8)
    scale = rng.uniform(0.01, 3, (n + 63) // 64).astype(np.float32)
    y = oracle.dequantize_blockwise(packed, scale, code, 64, n)
    table = oracle.codebook(code)
    want = (table[cidx] * np.repeat(scale, 64)[:n]).astype(np.float32)    # numpy binary32 multiply
    assert np.array_equal(y, want)
    # bfloat16 output: round-to-nearest-even of the same product (torch's conversion)
    yb = oracle.dequantize_blockwise(packed, scale, code, 64, n, oracle.BF16)
    tb = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)
    yh = oracle.dequantize_blockwise(packed, scale, code, 64, n, oracle.F16)
    assert np.array_equal(yh, want.astype(np.float16).view(np.uint16))


def test_conversions_against_library_routines():
    rng = np.random.default_rng(14)
    x = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-6).astype(np.float32),      # float16 subnormals
        (rng.standard_normal(1000) * 3e4).astype(np.float32),       # near float16 max
        np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 6.1035156e-05, 5.96e-08, 2.98e-08, 1.0 + 2 ** -8,
                  1.0 + 3 * 2 ** -8], dtype=np.float32),
    ])
    # ties in bfloat16: low 16 bits exactly 0x8000
    ties = (rng.integers(0, 2 ** 15, 500).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    bf = oracle.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, tb)
    h = oracle.f32_to_f16_bits(x)
    assert np.array_equal(h, x.astype(np.float16).view(np.uint16))
    allh = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    finite = ~np.isnan(allh.view(np.float16)) & ~np.isinf(allh.view(np.float16))
    back = oracle.f16_bits_to_f32(allh[finite])
    assert np.array_equal(back, allh[finite].view(np.float16).astype(np.float32))


@pytest.mark.parametrize("xdt", [oracle.F16, oracle.BF16])
def test_half_inputs_equal_their_float32_widening(xdt):
    rng = np.random.default_rng(15)
    xf = student_t(rng, 64 * 20 + 3)
    if xdt == oracle.F16:
        bits = xf.astype(np.float16).view(np.uint16)
        wide = bits.view(np.float16).astype(np.float32)
    else:
        bits = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        wide = (bits.astype(np.uint32) << 16).view(np.float32)
    for code in CODES:
        c1, a1 = oracle.quantize_blockwise(bits, code, 64, xdt)
        c2, a2 = oracle.quantize_blockwise(wide, code, 64)
        assert np.array_equal(c1, c2) and np.array_equal(a1, a2)
