"""GPU parity: libqb block-wise quantize / dequantize / nested quantization
against the CPU oracle, element by element, bit-exact (codes, absmax, nested
state and every dequantized output, in every output dtype)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, decorate, gpu_dequantize, gpu_quantize, host_bits, packed_len, to_device

pytestmark = pytest.mark.gpu

CODES = [oracle.DYN8, oracle.NF4, oracle.FP4]
BLOCKS = [64, 128, 256, 512, 1024, 2048, 4096]


def make_input(n, B, dt, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, n) * 0.02).astype(np.float32)
    x = decorate(x, B, dt, rng)
    if dt == oracle.F32:
        return x, x
    t = torch.from_numpy(x).to(TORCH_DT[dt])
    return t.view(torch.int16).numpy().view(np.uint16).copy(), t


def dev(xh, dt):
    return to_device(xh, TORCH_DT[dt])


def check_quantize(code, B, dt, n, seed, double_quant=False):
    xh, _ = make_input(n, B, dt, seed)
    xd = dev(xh, dt)
    want_c, want_a = oracle.quantize_blockwise(xh, code, B, dt)
    got_c, got_s = gpu_quantize(xd, code, B, double_quant)
    assert np.array_equal(got_c, want_c), f"codes differ at {np.flatnonzero(got_c != want_c)[:10]}"
    if not double_quant:
        assert np.array_equal(got_s.view(np.uint32), want_a.view(np.uint32))
        return xh, got_c, got_s
    c2, a2, mu = oracle.dq_quantize(want_a, 256)
    assert np.float32(got_s["mu"]).view(np.uint32) == np.float32(mu).view(np.uint32)
    assert np.array_equal(got_s["c2"], c2)
    assert np.array_equal(got_s["absmax2"].view(np.uint32), a2.view(np.uint32))
    assert np.all(got_s["a2_tail"] == -7.0), "wrote past absmax2"
    return xh, got_c, got_s


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("B", BLOCKS)
def test_quantize_parity_fp32(code, B):
    for n in (3 * 4096 * 4 + 37, 1 << 16, 123457):
        check_quantize(code, B, oracle.F32, n, seed=B * 7 + code + n)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("B", [64, 256, 2048, 4096])
def test_quantize_parity_half(code, dt, B):
    check_quantize(code, B, dt, 5 * 8192 + 1001, seed=B + dt * 11 + code)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, 127, 4095, 4097])
def test_quantize_small_and_ragged(code, n):
    for B in (64, 4096):
        check_quantize(code, B, oracle.F32, n, seed=n + B)


@pytest.mark.parametrize("code", CODES)
def test_quantize_zero_length_is_noop(code):
    from gpu_helpers import qb
    L = qb()
    x = torch.zeros(16, device=DEV)
    codes = torch.full((16,), 0xAB, dtype=torch.uint8, device=DEV)
    absmax = torch.full((1,), -7.0, device=DEV)
    L.qb_quantize(x, 0, code, 64, codes, absmax)
    torch.cuda.synchronize()
    assert torch.all(codes == 0xAB) and absmax.item() == -7.0


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("ydt", [oracle.F32, oracle.F16, oracle.BF16])
@pytest.mark.parametrize("B", [64, 512, 4096])
def test_dequantize_parity(code, ydt, B):
    n = 3 * 8192 + 777
    xh, _ = make_input(n, B, oracle.F32, seed=B + ydt)
    codes, absmax = oracle.quantize_blockwise(xh, code, B)
    got = gpu_dequantize(codes, absmax, code, B, n, ydt)
    want = oracle.dequantize_blockwise(codes, absmax, code, B, n, ydt)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("code", CODES)
def test_dequantize_arbitrary_codes(code):
    """Every code value (including FP4's negative zero) decodes like the oracle."""
    rng = np.random.default_rng(77)
    n = 8192 * 3 + 5
    codes = rng.integers(0, 256, packed_len(code, n)).astype(np.uint8)
    absmax = rng.uniform(0, 2, (n + 63) // 64).astype(np.float32)
    for ydt in (oracle.F32, oracle.BF16, oracle.F16):
        got = gpu_dequantize(codes, absmax, code, 64, n, ydt)
        want = oracle.dequantize_blockwise(codes, absmax, code, 64, n, ydt)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("B", [64, 256])
@pytest.mark.parametrize("dt", [oracle.F32, oracle.F16])
def test_nested_quantization_parity(code, B, dt):
    n = 64 * 256 * 7 + 3 * 64 + 11        # several second-level blocks and a ragged tail
    xh, got_c, got_s = check_quantize(code, B, dt, n, seed=900 + B + code, double_quant=True)
    for ydt in (oracle.BF16, oracle.F32):
        got = gpu_dequantize(got_c, got_s, code, B, n, ydt)
        want_c, want_a = oracle.quantize_blockwise(xh, code, B, dt)
        c2, a2, mu = oracle.dq_quantize(want_a, 256)
        want = oracle.dequantize(want_c, {"c2": c2, "absmax2": a2, "mu": mu}, code, B, n, ydt)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_nested_mean_wide_dynamic_range():
    """Absmax values spread over ~60 binades: the fp64 sum would not be exact,
    the exact mean must still match."""
    rng = np.random.default_rng(5)
    nblk = 3000
    scale = np.exp(rng.uniform(-20, 20, nblk)).astype(np.float32)
    x = (rng.standard_normal(nblk * 64).astype(np.float32) * np.repeat(scale, 64)).astype(np.float32)
    _, want_a = oracle.quantize_blockwise(x, oracle.NF4, 64)
    got_c, got_s = gpu_quantize(to_device(x), oracle.NF4, 64, double_quant=True)
    c2, a2, mu = oracle.dq_quantize(want_a, 256)
    assert np.float32(got_s["mu"]) == mu
    assert np.array_equal(got_s["c2"], c2) and np.array_equal(got_s["absmax2"], a2)
