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
QB_DT = {oracle.F32: 0, oracle.F16: 1, oracle.BF16: 2}
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


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("B", [64, 4096])
def test_multi_tensor_dequantize_equals_oracle(code, nested, B):
    """One grouped launch over many tensors (ragged, tiny, empty, several tiles)
    equals the oracle tensor by tensor; bytes past each output stay untouched."""
    from gpu_helpers import qb
    L = qb()
    rng = np.random.default_rng(300 + 10 * code + B + nested)
    sizes = [8192 * 3 + 77, 1, 0, 65, 8192, 64 * 256 * 3 + 5, 2, 4097, 0, 8191] + \
        [int(v) for v in rng.integers(1, 20000, 40)]
    ydt = oracle.BF16
    keep, entries, wants = [], [], []
    for i, n in enumerate(sizes):
        x = (rng.standard_normal(max(n, 1)) * 0.02).astype(np.float32)[:n]
        codes, absmax = oracle.quantize_blockwise(x, code, B) if n else (np.zeros(0, np.uint8), np.zeros(0, np.float32))
        y = torch.full((n + 8,), 7.0, dtype=TORCH_DT[ydt], device=DEV)
        cd = to_device(codes if codes.size else np.zeros(1, np.uint8))
        if nested:
            c2, a2, mu = oracle.dq_quantize(absmax, 256) if n else (np.zeros(1, np.uint8), np.zeros(1, np.float32),
                                                                     np.float32(0))
            st = {"c2": to_device(c2 if c2.size else np.zeros(1, np.uint8)),
                  "a2": to_device(a2 if a2.size else np.zeros(1, np.float32)),
                  "off": to_device(np.array([mu, 0, 0, 0], np.float32))}
            dq = L.make_dq(st["c2"], st["a2"], st["off"], 256)
            keep.append((cd, st, y))
            entries.append((cd, None, dq, n, y))
            want = oracle.dequantize(codes, {"c2": c2, "absmax2": a2, "mu": mu}, code, B, n, ydt) if n else None
        else:
            ad = to_device(absmax if absmax.size else np.zeros(1, np.float32))
            keep.append((cd, ad, y))
            entries.append((cd, ad, None, n, y))
            want = oracle.dequantize_blockwise(codes, absmax, code, B, n, ydt) if n else None
        wants.append(want)
    table = L.dequant_table(entries)
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    L.qb_multi_tensor_dequantize(table, len(sizes), code, B, 256, L.QB_BF16, ws)
    torch.cuda.synchronize()
    sentinel = torch.full((8,), 7.0, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for (n, want, (_, _, y)) in zip(sizes, wants, keep):
        got = host_bits(y)
        if n:
            assert np.array_equal(got[:n], want), f"tensor of {n} differs"
        assert np.array_equal(got[n:], sentinel), f"tensor of {n}: wrote past its end"


def test_multi_tensor_dequantize_rejects_mixed_nesting():
    from gpu_helpers import qb
    L = qb()
    n = 1000
    codes = torch.zeros(n, dtype=torch.uint8, device=DEV)
    absmax = torch.ones(16, device=DEV)
    c2 = torch.zeros(16, dtype=torch.uint8, device=DEV)
    a2 = torch.ones(4, device=DEV)
    off = torch.zeros(4, device=DEV)
    y = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    dq = L.make_dq(c2, a2, off, 256)
    table = L.dequant_table([(codes, absmax, None, n, y), (codes, None, dq, n, y)])
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(2), dtype=torch.uint8, device=DEV)
    with pytest.raises(L.QbError) as e:
        L.qb_multi_tensor_dequantize(table, 2, L.QB_DYN8, 64, 256, L.QB_BF16, ws)
    assert e.value.status == L.QB_EUNSUPPORTED


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("B,dt", [(64, oracle.F16), (4096, oracle.F32), (256, oracle.BF16)])
def test_multi_tensor_quantize_equals_oracle(code, nested, B, dt):
    """One grouped call over many tensors (ragged, tiny, empty, several tiles)
    gives every tensor's codes, absmax or nested state exactly as the oracle;
    bytes past each output stay untouched."""
    from gpu_helpers import qb
    L = qb()
    rng = np.random.default_rng(500 + 10 * code + B + nested + 3 * dt)
    sizes = [8192 * 3 + 77, 1, 0, 65, 8192, 64 * 256 * 3 + 5, 2, 4097, 0, 8191] + \
        [int(v) for v in rng.integers(1, 30000, 30)]
    bufs, entries, xs = [], [], []
    for i, n in enumerate(sizes):
        xh, _ = make_input(max(n, 1), B, dt, seed=7000 + i)
        xh = xh[:n]
        xs.append(xh)
        nb = (n + B - 1) // B
        xd = dev(xh if n else np.zeros(1, xh.dtype), dt)
        codes = torch.full((packed_len(code, n) + 16,), 0xAB, dtype=torch.uint8, device=DEV)
        if nested:
            c2 = torch.full((nb + 16,), 0xAB, dtype=torch.uint8, device=DEV)
            a2 = torch.full(((nb + 255) // 256 + 4,), -7.0, dtype=torch.float32, device=DEV)
            off = torch.full((4,), -7.0, dtype=torch.float32, device=DEV)
            dq = L.make_dq(c2, a2, off, 256)
            bufs.append((xd, codes, c2, a2, off))
            entries.append((xd, n, codes, None, dq))
        else:
            am = torch.full((nb + 4,), -7.0, dtype=torch.float32, device=DEV)
            bufs.append((xd, codes, am))
            entries.append((xd, n, codes, am, None))
    table = L.quant_table(entries)
    wsb = L.qb_multi_tensor_quantize_workspace_bytes(table, len(sizes), B)
    ws = torch.full((wsb,), 0xCD, dtype=torch.uint8, device=DEV)
    L.qb_multi_tensor_quantize(table, len(sizes), QB_DT[dt], code, B, 256, ws)
    torch.cuda.synchronize()
    for n, xh, b in zip(sizes, xs, bufs):
        nb = (n + B - 1) // B
        got_c = b[1].cpu().numpy()
        pl = packed_len(code, n)
        assert np.all(got_c[pl:] == 0xAB), f"tensor of {n}: codes written past the end"
        if not n:
            continue
        want_c, want_a = oracle.quantize_blockwise(xh, code, B, dt)
        assert np.array_equal(got_c[:pl], want_c), f"tensor of {n}: codes differ"
        if nested:
            c2, a2, mu = oracle.dq_quantize(want_a, 256)
            got_c2, got_a2, got_off = b[2].cpu().numpy(), b[3].cpu().numpy(), b[4].cpu().numpy()
            assert np.float32(got_off[0]).view(np.uint32) == np.float32(mu).view(np.uint32), f"mean of {n}"
            assert np.array_equal(got_c2[:nb], c2) and np.all(got_c2[nb:] == 0xAB)
            k2 = (nb + 255) // 256
            assert np.array_equal(got_a2[:k2].view(np.uint32), a2.view(np.uint32)) and np.all(got_a2[k2:] == -7.0)
        else:
            got_a = b[2].cpu().numpy()
            assert np.array_equal(got_a[:nb].view(np.uint32), want_a.view(np.uint32)) and np.all(got_a[nb:] == -7.0)


def test_multi_tensor_quantize_twice_reuses_workspace():
    """A second grouped nested call on the same (dirty) workspace gives the same
    result: the exponent bins are cleared by every call."""
    from gpu_helpers import qb
    L = qb()
    sizes = [64 * 1000 + 3, 8192 * 5, 777]
    xs = [dev(make_input(n, 64, oracle.F16, seed=40 + n)[0], oracle.F16) for n in sizes]
    outs = []
    for rep in range(2):
        entries, keep = [], []
        for x, n in zip(xs, sizes):
            nb = (n + 63) // 64
            codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=DEV)
            c2 = torch.empty(nb, dtype=torch.uint8, device=DEV)
            a2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=DEV)
            off = torch.empty(4, dtype=torch.float32, device=DEV)
            keep.append((codes, c2, a2, off))
            entries.append((x, n, codes, None, L.make_dq(c2, a2, off, 256)))
        table = L.quant_table(entries)
        if rep == 0:
            ws = torch.empty(L.qb_multi_tensor_quantize_workspace_bytes(table, len(sizes), 64), dtype=torch.uint8,
                             device=DEV)
        L.qb_multi_tensor_quantize(table, len(sizes), L.QB_F16, L.QB_NF4, 64, 256, ws)
        torch.cuda.synchronize()
        outs.append([tuple(t.cpu().numpy().tobytes() for t in k) for k in keep])
    assert outs[0] == outs[1]
