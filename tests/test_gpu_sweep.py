"""GPU parity sweep: every kernel instantiation the library compiles runs at
least once against the CPU oracle, at small ragged sizes.

The kernels are templates over block size, data types, code width, nesting,
grouping, optimizer kind, m-tiles and K alignment.  The other GPU test files
check each of those dimensions in depth; this file walks every combination
that is compiled:

- quantize and dequantize for every code, block size, input and output dtype,
  plain and nested (every second-level block size), one tensor and grouped;
- the user-code kernels for every block size and dtype, and the quantile
  estimator for every input dtype;
- every optimizer kind at every block size and (gradient, parameter) dtype
  pair, one tensor and grouped (the layer-wise kinds are grouped only), and
  the kinds with a never-negative state again with it in the unsigned code;
- the fused 4-bit product for every compute dtype, absmax form, m-tile count
  and K alignment.

The bar is the other files' bar: codes, absmax, nested state, optimizer
states and dequantized outputs bit-exact, nothing written past an output;
parameters bit-exact except AdamW and LAMB (binary32: 1e-6 relative;
16-bit: one ulp per step, the oracle stepping from the device's
parameters); products within the binary32 summation bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, packed_len, qb, to_device
from test_gpu_matmul import check as mm_check
from test_gpu_matmul import make_case as mm_case
from test_gpu_matmul import run_gpu as mm_run
from test_gpu_param_dtypes import KINDS, LAYERWISE, check_params, lib_hp

pytestmark = pytest.mark.gpu

BLOCKS = [64, 128, 256, 512, 1024, 2048, 4096]
DTYPES = [oracle.F32, oracle.F16, oracle.BF16]
CODES = [oracle.DYN8, oracle.NF4, oracle.FP4]
SENT_CODE, SENT_F32 = 0xAB, -7.0


def host_values(n, dt, rng, scale):
    """n Student-t(3) values times scale in dtype dt (16-bit types as uint16 bits)."""
    x = (rng.standard_t(3, max(n, 1)) * scale).astype(np.float32)[:n]
    if dt == oracle.F32:
        return x
    return torch.from_numpy(x).to(TORCH_DT[dt]).view(torch.int16).numpy().view(np.uint16).copy()


def dev_or_dummy(a, dt=None):
    return to_device(a if a.size else np.zeros(1, a.dtype), dt)


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------

def gpu_quantize_all(L, xs, xdt, code, B, nested, B2, multi):
    """Quantize every host array of xs (one call each, or one grouped call);
    returns per tensor the device buffers (codes, absmax) or (codes, c2, a2, off)."""
    bufs, entries = [], []
    for x in xs:
        n = x.size
        nb = -(-n // B)
        xd = dev_or_dummy(x, TORCH_DT[xdt])
        codes = torch.full((packed_len(code, n) + 8,), SENT_CODE, dtype=torch.uint8, device=DEV)
        if nested:
            c2 = torch.full((nb + 8,), SENT_CODE, dtype=torch.uint8, device=DEV)
            a2 = torch.full((-(-nb // B2) + 4,), SENT_F32, dtype=torch.float32, device=DEV)
            off = torch.full((4,), SENT_F32, dtype=torch.float32, device=DEV)
            if multi:
                dq = L.make_dq(c2, a2, off, B2)
            else:
                ws = torch.empty(max(L.qb_dq_workspace_bytes(n, B), 1), dtype=torch.uint8, device=DEV)
                dq = L.make_dq(c2, a2, off, B2, ws)
                L.qb_quantize(xd, n, code, B, codes, None, dq)
            bufs.append((xd, codes, c2, a2, off))
            entries.append((xd, n, codes, None, dq))
        else:
            am = torch.full((nb + 4,), SENT_F32, dtype=torch.float32, device=DEV)
            if not multi:
                L.qb_quantize(xd, n, code, B, codes, am)
            bufs.append((xd, codes, am))
            entries.append((xd, n, codes, am, None))
    if multi:
        table = L.quant_table(entries)
        ws = torch.empty(L.qb_multi_tensor_quantize_workspace_bytes(table, len(xs), B), dtype=torch.uint8, device=DEV)
        L.qb_multi_tensor_quantize(table, len(xs), xdt, code, B, B2, ws)
    torch.cuda.synchronize()
    return bufs


def check_quantized(x, b, code, B, xdt, nested, B2, what):
    """The device codes and absmax (or nested state) equal the oracle's; returns
    the oracle's codes and state (absmax, or the nested dict)."""
    n = x.size
    nb = -(-n // B)
    pl = packed_len(code, n)
    got_c = b[1].cpu().numpy()
    assert np.all(got_c[pl:] == SENT_CODE), f"{what}: codes written past the end"
    if not n:
        return None, None
    want_c, want_a = oracle.quantize_blockwise(x, code, B, xdt)
    assert np.array_equal(got_c[:pl], want_c), f"{what}: codes differ at {np.flatnonzero(got_c[:pl] != want_c)[:8]}"
    if not nested:
        got_a = b[2].cpu().numpy()
        assert np.array_equal(got_a[:nb].view(np.uint32), want_a.view(np.uint32)), f"{what}: absmax"
        assert np.all(got_a[nb:] == SENT_F32), f"{what}: absmax written past the end"
        return want_c, want_a
    c2, a2, mu = oracle.dq_quantize(want_a, B2)
    k2 = -(-nb // B2)
    got_c2, got_a2, got_off = b[2].cpu().numpy(), b[3].cpu().numpy(), b[4].cpu().numpy()
    assert np.float32(got_off[0]).view(np.uint32) == np.float32(mu).view(np.uint32), f"{what}: nested mean"
    assert np.array_equal(got_c2[:nb], c2) and np.all(got_c2[nb:] == SENT_CODE), f"{what}: nested codes"
    assert np.array_equal(got_a2[:k2].view(np.uint32), a2.view(np.uint32)), f"{what}: nested absmax"
    assert np.all(got_a2[k2:] == SENT_F32), f"{what}: nested absmax written past the end"
    return want_c, {"c2": c2, "absmax2": a2, "mu": mu}


def gpu_dequantize_all(L, bufs, sizes, code, B, nested, B2, multi, ydt):
    """Dequantize every tensor from its device codes and state into ydt (one call
    each, or one grouped call); returns the host outputs with 8 sentinels each."""
    ys, entries, keep = [], [], []
    for b, n in zip(bufs, sizes):
        y = torch.full((n + 8,), 7.0, dtype=TORCH_DT[ydt], device=DEV)
        if nested:
            dq = L.make_dq(b[2], b[3], b[4], B2)
            keep.append(dq)
            if not multi:
                L.qb_dequantize(b[1], None, dq, code, B, n, y)
            entries.append((b[1], None, dq, n, y))
        else:
            if not multi:
                L.qb_dequantize(b[1], b[2], None, code, B, n, y)
            entries.append((b[1], b[2], None, n, y))
        ys.append(y)
    if multi:
        table = L.dequant_table(entries)
        ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
        L.qb_multi_tensor_dequantize(table, len(sizes), code, B, B2, ydt, ws)
    torch.cuda.synchronize()
    return [host_bits(y) for y in ys]


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("xdt", DTYPES)
def test_quantize_dequantize_every_instantiation(code, xdt):
    L = qb()
    rng = np.random.default_rng(100 + 10 * code + xdt)
    sentinel = {dt: host_bits(torch.full((8,), 7.0, dtype=TORCH_DT[dt])) for dt in DTYPES}
    for bi, B in enumerate(BLOCKS):
        for nested in (False, True):
            # over the block-size loop every second-level block size comes up
            B2 = BLOCKS[(bi + code + 3 * nested) % len(BLOCKS)]
            for multi in (False, True):
                sizes = [2 * B + 3, 1, 0, B + 1, 5 * B + 7] if multi else [3 * B + 17]
                what = f"code={code} xdt={xdt} B={B} nested={nested} B2={B2} multi={multi}"
                xs = [host_values(n, xdt, rng, 0.02) for n in sizes]
                bufs = gpu_quantize_all(L, xs, xdt, code, B, nested, B2, multi)
                wants = [check_quantized(x, b, code, B, xdt, nested, B2, f"{what} tensor {i}")
                         for i, (x, b) in enumerate(zip(xs, bufs))]
                for ydt in DTYPES:
                    ys = gpu_dequantize_all(L, bufs, sizes, code, B, nested, B2, multi, ydt)
                    for i, (n, (wc, ws), y) in enumerate(zip(sizes, wants, ys)):
                        assert np.array_equal(y[n:], sentinel[ydt]), f"{what} ydt={ydt} tensor {i}: wrote past its end"
                        if not n:
                            continue
                        want = oracle.dequantize(wc, ws, code, B, n, ydt, blocksize2=B2)
                        assert np.array_equal(y[:n].view(np.uint8), want.view(np.uint8)), \
                            f"{what} ydt={ydt} tensor {i}: output differs"


@pytest.mark.parametrize("xdt", DTYPES)
def test_user_code_and_quantile_kernels_every_instantiation(xdt):
    L = qb()
    rng = np.random.default_rng(200 + xdt)
    x_est = host_values(4096 * 3 + 5, xdt, rng, 0.02)
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    ws = torch.empty(L.qb_quantile_workspace_bytes(x_est.size), dtype=torch.uint8, device=DEV)
    avg = torch.empty(257, dtype=torch.float64, device=DEV)
    L.qb_estimate_quantiles(to_device(x_est, TORCH_DT[xdt]), x_est.size, t, ws, averages=avg)
    torch.cuda.synchronize()
    cb = t.cpu().numpy().view(np.float32)[:256].copy()
    assert np.array_equal(cb.view(np.uint32), oracle.estimate_quantiles(x_est, xdt=xdt).view(np.uint32)), \
        f"xdt={xdt}: estimated quantile code"
    assert np.array_equal(avg.cpu().numpy().view(np.uint64),
                          oracle.quantile_averages(x_est, xdt=xdt).view(np.uint64)), f"xdt={xdt}: averages"
    for B in BLOCKS:
        n = 3 * B + 17
        nb = -(-n // B)
        x = host_values(n, xdt, rng, 0.02)
        codes = torch.full((n + 8,), SENT_CODE, dtype=torch.uint8, device=DEV)
        absmax = torch.full((nb + 4,), SENT_F32, device=DEV)
        L.qb_quantize_code(to_device(x, TORCH_DT[xdt]), n, t, B, codes, absmax)
        want_c, want_a = oracle.quantize_custom(x, cb, B, xdt)
        got_c, got_a = host_bits(codes), host_bits(absmax)
        what = f"xdt={xdt} B={B}"
        assert np.array_equal(got_c[:n], want_c) and np.all(got_c[n:] == SENT_CODE), f"{what}: codes"
        assert np.array_equal(got_a[:nb].view(np.uint32), want_a.view(np.uint32)), f"{what}: absmax"
        assert np.all(got_a[nb:] == SENT_F32), f"{what}: absmax written past the end"
        for ydt in DTYPES:
            y = torch.empty(n, dtype=TORCH_DT[ydt], device=DEV)
            L.qb_dequantize_code(codes, absmax, t, B, n, y)
            want = oracle.dequantize_custom(want_c, want_a, cb, B, n, ydt)
            assert np.array_equal(host_bits(y).view(np.uint8), want.view(np.uint8)), f"{what} ydt={ydt}: output"


# ---------------------------------------------------------------------------
# optimizers
# ---------------------------------------------------------------------------

# (gradient dtype, parameter dtype): binary32 parameters take any gradient
# dtype, 16-bit parameters a gradient of their own dtype
PAIRS = [(oracle.F32, oracle.F32), (oracle.F16, oracle.F32), (oracle.BF16, oracle.F32),
         (oracle.F16, oracle.F16), (oracle.BF16, oracle.BF16)]


# the kinds with a never-negative state also run with it in the unsigned code
NONNEG = ("adamw", "adam", "rmsprop", "lamb")
OPT_CASES = [(n, oracle.DYN8) for n in KINDS] + [(n, oracle.UDYN8) for n in NONNEG]


@pytest.mark.parametrize("name,vcode", OPT_CASES)
def test_optimizer_every_instantiation(name, vcode):
    kind, hp, exact = KINDS[name]
    L = qb()
    two = oracle.OPTIMIZER_STATES[kind] == 2
    rng = np.random.default_rng(300 + kind + 7 * vcode)
    zero = {oracle.DYN8: 127, oracle.UDYN8: 0}
    z1 = zero[vcode] if kind == oracle.RMSPROP else 127     # codes of 0.0 of state 1 and state 2
    z2 = zero[vcode]
    for B in BLOCKS:
        for gdt, pdt in PAIRS:
            for multi in ((True,) if name in LAYERWISE else (False, True)):
                sizes = [B + 5, 3 * B + 1, 1] if multi else [2 * B + 37]
                host, dev = [], []
                for n in sizes:
                    nb = -(-n // B)
                    h = [host_values(n, pdt, rng, 0.02), np.full(n, z1, np.uint8), np.zeros(nb, np.float32),
                         np.full(n, z2, np.uint8), np.zeros(nb, np.float32)]
                    host.append(h)
                    dev.append([to_device(h[0], TORCH_DT[pdt])] + [to_device(a) for a in h[1:]])
                for step in (1, 2):
                    gs = [host_values(n, gdt, rng, 1e-3) for n in sizes]
                    gd = [to_device(g, TORCH_DT[gdt]) for g in gs]
                    h = lib_hp(kind, hp, step)
                    h.v_code = vcode
                    if multi:
                        table = L.tensor_table([(d[0], g, d[1], d[3] if two else None, d[2], d[4] if two else None)
                                                for d, g in zip(dev, gd)])
                        ws = torch.empty(L.qb_optimizer_workspace_bytes(h, table, len(sizes), B), dtype=torch.uint8,
                                         device=DEV)
                        L.qb_multi_tensor_optimizer_step(h, table, len(sizes), gdt, B, ws, pdt=pdt)
                    else:
                        d, g, n = dev[0], gd[0], sizes[0]
                        L.qb_optimizer8bit_step(h, d[0], g, n, d[1], d[3] if two else None, d[2],
                                                d[4] if two else None, B)
                    for hh, g in zip(host, gs):
                        oracle.optim8bit_step(kind, hh[0], g, hh[1], hh[2], hh[3] if two else None,
                                              hh[4] if two else None, B, step=step, gdt=gdt, pdt=pdt, vcode=vcode,
                                              **hp)
                    torch.cuda.synchronize()
                    for i, (hh, d) in enumerate(zip(host, dev)):
                        what = f"{name} v={vcode} B={B} gdt={gdt} pdt={pdt} multi={multi} step {step} tensor {i}"
                        for k in ((1, 2, 3, 4) if two else (1, 2)):
                            assert np.array_equal(host_bits(d[k]).view(np.uint8), hh[k].view(np.uint8)), \
                                f"{what}: state array {k}"
                        got = host_bits(d[0])
                        if pdt != oracle.F32:
                            check_params(got, hh[0], pdt, exact, what)
                        elif exact:
                            assert np.array_equal(got.view(np.uint32), hh[0].view(np.uint32)), f"{what}: params"
                        else:
                            np.testing.assert_allclose(got, hh[0], rtol=1e-6, atol=2e-8, err_msg=f"{what}: params")
                        hh[0][:] = got          # the next step starts from the device's parameters


# ---------------------------------------------------------------------------
# fused 4-bit product
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("xdt", DTYPES)
@pytest.mark.parametrize("nested", [False, True])
def test_matmul_every_instantiation(xdt, nested):
    for M in (5, 20, 40):               # 1, 2 and 4 m-tiles per workgroup
        for K in (256, 160):            # K a multiple of 128, and not
            N = 24
            x, codes, scale, nst = mm_case(M, K, N, 64, xdt, nested, seed=M * 1000 + K + 7 * xdt + nested)
            y = mm_run(x, xdt, codes, scale, nst, oracle.NF4, 64, N)
            mm_check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"xdt={xdt} nested={nested} M={M} K={K}")
