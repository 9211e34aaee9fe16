"""GPU parity: user codes (qb_prepare_code, qb_quantize_code, qb_dequantize_code)
and the estimated quantile code (qb_estimate_quantiles) against the CPU
oracle, bit-exact: codes, absmax, outputs, the estimated code's entries, and its
device thresholds equal the host's for the same entries."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu


def table_of(values):
    L = qb()
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    L.qb_prepare_code(list(values), t)
    return t


def read_table(t):
    torch.cuda.synchronize()
    a = t.cpu().numpy()[:2048].view(np.float32)
    return a[:256].copy(), a[256:].copy()


def bucket_index(t):
    """The table's index of thresholds by bucket of n (bytes after the entries
    and thresholds)."""
    torch.cuda.synchronize()
    return t.cpu().numpy()[2048:].copy()


def codes_of(name):
    rng = np.random.default_rng(21)
    if name == "linear":
        return oracle.linear_codebook()
    if name == "dynamic":
        return oracle.codebook(oracle.DYN8)
    if name == "symmetric_no_zero":
        half = np.sort(rng.uniform(0.001, 1.0, 128)).astype(np.float32)
        half[-1] = 1.0
        return np.concatenate([-half[::-1], half]).astype(np.float32)
    if name == "crowded":
        # 240 entries (with repeats) inside [0, 2^-11) share one encoder bucket;
        # the rest spread over [-1, 1]
        tight = np.sort(np.round(rng.uniform(0, 2.0 ** -11, 240), 7)).astype(np.float32)
        tight[::17] = tight[1::17][:tight[::17].size]
        wide = np.linspace(-1, 1, 16).astype(np.float32)
        return np.sort(np.concatenate([tight, wide])).astype(np.float32)
    return oracle.estimate_quantiles((rng.standard_t(3, 50000) * 0.02).astype(np.float32))


def make_x(n, dt, seed):
    x = (np.random.default_rng(seed).standard_t(3, n) * 0.02).astype(np.float32)
    if dt == oracle.F32:
        return x, x
    t = torch.from_numpy(x).to(TORCH_DT[dt])
    return t.view(torch.int16).numpy().view(np.uint16).copy(), t


@pytest.mark.parametrize("name", ["linear", "dynamic", "symmetric_no_zero", "quantile", "crowded"])
@pytest.mark.parametrize("B,dt", [(64, oracle.F32), (256, oracle.BF16), (2048, oracle.F16), (4096, oracle.F32)])
def test_user_code_roundtrip_equals_oracle(name, B, dt):
    L = qb()
    cb = codes_of(name)
    t = table_of(cb)
    n = B * 7 + 4096 * 3 + 123
    xh, _ = make_x(n, dt, seed=B + dt)
    xd = to_device(xh, TORCH_DT[dt])
    nb = (n + B - 1) // B
    codes = torch.full((n + 8,), 0xAB, dtype=torch.uint8, device=DEV)
    absmax = torch.full((nb + 2,), -7.0, device=DEV)
    _, thr = read_table(t)
    fb = [int(np.float32(min(max(v, np.float32(-1)), np.float32(1))) * np.float32(2048) + np.float32(2048))
          for v in thr[:255]]
    want_first = (np.array(fb)[None, :] < np.arange(4098)[:, None]).sum(axis=1)
    assert np.array_equal(bucket_index(t)[:4098], want_first) and not bucket_index(t)[4098:].any()
    L.qb_quantize_code(xd, n, t, B, codes, absmax)
    want_c, want_a = oracle.quantize_custom(xh, cb, B, dt)
    got_c, got_a = host_bits(codes), host_bits(absmax)
    assert np.array_equal(got_c[:n], want_c) and np.all(got_c[n:] == 0xAB)
    assert np.array_equal(got_a[:nb].view(np.uint32), want_a.view(np.uint32)) and np.all(got_a[nb:] == -7.0)
    for ydt in (oracle.F32, oracle.BF16):
        y = torch.empty(n, dtype=TORCH_DT[ydt], device=DEV)
        L.qb_dequantize_code(codes, absmax, t, B, n, y)
        want = oracle.dequantize_custom(want_c, want_a, cb, B, n, ydt)
        assert np.array_equal(host_bits(y).view(np.uint8), want.view(np.uint8))
    if name == "dynamic":                   # the user-code path reproduces the built-in code
        c2 = torch.empty(n, dtype=torch.uint8, device=DEV)
        a2 = torch.empty(nb, device=DEV)
        L.qb_quantize(xd, n, L.QB_DYN8, B, c2, a2)
        torch.cuda.synchronize()
        assert torch.equal(c2, codes[:n]) and torch.equal(a2, absmax[:nb])


@pytest.mark.parametrize("n", [1, 2, 257, 4096, 4097, 4096 * 10 + 5, 1_000_003])
@pytest.mark.parametrize("dt", [oracle.F32, oracle.BF16])
def test_estimated_quantile_code_equals_oracle(n, dt):
    L = qb()
    xh, _ = make_x(n, dt, seed=n)
    if n > 1000:
        xh[::97] = 0 if dt != oracle.F32 else np.float32(0.0)        # repeated values
        if dt == oracle.F32:
            xh[5::211] = np.float32(-0.0)                             # negative zeros count as +0
    xd = to_device(xh, TORCH_DT[dt])
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    ws = torch.empty(L.qb_quantile_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    avg = torch.empty(257, dtype=torch.float64, device=DEV)
    L.qb_estimate_quantiles(xd, n, t, ws, averages=avg)
    vals, thr = read_table(t)
    want = oracle.estimate_quantiles(xh, xdt=dt)
    assert np.array_equal(vals.view(np.uint32), want.view(np.uint32))
    want_avg = oracle.quantile_averages(xh, xdt=dt)
    assert np.array_equal(avg.cpu().numpy().view(np.uint64), want_avg.view(np.uint64))
    # the device thresholds and bucket index are the host's for the same entries
    host_t = table_of(vals)
    _, host_thr = read_table(host_t)
    assert np.array_equal(thr.view(np.uint32), host_thr.view(np.uint32))
    assert np.array_equal(bucket_index(t), bucket_index(host_t))


@pytest.mark.parametrize("nchunks", [257, 601, 2000])
def test_quantile_averages_are_exact_means_over_many_binades(nchunks):
    """Order statistics spread over 2^-60 .. 2^60 with both signs, more than
    256 chunks and a ragged last chunk: every average equals the oracle's exact
    mean rounded once, bit for bit (a plain binary64 sum misses it)."""
    L = qb()
    rng = np.random.default_rng(nchunks)
    n = 4096 * (nchunks - 1) + 1000
    mag = np.ldexp(rng.uniform(1.0, 2.0, n), rng.integers(-60, 61, n))
    xh = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    xh[rng.integers(0, n, 2000)] = np.float32(-0.0)
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    ws = torch.empty(L.qb_quantile_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    avg = torch.full((257,), float("nan"), dtype=torch.float64, device=DEV)
    L.qb_estimate_quantiles(to_device(xh), n, t, ws, averages=avg)
    want_avg = oracle.quantile_averages(xh)
    assert np.array_equal(avg.cpu().numpy().view(np.uint64), want_avg.view(np.uint64))
    vals, _ = read_table(t)
    assert np.array_equal(vals.view(np.uint32), oracle.estimate_quantiles(xh).view(np.uint32))


def test_quantile_code_of_a_uniform_grid():
    # one chunk (257 k <= 4096 values) holding a shuffled 0, 1, ..., 257 k - 1:
    # the closed form (i + 1/2) / 255.5 of the oracle's pin
    L = qb()
    k = 15
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    one = np.random.default_rng(1).permutation(257 * k).astype(np.float32)
    ws = torch.empty(L.qb_quantile_workspace_bytes(one.size), dtype=torch.uint8, device=DEV)
    L.qb_estimate_quantiles(to_device(one), one.size, t, ws)
    vals, _ = read_table(t)
    want = np.array([(i + 0.5) / 255.5 for i in range(256)], dtype=np.float32)
    assert np.array_equal(vals, want)


def test_estimate_then_quantize_a_large_tensor():
    """The full quantile flow on 16M values: estimate the code on the device,
    quantize and dequantize with it; sampled blocks against the oracle."""
    L = qb()
    n, B = 1 << 24, 2048
    x = torch.empty(n, device=DEV).normal_(0, 0.02, generator=torch.Generator(device=DEV).manual_seed(3))
    t = torch.empty(L.qb_code_table_bytes(), dtype=torch.uint8, device=DEV)
    ws = torch.empty(L.qb_quantile_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    avg = torch.empty(257, dtype=torch.float64, device=DEV)
    L.qb_estimate_quantiles(x, n, t, ws, averages=avg)
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(n // B, device=DEV)
    L.qb_quantize_code(x, n, t, B, codes, absmax)
    y = torch.empty(n, device=DEV)
    L.qb_dequantize_code(codes, absmax, t, B, n, y)
    vals, _ = read_table(t)
    xh = x.cpu().numpy()
    assert np.array_equal(vals, oracle.estimate_quantiles(xh))
    assert np.array_equal(avg.cpu().numpy().view(np.uint64), oracle.quantile_averages(xh).view(np.uint64))
    blocks = np.random.default_rng(4).choice(n // B, 256, replace=False)
    idx = torch.from_numpy(blocks).to(DEV)
    xs = x.view(-1, B).index_select(0, idx).cpu().numpy().reshape(-1)
    want_c, want_a = oracle.quantize_custom(xs, vals, B)
    assert np.array_equal(codes.view(-1, B).index_select(0, idx).cpu().numpy().reshape(-1), want_c)
    assert np.array_equal(absmax.index_select(0, idx).cpu().numpy(), want_a)
    want_y = oracle.dequantize_custom(want_c, want_a, vals, B, xs.size)
    assert np.array_equal(y.view(-1, B).index_select(0, idx).cpu().numpy().reshape(-1), want_y)


@pytest.mark.parametrize("name", ["edge_grid", "crowded", "dynamic", "linear"])
def test_user_code_on_bucket_edges(name):
    """Values at, and one ulp beside, every encoder bucket edge and every
    threshold, in blocks whose absmax is 1 (so the normalized value is the
    input itself).  edge_grid is the code (k + 1/2)/128 - 1, whose midpoints are
    bucket edges: its thresholds sit on an edge (negative side) or one ulp
    above it (positive side, ties toward the smaller magnitude)."""
    L = qb()
    B = 2048
    if name == "edge_grid":
        cb = ((np.arange(256) + 0.5) / 128 - 1).astype(np.float32)
    else:
        cb = codes_of(name)
    t = table_of(cb)
    _, thr = read_table(t)
    edges = (np.arange(4097) / 2048 - 1).astype(np.float32)
    core = np.concatenate([edges, thr[:255]])
    core = core[np.abs(core) <= 1]
    vals = np.concatenate([core, np.nextafter(core, np.float32(2)), np.nextafter(core, np.float32(-2)),
                           np.float32([0.0, -0.0, 1e-30, -1e-30])]).astype(np.float32)
    vals = vals[np.abs(vals) <= 1]
    per = B - 1
    nb = -(-vals.size // per)
    x = np.zeros(nb * B, np.float32)
    for b in range(nb):
        chunk = vals[b * per:(b + 1) * per]
        x[b * B] = 1.0
        x[b * B + 1:b * B + 1 + chunk.size] = chunk
    n = x.size - 5                                       # a ragged last block
    x = x[:n].copy()
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(nb, device=DEV)
    L.qb_quantize_code(to_device(x), n, t, B, codes, absmax)
    want_c, want_a = oracle.quantize_custom(x, cb, B)
    assert np.all(want_a == 1.0)
    got = host_bits(codes)
    assert np.array_equal(got, want_c), np.flatnonzero(got != want_c)[:8]
