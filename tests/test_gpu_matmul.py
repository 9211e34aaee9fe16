"""GPU parity: qb_dequant_matmul (the product of a 4-bit layer in its compute
dtype) against the CPU oracle.  The oracle multiplies the dequantized weights
exactly (binary64); the kernel adds the K products in binary32 in an order of
its own, so every output must lie within

    e = (K + 2) 2^-23 sum_k |x_mk w_nk|

of the exact product, plus half a unit in the last place of the output dtype
for the final rounding.  Nearly all outputs equal the correctly rounded exact
product; the test reports that share and requires most of them."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu

MANT = {oracle.F32: 23, oracle.BF16: 7, oracle.F16: 10}
MIN_EXP = {oracle.F32: -126, oracle.BF16: -126, oracle.F16: -14}


def ulp(v, dt):
    """Unit in the last place of |v| in dtype dt (subnormal spacing below the normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
    e = np.maximum(e, MIN_EXP[dt])
    return np.exp2(e - MANT[dt])


def to_float(bits, dt):
    return bits.astype(np.float64) if dt == oracle.F32 else oracle.convert(bits.reshape(-1), dt, oracle.F32).reshape(
        bits.shape).astype(np.float64)


def rounded(s, dt):
    f = s.astype(np.float32)                        # within the bound's slack for fp32 outputs
    if dt == oracle.F32:
        return f.astype(np.float64)
    return torch.from_numpy(s).to(TORCH_DT[dt]).double().numpy()


def make_case(M, K, N, B, xdt, nested, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, N * K // 2, dtype=np.uint8)
    nb = -(-N * K // B)
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    x = x32 if xdt == oracle.F32 else oracle.convert(x32.reshape(-1), oracle.F32, xdt).reshape(M, K)
    if nested:
        c2 = rng.integers(0, 256, nb, dtype=np.uint8)
        a2 = (rng.random(-(-nb // 256)) * 0.02 + 0.005).astype(np.float32)
        mu = np.float32(0.03)
        scale = oracle.dq_decode(c2, a2, mu, 256)
        return x, codes, scale, (c2, a2, mu)
    return x, codes, (rng.random(nb) * 0.1 + 0.005).astype(np.float32), None


def run_gpu(x, xdt, codes, scale, nested, code, B, N):
    L = qb()
    M, K = x.shape
    xd = to_device(x, TORCH_DT[xdt]).reshape(M, K)
    y = torch.full((M, N), float("nan"), dtype=TORCH_DT[xdt], device=DEV)
    cd = to_device(codes)
    if nested:
        c2, a2, mu = nested
        keep = [to_device(c2), to_device(a2), torch.tensor([mu], dtype=torch.float32, device=DEV)]
        dq = L.make_dq(keep[0], keep[1], keep[2], 256)
        L.qb_dequant_matmul(xd, cd, None, code, B, N, y, dq=dq)
    else:
        L.qb_dequant_matmul(xd, cd, to_device(scale), code, B, N, y)
    torch.cuda.synchronize()
    return host_bits(y)


def check(y_bits, x, xdt, codes, scale, code, B, N, what):
    M, K = x.shape
    s, a = oracle.dequant_matmul(x, xdt, codes, scale, code, B, N)
    y = to_float(y_bits, xdt)
    e = (K + 2) * 2.0 ** -23 * a
    bound = e + 0.5 * ulp(np.abs(s) + e, xdt)
    err = np.abs(y - s)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    assert np.all(err <= bound), f"{what}: {np.sum(err > bound)} outputs beyond the bound, worst {np.max(err / bound)}"
    exact = np.mean(y == rounded(s, xdt))
    # a 16-bit output hides the binary32 sum's error below its half ulp almost
    # always; a binary32 output shows it
    if xdt != oracle.F32:
        assert exact >= 0.9, f"{what}: only {exact:.4f} of outputs correctly rounded"
    return exact


# M picks the kernel's m-tiles per workgroup (1 up to 16 rows, 2 up to 32, else 4); K a multiple of 128 or not
SHAPES = [(1, 4096, 300), (16, 512, 64), (37, 4096, 100), (64, 256, 48), (65, 1024, 33), (3, 32, 17),
          (16, 160, 40), (130, 96, 16), (17, 1024, 40), (32, 160, 24), (29, 4096, 33)]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16, oracle.F32])
def test_shapes_and_dtypes(M, K, N, xdt):
    x, codes, scale, _ = make_case(M, K, N, 64, xdt, False, seed=M * 7 + K + N)
    y = run_gpu(x, xdt, codes, scale, None, oracle.NF4, 64, N)
    check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"M={M} K={K} N={N} dt={xdt}")


@pytest.mark.parametrize("code", [oracle.NF4, oracle.FP4])
@pytest.mark.parametrize("B", [64, 128, 256, 4096])
@pytest.mark.parametrize("nested", [False, True])
def test_codes_blocks_and_nesting(code, B, nested):
    M, K, N = 9, 2048, 72
    x, codes, scale, nst = make_case(M, K, N, B, oracle.BF16, nested, seed=B + code + 3 * nested)
    y = run_gpu(x, oracle.BF16, codes, scale, nst, code, B, N)
    check(y, x, oracle.BF16, codes, scale, code, B, N, f"code={code} B={B} nested={nested}")


def test_blocks_spanning_rows():
    # B = 4096 > K = 160: a block's absmax covers parts of several weight rows
    M, K, N, B = 5, 160, 70, 4096
    x, codes, scale, _ = make_case(M, K, N, B, oracle.BF16, False, seed=9)
    y = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, B, N)
    check(y, x, oracle.BF16, codes, scale, oracle.NF4, B, N, "B > K")


def test_repeatable_and_equal_to_the_unfused_product_within_the_bound():
    """The same bits on every run; and dequantize + torch matmul (binary32) is
    within the same bound of the oracle (a second, independent route)."""
    L = qb()
    M, K, N, B = 16, 4096, 256, 64
    x, codes, scale, _ = make_case(M, K, N, B, oracle.BF16, False, seed=11)
    y1 = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, B, N)
    y2 = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, B, N)
    assert np.array_equal(y1, y2)
    w = torch.empty(N * K, dtype=torch.bfloat16, device=DEV)
    L.qb_dequantize(to_device(codes), to_device(scale), None, oracle.NF4, B, N * K, w)
    ref = (to_device(x, torch.bfloat16).reshape(M, K).float() @ w.reshape(N, K).float().T.contiguous()).to(torch.bfloat16)
    check(host_bits(ref), x, oracle.BF16, codes, scale, oracle.NF4, B, N, "unfused route")


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("NK", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_7b_layer_shapes(M, NK):
    """The 7B decoder's projection shapes (NF4, nested, B = 64), bf16 compute."""
    N, K = NK
    x, codes, scale, nst = make_case(M, K, N, 64, oracle.BF16, True, seed=N + K + M)
    y = run_gpu(x, oracle.BF16, codes, scale, nst, oracle.NF4, 64, N)
    check(y, x, oracle.BF16, codes, scale, oracle.NF4, 64, N, f"7B {N}x{K} M={M}")


# the tiled kernel (16-bit compute dtypes, K a multiple of 128, M >= 65): tiles
# of 64 x 64 below 512 rows, 128 x 128 from 512; ragged M and N, one step of K
TILED = [(65, 128, 64), (100, 256, 130), (200, 1024, 197), (511, 512, 257), (512, 384, 128), (700, 640, 300),
         (1000, 1152, 129)]


@pytest.mark.parametrize("M,K,N", TILED)
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16])
def test_tiled_shapes(M, K, N, xdt):
    x, codes, scale, _ = make_case(M, K, N, 64, xdt, False, seed=M + 3 * K + N)
    y = run_gpu(x, xdt, codes, scale, None, oracle.NF4, 64, N)
    check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"tiled M={M} K={K} N={N} dt={xdt}")


@pytest.mark.parametrize("code", [oracle.NF4, oracle.FP4])
@pytest.mark.parametrize("B", [64, 256, 4096])
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M", [96, 600])
def test_tiled_codes_blocks_and_nesting(code, B, nested, M):
    K, N = 1024, 192
    x, codes, scale, nst = make_case(M, K, N, B, oracle.BF16, nested, seed=B + code + 5 * nested + M)
    y = run_gpu(x, oracle.BF16, codes, scale, nst, code, B, N)
    check(y, x, oracle.BF16, codes, scale, code, B, N, f"tiled M={M} code={code} B={B} nested={nested}")


def test_tiled_blocks_spanning_rows():
    M, K, N, B = 130, 128, 70, 4096                     # B > K: one absmax over parts of several rows
    x, codes, scale, _ = make_case(M, K, N, B, oracle.BF16, False, seed=19)
    y = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, B, N)
    check(y, x, oracle.BF16, codes, scale, oracle.NF4, B, N, "tiled B > K")


def test_tiled_repeatable():
    M, K, N = 640, 2048, 384
    x, codes, scale, _ = make_case(M, K, N, 64, oracle.BF16, False, seed=23)
    y1 = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, 64, N)
    y2 = run_gpu(x, oracle.BF16, codes, scale, None, oracle.NF4, 64, N)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M", [256, 1024])
@pytest.mark.parametrize("NK", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_7b_layer_shapes_many_rows(M, NK):
    """The 7B projection shapes at 256 and 1024 rows (NF4, nested, B = 64, bf16):
    every row computed on the GPU; 48 seeded rows (the first, the last and
    random ones) checked against the oracle's exact product, rows being
    independent of each other."""
    N, K = NK
    x, codes, scale, nst = make_case(M, K, N, 64, oracle.BF16, True, seed=N + K + M)
    y = run_gpu(x, oracle.BF16, codes, scale, nst, oracle.NF4, 64, N)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, 46, replace=False)]))
    check(y[rows], x[rows], oracle.BF16, codes, scale, oracle.NF4, 64, N, f"7B {N}x{K} M={M} (sampled rows)")


# every instantiation of the tiled kernel: 64 x 64 and 128 x 128 tiles (M below / from 512), one or two k halves
# per step (K a multiple of 128 only / of 256), plain and nested, bf16 and fp16
@pytest.mark.parametrize("M,K", [(100, 384), (100, 512), (600, 384), (600, 512)])
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("nested", [False, True])
def test_tiled_every_instantiation(M, K, xdt, nested):
    N = 130
    x, codes, scale, nst = make_case(M, K, N, 64, xdt, nested, seed=M + K + 3 * xdt + 7 * nested)
    y = run_gpu(x, xdt, codes, scale, nst, oracle.NF4, 64, N)
    check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"tiled M={M} K={K} xdt={xdt} nested={nested}")


# up to 8 rows of activations (decode): the rows are staged in LDS while M * K * 2 <= 64 KiB (K rounded up to
# whole steps of 128), with one step of codes in flight per wave up to 4 steps a wave (K <= 4096), two beyond.
# Staged: M = 1 up to K = 32768, M = 2 up to 16384, M = 3 up to 10880, M = 4 up to 8192, M = 5 up to 6528, M = 8 up
# to 4096; the others load x per step.
@pytest.mark.parametrize("K", [160, 4096, 5152, 11008, 33024])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("nested", [False, True])
def test_decode_rows(K, M, xdt, nested):
    N = 40
    x, codes, scale, nst = make_case(M, K, N, 64, xdt, nested, seed=K + 3 * xdt + 7 * nested + 11 * M)
    y = run_gpu(x, xdt, codes, scale, nst, oracle.NF4, 64, N)
    check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"decode M={M} K={K} xdt={xdt} nested={nested}")
