"""GPU parity: qb_dequant_matmul_grouped (several 4-bit weights against the
same activations in one launch) equals qb_dequant_matmul on each weight bit
for bit, and so lies within the product's binary32 summation bound of the
oracle (checked here again for every weight of the small cases)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device
from test_gpu_matmul import check, make_case, run_gpu

pytestmark = pytest.mark.gpu


def grouped(x, xdt, weights, code, B):
    """weights: list of (codes, scale, nested, N) host arrays; returns the y bits of each."""
    L = qb()
    M, K = x.shape
    xd = to_device(x, TORCH_DT[xdt]).reshape(M, K)
    keep, rows, ys = [], [], []
    for codes, scale, nested, N in weights:
        y = torch.full((M, max(N, 1)), float("nan"), dtype=TORCH_DT[xdt], device=DEV)[:, :N].contiguous()
        cd = to_device(codes) if N else torch.empty(16, dtype=torch.uint8, device=DEV)
        if nested:
            c2, a2, mu = nested
            t = [to_device(c2), to_device(a2), torch.tensor([mu], dtype=torch.float32, device=DEV)]
            dq = L.make_dq(t[0], t[1], t[2], 256)
            keep += t
            rows.append((cd, None, dq, N, y))
        else:
            a = to_device(scale) if N else torch.empty(4, dtype=torch.float32, device=DEV)
            keep.append(a)
            rows.append((cd, a, None, N, y))
        keep.append(cd)
        ys.append(y)
    table = L.matmul_weights(rows)
    L.qb_dequant_matmul_grouped(xd, table, len(rows), code, B)
    torch.cuda.synchronize()
    return [host_bits(y) for y in ys]


def case(M, K, Ns, xdt, nested, B, seed):
    x = None
    weights = []
    for i, N in enumerate(Ns):
        xi, codes, scale, nst = make_case(M, K, max(N, 1), B, xdt, nested, seed=seed + 101 * i)
        x = xi if x is None else x
        weights.append((codes, scale, nst, N))
    return x, weights


# M: one, two and four m-tiles of the small-M kernel, then the tiled kernel's regime (bf16 / fp16 with K a
# multiple of 128) where the call launches once per weight; K = 160 keeps the small kernel at every M
@pytest.mark.parametrize("M", [1, 2, 4, 7, 16, 24, 33, 64, 100, 300])
@pytest.mark.parametrize("K", [512, 160])
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16, oracle.F32])
@pytest.mark.parametrize("nested", [False, True])
def test_grouped_equals_single_calls(M, K, xdt, nested):
    Ns = [48, 130, 16]
    x, weights = case(M, K, Ns, xdt, nested, 64, seed=M + K + 5 * xdt + 17 * nested)
    got = grouped(x, xdt, weights, oracle.NF4, 64)
    for (codes, scale, nst, N), y in zip(weights, got):
        single = run_gpu(x, xdt, codes, scale, nst, oracle.NF4, 64, N)
        assert np.array_equal(y, single), f"M={M} K={K} N={N}: grouped differs from the single call"
        check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"grouped M={M} K={K} N={N}")


@pytest.mark.parametrize("code", [oracle.NF4, oracle.FP4])
@pytest.mark.parametrize("B", [64, 256, 4096])
def test_grouped_codes_blocks_and_empty_weights(code, B):
    # up to the limit of eight weights, two of them empty (skipped)
    M, K = 5, 1024
    Ns = [64, 0, 17, 100, 0, 33, 200, 8]
    x, weights = case(M, K, Ns, oracle.BF16, False, B, seed=B + code)
    got = grouped(x, oracle.BF16, weights, code, B)
    for (codes, scale, nst, N), y in zip(weights, got):
        if N == 0:
            continue
        assert np.array_equal(y, run_gpu(x, oracle.BF16, codes, scale, nst, code, B, N))
        check(y, x, oracle.BF16, codes, scale, code, B, N, f"code={code} B={B} N={N}")


@pytest.mark.parametrize("M", [1, 4, 8, 16])
@pytest.mark.parametrize("layer", ["qkv", "gate_up"])
def test_grouped_7b_projections(M, layer):
    """A 7B decoder layer's q/k/v (3 x 4096 x 4096) or gate/up (2 x 11008 x 4096)
    in one launch: bit for bit the single calls."""
    Ns = [4096] * 3 if layer == "qkv" else [11008] * 2
    K = 4096
    x, weights = case(M, K, Ns, oracle.BF16, True, 64, seed=M + len(Ns))
    got = grouped(x, oracle.BF16, weights, oracle.NF4, 64)
    for (codes, scale, nst, N), y in zip(weights, got):
        assert np.array_equal(y, run_gpu(x, oracle.BF16, codes, scale, nst, oracle.NF4, 64, N))


@pytest.mark.parametrize("K", [5152, 11008])
@pytest.mark.parametrize("M", [1, 2, 6])
@pytest.mark.parametrize("xdt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("nested", [False, True])
def test_grouped_decode_row_deep(K, M, xdt, nested):
    """Staged rows of activations with more than 4 steps of K per wave (two steps of codes in flight)."""
    x, weights = case(M, K, [48, 130], xdt, nested, 64, seed=K + 5 * xdt + 17 * nested + 3 * M)
    got = grouped(x, xdt, weights, oracle.NF4, 64)
    for (codes, scale, nst, N), y in zip(weights, got):
        assert np.array_equal(y, run_gpu(x, xdt, codes, scale, nst, oracle.NF4, 64, N))
        check(y, x, xdt, codes, scale, oracle.NF4, 64, N, f"grouped decode K={K} N={N}")
