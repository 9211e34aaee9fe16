"""Pins of the oracle's 4-bit layer product dequant_matmul (CPU only): the
orientation y = x W^T, the dequantized weights it multiplies (those of the
pinned dequantize_blockwise), and its bound term."""
import numpy as np
import pytest
import torch

import oracle


def random_weights(N, K, B, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, N * K // 2, dtype=np.uint8)
    absmax = (rng.random(-(-N * K // B)) * 0.1 + 0.01).astype(np.float32)
    return codes, absmax


@pytest.mark.parametrize("xdt", [oracle.F32, oracle.BF16, oracle.F16])
def test_identity_activations_return_the_dequantized_weights(xdt):
    # x = I (M = K): y[m, n] = W[n, m], i.e. y = W^T, entry for entry
    N, K, B = 48, 64, 64
    codes, absmax = random_weights(N, K, B, 1)
    eye = np.eye(K, dtype=np.float32)
    x = eye if xdt == oracle.F32 else oracle.convert(eye.reshape(-1), oracle.F32, xdt).reshape(K, K)
    s, a = oracle.dequant_matmul(x, xdt, codes, absmax, oracle.NF4, B, N)
    w = oracle.dequantize_blockwise(codes, absmax, oracle.NF4, B, N * K, ydt=xdt)
    wf = (w if xdt == oracle.F32 else oracle.convert(w, xdt, oracle.F32)).reshape(N, K)
    assert np.array_equal(s, wf.T.astype(np.float64))
    assert np.array_equal(a, np.abs(wf.T).astype(np.float64))


def test_product_equals_torch_on_the_dequantized_matrix():
    # against torch's float64 matmul of the same bf16 operands
    M, N, K, B = 7, 33, 256, 64
    codes, absmax = random_weights(N, K, B, 2)
    xb = torch.randn(M, K, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    x = xb.view(torch.int16).numpy().view(np.uint16)
    s, a = oracle.dequant_matmul(x, oracle.BF16, codes, absmax, oracle.FP4, B, N)
    w = oracle.dequantize_blockwise(codes, absmax, oracle.FP4, B, N * K, ydt=oracle.BF16)
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().reshape(N, K)
    want = xb.double() @ wt.T
    assert np.allclose(s, want.numpy(), rtol=1e-13, atol=1e-13)
    assert np.all(a >= np.abs(s))


def test_blocks_of_one_weight_row_scale_its_outputs():
    # scaling the absmax of every block of weight row n by 2 doubles y[:, n] exactly
    M, N, K, B = 5, 16, 128, 64
    codes, absmax = random_weights(N, K, B, 4)
    x = np.random.default_rng(5).standard_normal((M, K)).astype(np.float32)
    s, _ = oracle.dequant_matmul(x, oracle.F32, codes, absmax, oracle.NF4, B, N)
    a2 = absmax.copy()
    a2[3 * K // B:4 * K // B] *= 2
    s2, _ = oracle.dequant_matmul(x, oracle.F32, codes, a2, oracle.NF4, B, N)
    assert np.array_equal(s2[:, 3], 2 * s[:, 3])
    assert np.array_equal(np.delete(s2, 3, axis=1), np.delete(s, 3, axis=1))
