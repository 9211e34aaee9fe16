"""bench.py's host-side figures (CPU): the per-block round-trip error summary
and the algorithmic byte counts it reports."""
import numpy as np
import torch

import bench


def test_roundtrip_error_stats_on_known_blocks():
    B = 4
    # three blocks: errors 0 / [0.1, 0, 0, 0] / [0.2, 0.2, 0.2, 0.2]; absmax 1, 2, 4
    x = torch.tensor([1.0, 0, 0, 0, 2.0, 0, 0, 0, 4.0, 1, 1, 1])
    y = x.clone()
    y[4] -= 0.1
    y[8:] += 0.2
    st = bench.roundtrip_error_stats(torch, x, y, B)
    assert st["blocks"] == 3
    bm = st["block_max_abs_err"]
    assert np.isclose(bm["max"], 0.2, atol=1e-6) and np.isclose(bm["mean"], (0 + 0.1 + 0.2) / 3, atol=1e-6)
    assert np.isclose(st["block_mean_abs_err"]["max"], 0.2, atol=1e-6)
    assert np.isclose(st["block_max_rel_err"]["max"], 0.05, atol=1e-6)      # 0.1 / 2 and 0.2 / 4
    assert np.isclose(st["block_mean_rel_err"]["mean"], (0 + 0.025 / 2 + 0.2 / 4) / 3, atol=1e-6)


def test_algorithmic_byte_counts():
    assert bench.q8_bytes_per_elem(2048) == 5.0 + 4.0 / 2048                 # one pass
    assert np.isclose(bench.adam_bytes_per_param(), 14.0078125)
    assert np.isclose(bench.w4_bytes_per_weight(), 2.5159, atol=1e-4)
    # the fused 4-bit product at 4096 x 4096, one row of activations: 8.67 MB
    assert np.isclose(bench.dq4_matmul_bytes(1, 4096, 4096) / 1e6, 8.67, atol=0.01)
