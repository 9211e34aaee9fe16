"""Pins of the oracle's AdamW step (CPU only).

The pages present the 8-bit optimizer as a drop-in replacement for AdamW with
the same lr / betas / eps ("bitsandbytes - Quantização de LLM", section
Workflow 3; "Py之bitsandbytes", section 使用8位优化器), so the update is read as
torch.optim.AdamW's, with both moments stored as block-wise dynamic 8-bit codes.
"""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def rnd(seed, n, scale):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def test_fp32_state_update_matches_torch_adamw():
    n = 10000
    p = rnd(1, n, 0.02)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["wd"], foreach=False)
    for step in range(1, 11):
        g = rnd(100 + step, n, 1e-3)
        oracle.adamw32_step(p, g, m, v, step=step, **HP)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        st = opt.state[tp]
        # the two differ only in rounding order: within 1e-6 relative of each
        # tensor's scale (elementwise relative error is meaningless near 0)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-6, atol=1e-6 * 0.02)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-6, atol=1e-6 * np.abs(m).max())
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-6, atol=1e-6 * np.abs(v).max())


def test_host_scalars_closed_form():
    for step in (1, 2, 10, 1000):
        s = oracle.adam_scalars(step=step, **HP)
        b1, b2 = HP["beta1"], HP["beta2"]
        assert s["s1"] == np.float32(HP["lr"] / (1 - b1 ** step))
        assert abs(float(s["s2"]) - 1 / np.sqrt(1 - b2 ** step)) <= 1e-7 / np.sqrt(1 - b2 ** step)
        assert s["dec"] == np.float32(1 - HP["lr"] * HP["wd"])
        assert s["ob1"] == np.float32(0.1) and s["ob2"] == np.float32(0.001)
        assert s["b1"] == np.float32(0.9) and s["b2"] == np.float32(0.999)


def fresh_state(n, B):
    nb = (n + B - 1) // B
    return (np.full(n, 127, np.uint8), np.full(n, 127, np.uint8),
            np.zeros(nb, np.float32), np.zeros(nb, np.float32))


def test_step_one_closed_form():
    n, B = 2048 * 3 + 100, 2048
    p0 = rnd(2, n, 0.02)
    g = rnd(3, n, 1e-3)
    p = p0.copy()
    cm, cv, am, av = fresh_state(n, B)
    oracle.adamw8bit_step(p, g, cm, cv, am, av, B, step=1, **HP)
    # from zero moments the bias-corrected moments are g and g^2
    want = p0.astype(np.float64) * (1 - HP["lr"] * HP["wd"]) - HP["lr"] * g / (np.abs(g.astype(np.float64)) + HP["eps"])
    np.testing.assert_allclose(p, want, rtol=1e-6, atol=1e-6 * 0.02)   # relative to the parameter scale
    # the new state is exactly the block-wise quantization of m' = (1-b1) g and v' = (1-b2) g^2
    ob1 = np.float32(1 - 0.9)
    ob2 = np.float32(1 - 0.999)
    m1 = (ob1 * g).astype(np.float32)
    v1 = (ob2 * (g * g).astype(np.float32)).astype(np.float32)
    qm, qam = oracle.quantize_blockwise(m1, oracle.DYN8, B)
    qv, qav = oracle.quantize_blockwise(v1, oracle.DYN8, B)
    assert np.array_equal(cm, qm) and np.array_equal(am, qam)
    assert np.array_equal(cv, qv) and np.array_equal(av, qav)


def test_zero_gradient_from_zero_state():
    n, B = 5000, 256
    p0 = rnd(4, n, 0.02)
    p = p0.copy()
    cm, cv, am, av = fresh_state(n, B)
    oracle.adamw8bit_step(p, np.zeros(n, np.float32), cm, cv, am, av, B, step=1, **HP)
    assert np.all(cm == 127) and np.all(cv == 127) and np.all(am == 0) and np.all(av == 0)
    dec = np.float32(1 - HP["lr"] * HP["wd"])
    assert np.array_equal(p, (p0 * dec).astype(np.float32))


def test_eight_bit_step_is_dequantize_update_requantize():
    """Composition: the 8-bit step equals dequantizing the state, one fp32-state
    step, and quantizing the new moments again (all with the pinned pieces)."""
    n, B = 4096 * 3 + 333, 4096
    p = rnd(5, n, 0.02)
    cm, cv, am, av = fresh_state(n, B)
    for step in range(1, 6):
        g = rnd(200 + step, n, 1e-3)
        m = oracle.dequantize_blockwise(cm, am, oracle.DYN8, B, n)
        v = oracle.dequantize_blockwise(cv, av, oracle.DYN8, B, n)
        p32 = p.copy()
        oracle.adamw32_step(p32, g, m, v, step=step, **HP)
        oracle.adamw8bit_step(p, g, cm, cv, am, av, B, step=step, **HP)
        assert np.array_equal(p, p32)
        qm, qam = oracle.quantize_blockwise(m, oracle.DYN8, B)
        qv, qav = oracle.quantize_blockwise(v, oracle.DYN8, B)
        assert np.array_equal(cm, qm) and np.array_equal(am, qam)
        assert np.array_equal(cv, qv) and np.array_equal(av, qav)


def test_blocks_are_independent():
    n, B = 2048 * 6, 2048
    p = rnd(6, n, 0.02)
    g = rnd(7, n, 1e-3)
    whole = [p.copy(), *fresh_state(n, B)]
    oracle.adamw8bit_step(whole[0], g, *whole[1:], B, step=1, **HP)
    for b in range(6):
        sl = slice(b * B, (b + 1) * B)
        part = [p[sl].copy(), *fresh_state(B, B)]
        oracle.adamw8bit_step(part[0], g[sl], *part[1:], B, step=1, **HP)
        assert np.array_equal(part[0], whole[0][sl])
        assert np.array_equal(part[1], whole[1][sl]) and np.array_equal(part[2], whole[2][sl])
        assert part[3][0] == whole[3][b] and part[4][0] == whole[4][b]


def test_bf16_gradients_equal_their_widening():
    n, B = 3000, 256
    g32 = rnd(8, n, 1e-3)
    gb = torch.from_numpy(g32).to(torch.bfloat16)
    bits = gb.view(torch.int16).numpy().view(np.uint16)
    wide = gb.float().numpy()
    a = [rnd(9, n, 0.02), *fresh_state(n, B)]
    b = [a[0].copy(), *fresh_state(n, B)]
    oracle.adamw8bit_step(a[0], bits, *a[1:], B, step=1, gdt=oracle.BF16, **HP)
    oracle.adamw8bit_step(b[0], wide, *b[1:], B, step=1, **HP)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
