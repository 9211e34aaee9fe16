"""Pins of the oracle's sibling 8-bit optimizers (CPU only).

The pages list 8-bit Adam, SGD, RMSprop and Lion beside AdamW as drop-in
replacements that keep their optimizer's hyperparameters ("bitsandbytes深度解析",
section 优化器模块深度分析; "Py之bitsandbytes", sections 1 and 使用8位优化器).
Adam, SGD and RMSprop are pinned to torch.optim's implementations (an
independent library) with binary32 states; Lion, which torch does not ship, to
its closed forms.  The 8-bit variants are pinned by their structure: the new
codes are exactly the block-wise quantization of the updated binary32 states.
"""
import numpy as np
import pytest
import torch

import oracle


def rnd(seed, n, scale):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def close(a, b, scale):
    # the two differ only in rounding order: within 1e-6 relative of each
    # tensor's scale (elementwise relative error is meaningless near 0)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6 * scale)


def run_against_torch(kind, topt, hp, n=10000, steps=10):
    p = rnd(1, n, 0.02)
    x1 = np.zeros(n, np.float32)
    x2 = np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = topt([tp])
    for step in range(1, steps + 1):
        g = rnd(100 + step, n, 1e-3)
        oracle.optim32_step(kind, p, g, x1, x2 if oracle.OPTIMIZER_STATES[kind] == 2 else None, step=step, **hp)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        close(p, tp.detach().numpy(), 0.02)
    return p, x1, x2, opt.state[tp]


# With L2-coupled decay, gw = g + wd*p can cancel to |gw| ~ eps, where the
# update gw / (|gw| + eps) turns a one-ulp difference in how gw is rounded (torch
# may fuse that multiply-add) into a large relative change: eps = 1e-6 keeps
# every element well conditioned for the comparison.
def test_adam_l2_matches_torch_adam():
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.995, eps=1e-6, wd=0.01)
    _, m, v, st = run_against_torch(
        oracle.ADAM, lambda ps: torch.optim.Adam(ps, lr=1e-3, betas=(0.9, 0.995), eps=1e-6, weight_decay=0.01,
                                                 foreach=False), hp)
    close(m, st["exp_avg"].numpy(), np.abs(m).max())
    close(v, st["exp_avg_sq"].numpy(), np.abs(v).max())


def test_adam_without_decay_equals_adamw_without_decay():
    n = 5000
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0)
    pa, pw = rnd(3, n, 0.02), rnd(3, n, 0.02)
    ma, va, mw, vw = (np.zeros(n, np.float32) for _ in range(4))
    for step in range(1, 6):
        g = rnd(50 + step, n, 1e-3)
        oracle.optim32_step(oracle.ADAM, pa, g, ma, va, step=step, **hp)
        oracle.optim32_step(oracle.ADAMW, pw, g, mw, vw, step=step, **hp)
    assert np.array_equal(pa, pw) and np.array_equal(ma, mw) and np.array_equal(va, vw)


@pytest.mark.parametrize("nesterov,dampening,wd", [(False, 0.0, 0.0), (False, 0.1, 1e-2), (True, 0.0, 1e-2)])
def test_sgd_momentum_matches_torch_sgd(nesterov, dampening, wd):
    hp = dict(lr=1e-2, beta1=0.9, wd=wd, dampening=dampening, nesterov=nesterov)
    _, buf, _, st = run_against_torch(
        oracle.SGD, lambda ps: torch.optim.SGD(ps, lr=1e-2, momentum=0.9, dampening=dampening, weight_decay=wd,
                                               nesterov=nesterov, foreach=False), hp)
    close(buf, st["momentum_buffer"].numpy(), np.abs(buf).max())


def test_rmsprop_matches_torch_rmsprop():
    hp = dict(lr=1e-3, beta2=0.99, eps=1e-6, wd=1e-2)
    _, v, _, st = run_against_torch(
        oracle.RMSPROP, lambda ps: torch.optim.RMSprop(ps, lr=1e-3, alpha=0.99, eps=1e-6, weight_decay=1e-2,
                                                       foreach=False), hp)
    close(v, st["square_avg"].numpy(), np.abs(v).max())


def test_lion_closed_forms():
    n = 4096
    lr, b1, b2, wd = 1e-4, 0.9, 0.99, 0.1
    p0 = rnd(4, n, 0.02)
    m0 = rnd(5, n, 1e-3)
    g = rnd(6, n, 1e-3)
    g[:16] = 0.0
    m0[:8] = 0.0                                  # c = 0 exactly: sign 0, the parameter only decays
    p, m = p0.copy(), m0.copy()
    oracle.optim32_step(oracle.LION, p, g, m, step=7, lr=lr, beta1=b1, beta2=b2, wd=wd)
    c = (np.float32(b1) * m0).astype(np.float32) + (np.float32(1 - b1) * g).astype(np.float32)
    dec = np.float32(1 - lr * wd)
    want_p = ((p0 * dec).astype(np.float32) - np.float32(lr) * np.sign(c).astype(np.float32)).astype(np.float32)
    assert np.array_equal(p, want_p)
    # every parameter moves by exactly lr (after the decay) unless c == 0
    moved = np.abs((p0 * dec).astype(np.float64) - p.astype(np.float64))
    assert np.all(moved[:8] == 0.0)
    assert np.allclose(moved[8:], lr, rtol=1e-6 * 0.02 / lr + 1e-3)
    # the momentum tracks the gradient with beta2, not beta1
    want_m = (np.float32(b2) * m0).astype(np.float32) + (np.float32(1 - b2) * g).astype(np.float32)
    assert np.array_equal(m, want_m)
    # from zero state the direction is sign(g)
    p, m = p0.copy(), np.zeros(n, np.float32)
    oracle.optim32_step(oracle.LION, p, g, m, step=1, lr=lr, beta1=b1, beta2=b2, wd=0.0)
    assert np.array_equal(p, (p0 - np.float32(lr) * np.sign(g).astype(np.float32)).astype(np.float32))


def test_sgd_first_step_takes_the_gradient():
    n = 3000
    p0, g = rnd(7, n, 0.02), rnd(8, n, 1e-3)
    p, buf = p0.copy(), rnd(9, n, 1.0)            # a stale buffer is ignored at step 1
    oracle.optim32_step(oracle.SGD, p, g, buf, step=1, lr=0.1, beta1=0.9, dampening=0.5)
    assert np.array_equal(buf, g)
    assert np.array_equal(p, (p0 - (np.float32(0.1) * g).astype(np.float32)).astype(np.float32))


STATE_KINDS = [(oracle.ADAM, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)),
               (oracle.LION, dict(lr=1e-4, beta1=0.9, beta2=0.99, wd=0.1)),
               (oracle.SGD, dict(lr=1e-2, beta1=0.9, dampening=0.0, wd=1e-4, nesterov=True)),
               (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, eps=1e-8, wd=0.0))]


@pytest.mark.parametrize("kind,hp", STATE_KINDS)
def test_8bit_state_is_the_quantized_binary32_update(kind, hp):
    """One 8-bit step = decode the states, the binary32 update, block-wise
    re-quantization: the same step on decoded binary32 states gives the same
    parameters, and quantizing its states gives the codes and absmax."""
    n, B = 2048 * 4 + 333, 2048
    two = oracle.OPTIMIZER_STATES[kind] == 2
    p0, g = rnd(10 + kind, n, 0.02), rnd(20 + kind, n, 1e-3)
    # a non-trivial state: quantize some binary32 states first
    s1 = rnd(30 + kind, n, 1e-3)
    s2 = np.abs(rnd(40 + kind, n, 1e-6))
    if kind == oracle.RMSPROP:
        s1 = np.abs(s1)
    c1, a1 = oracle.quantize_blockwise(s1, oracle.DYN8, B)
    c2, a2 = oracle.quantize_blockwise(s2, oracle.DYN8, B)
    d1 = oracle.dequantize_blockwise(c1, a1, oracle.DYN8, B, n)
    d2 = oracle.dequantize_blockwise(c2, a2, oracle.DYN8, B, n)
    step = 3
    p32, x1, x2 = p0.copy(), d1.copy(), d2.copy()
    oracle.optim32_step(kind, p32, g, x1, x2 if two else None, step=step, **hp)
    p8 = p0.copy()
    oracle.optim8bit_step(kind, p8, g, c1, a1, c2 if two else None, a2 if two else None, B, step=step, **hp)
    assert np.array_equal(p8, p32)
    q1, qa1 = oracle.quantize_blockwise(x1, oracle.DYN8, B)
    assert np.array_equal(c1, q1) and np.array_equal(a1, qa1)
    if two:
        q2, qa2 = oracle.quantize_blockwise(x2, oracle.DYN8, B)
        assert np.array_equal(c2, q2) and np.array_equal(a2, qa2)


@pytest.mark.parametrize("kind,hp", STATE_KINDS)
def test_8bit_blocks_are_independent(kind, hp):
    n, B = 2048 * 6, 2048
    two = oracle.OPTIMIZER_STATES[kind] == 2
    p, g = rnd(60, n, 0.02), rnd(61, n, 1e-3)
    c1, a1 = np.full(n, 127, np.uint8), np.zeros(n // B, np.float32)
    c2, a2 = np.full(n, 127, np.uint8), np.zeros(n // B, np.float32)
    oracle.optim8bit_step(kind, p, g, c1, a1, c2 if two else None, a2 if two else None, B, step=1, **hp)
    perm = np.random.default_rng(62).permutation(n // B)
    idx = (perm[:, None] * B + np.arange(B)).reshape(-1)
    pp, gp = rnd(60, n, 0.02)[idx], g[idx]
    e1, b1 = np.full(n, 127, np.uint8), np.zeros(n // B, np.float32)
    e2, b2 = np.full(n, 127, np.uint8), np.zeros(n // B, np.float32)
    oracle.optim8bit_step(kind, pp, gp, e1, b1, e2 if two else None, b2 if two else None, B, step=1, **hp)
    assert np.array_equal(pp, p[idx]) and np.array_equal(e1, c1[idx]) and np.array_equal(b1, a1[perm])
    if two:
        assert np.array_equal(e2, c2[idx]) and np.array_equal(b2, a2[perm])


def test_invalid_optimizer_arguments_rejected():
    p = np.zeros(10, np.float32)
    with pytest.raises(RuntimeError):
        oracle.optim32_step(oracle.SGD, p, p.copy(), p.copy(), step=1, lr=0.1, beta1=0.0)   # SGD needs momentum
    with pytest.raises(RuntimeError):
        oracle.optim32_step(7, p, p.copy(), p.copy(), step=1, lr=0.1)
    with pytest.raises(RuntimeError):
        oracle.optim32_step(oracle.LION, p, p.copy(), p.copy(), step=0, lr=0.1)
