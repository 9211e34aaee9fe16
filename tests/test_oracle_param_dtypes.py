"""Pins of the oracle's optimizer step on 16-bit parameters (CPU only).

Reading: a float16 / bfloat16 parameter is widened to binary32 (exact), takes
the binary32 update of its kind, and is rounded once to nearest even back to
its dtype; the gradient has the parameter's dtype (16-bit training next to the
8-bit optimizer: "bitsandbytes - Quantização de LLM", section Workflow 3).
The conversions are pinned against torch's (an independent implementation),
the step by the exact properties the reading implies.
"""
import numpy as np
import pytest
import torch

import oracle

TDT = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}
KINDS = [(oracle.ADAMW, dict(lr=1e-3, wd=0.01)), (oracle.ADAM, dict(lr=1e-3, wd=0.01)),
         (oracle.LION, dict(lr=1e-4, beta2=0.99, wd=0.1)), (oracle.SGD, dict(lr=1e-2, beta1=0.9, wd=1e-4)),
         (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, wd=0.01)), (oracle.LAMB, dict(lr=2e-3, eps=1e-6, wd=0.01)),
         (oracle.LARS, dict(lr=0.5, beta1=0.9, wd=5e-4, trust=1e-3))]


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_conversions_equal_torch(dt):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-8, 1e-3, 1.0, 1e3)]).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 65504.0, 65520.0, 1e-7, -3e-8])])
    want = bits(torch.from_numpy(x).to(TDT[dt]))
    got = oracle.convert(x, oracle.F32, dt)
    assert np.array_equal(got, want)
    back = oracle.convert(got, dt, oracle.F32)
    assert np.array_equal(back.view(np.uint32),
                          torch.from_numpy(got.view(np.int16)).view(TDT[dt]).float().numpy().view(np.uint32))


def half_params(n, seed, dt):
    p = (np.random.default_rng(seed).standard_normal(n) * 0.02).astype(np.float32)
    return bits(torch.from_numpy(p).to(TDT[dt]))


def half_grad(n, seed, dt):
    g = (np.random.default_rng(seed).standard_normal(n) * 1e-3).astype(np.float32)
    return bits(torch.from_numpy(g).to(TDT[dt]))


@pytest.mark.parametrize("kind,hp", KINDS)
@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_step_is_the_binary32_step_rounded_by_torch(kind, hp, dt):
    """One 8-bit step on 16-bit parameters equals the binary32-parameter step
    from the widened values, with the result rounded by torch's conversion;
    states bit for bit."""
    n, B = 2048 * 3 + 77, 2048
    two = oracle.OPTIMIZER_STATES[kind] == 2
    ph, g = half_params(n, 2, dt), half_grad(n, 3, dt)
    nb = -(-n // B)
    st = [np.full(n, 127, np.uint8), np.zeros(nb, np.float32), np.full(n, 127, np.uint8), np.zeros(nb, np.float32)]
    st32 = [a.copy() for a in st]
    oracle.optim8bit_step(kind, ph, g, st[0], st[1], st[2] if two else None, st[3] if two else None, B,
                          step=1, gdt=dt, pdt=dt, **hp)
    p32 = torch.from_numpy(half_params(n, 2, dt).view(np.int16)).view(TDT[dt]).float().numpy()
    oracle.optim8bit_step(kind, p32, g, st32[0], st32[1], st32[2] if two else None, st32[3] if two else None, B,
                          step=1, gdt=dt, **hp)
    assert np.array_equal(ph, bits(torch.from_numpy(p32).to(TDT[dt])))
    for a, b in zip(st[:4 if two else 2], st32[:4 if two else 2]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_updates_below_half_an_ulp_are_lost(dt):
    # the one rounding per step: a step smaller than half a unit in the last
    # place leaves the parameter unchanged (SGD, lr so small that every
    # |lr * g| < ulp(p) / 2)
    n = 4096
    p = half_params(n, 4, dt)
    pw = oracle.convert(p, dt, oracle.F32)
    ulp = np.spacing(np.abs(pw)).astype(np.float64) * (2.0 ** (13 if dt == oracle.F16 else 16))
    g = half_grad(n, 5, dt)
    gw = oracle.convert(g, dt, oracle.F32).astype(np.float64)
    lr = 0.4 * float(np.min(ulp / np.maximum(np.abs(gw), 1e-30)))
    before = p.copy()
    oracle.optim32_step(oracle.SGD, p, g, np.zeros(n, np.float32), step=1, lr=lr, beta1=0.9, gdt=dt, pdt=dt)
    assert np.array_equal(p, before)


def test_adamw_states_do_not_depend_on_the_parameter_dtype():
    # AdamW's states never read p: over several steps they equal the binary32
    # parameter run's, bit for bit, while the parameters differ
    n, B = 5000, 2048
    ph = half_params(n, 6, oracle.BF16)
    p32 = oracle.convert(ph, oracle.BF16, oracle.F32)
    s16 = [np.full(n, 127, np.uint8), np.zeros(3, np.float32), np.full(n, 127, np.uint8), np.zeros(3, np.float32)]
    s32 = [a.copy() for a in s16]
    for step in range(1, 5):
        g = half_grad(n, 10 + step, oracle.BF16)
        oracle.optim8bit_step(oracle.ADAMW, ph, g, s16[0], s16[1], s16[2], s16[3], B, step=step, gdt=oracle.BF16,
                              pdt=oracle.BF16, lr=1e-3, wd=0.01)
        oracle.optim8bit_step(oracle.ADAMW, p32, g, s32[0], s32[1], s32[2], s32[3], B, step=step,
                              gdt=oracle.BF16, lr=1e-3, wd=0.01)
        for a, b in zip(s16, s32):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert not np.array_equal(oracle.convert(ph, oracle.BF16, oracle.F32), p32)
