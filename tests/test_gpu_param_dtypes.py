"""GPU parity: the fused 8-bit optimizer steps on float16 / bfloat16 parameters
(with gradients of the same dtype) against the CPU oracle, for every kind,
through the single-tensor and the multi-tensor calls.  States, codes and
absmax bit-exact; parameters bit-exact for the kinds whose parameter update is
separately rounded; AdamW and LAMB (hardware square root and reciprocal in the
binary32 update) within one unit in the last place of the 16-bit result at
every step, the oracle taking each step from the device's parameters."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu

KINDS = {
    "adamw": (oracle.ADAMW, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01), False),
    "adam": (oracle.ADAM, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01), True),
    "lion": (oracle.LION, dict(lr=1e-4, beta1=0.9, beta2=0.99, wd=0.1), True),
    "sgd": (oracle.SGD, dict(lr=1e-2, beta1=0.9, dampening=0.1, wd=1e-4), True),
    "rmsprop": (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, eps=1e-8, wd=0.01), True),
    "lamb": (oracle.LAMB, dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, wd=0.01), False),
    "lars": (oracle.LARS, dict(lr=0.5, beta1=0.9, wd=5e-4, trust=1e-3), True),
}
LAYERWISE = ("lamb", "lars")


def lib_hp(kind, hp, step):
    h = dict(hp)
    wd = h.pop("wd", 0.0)
    trust = h.pop("trust", 0.0)
    return qb().optim_hparams(kind, weight_decay=wd, step=step, trust_coefficient=trust, **h)


def half(n, seed, scale, dt):
    x = (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)
    return torch.from_numpy(x).to(TORCH_DT[dt]).view(torch.int16).numpy().view(np.uint16).copy()


def ordered(u, dt):
    """16-bit patterns to integers that order like the values (for ulp distances)."""
    w = u.astype(np.int32)
    return np.where(w & 0x8000, -(w & 0x7FFF), w & 0x7FFF)


def check_params(got, want, dt, exact, what):
    if exact:
        assert np.array_equal(got, want), f"{what}: params differ at {np.flatnonzero(got != want)[:8]}"
    else:
        d = np.abs(ordered(got, dt) - ordered(want, dt))
        assert d.max() <= 1, f"{what}: params {d.max()} ulp apart"


@pytest.mark.parametrize("name", list(KINDS))
@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_16bit_params_equal_oracle(name, dt):
    kind, hp, exact = KINDS[name]
    L = qb()
    two = oracle.OPTIMIZER_STATES[kind] == 2
    sizes = [2048 * 3 + 77, 1, 4096, 65, 300001]
    B = 2048
    host = []
    dev = []
    for i, n in enumerate(sizes):
        nb = -(-n // B)
        h = [half(n, 10 + i, 0.02, dt), np.full(n, 127, np.uint8), np.zeros(nb, np.float32),
             np.full(n, 127, np.uint8), np.zeros(nb, np.float32)]
        host.append(h)
        dev.append([to_device(h[0], TORCH_DT[dt])] + [to_device(a) for a in h[1:]])
    for step in range(1, 4):
        gs = [half(n, 100 * step + i, 1e-3, dt) for i, n in enumerate(sizes)]
        gd = [to_device(g, TORCH_DT[dt]) for g in gs]
        h = lib_hp(kind, hp, step)
        if name in LAYERWISE or step == 2:         # one multi-tensor launch
            table = L.tensor_table([(d[0], g, d[1], d[3] if two else None, d[2], d[4] if two else None)
                                    for d, g in zip(dev, gd)])
            ws = torch.empty(L.qb_optimizer_workspace_bytes(h, table, len(sizes), B), dtype=torch.uint8,
                             device=DEV)
            L.qb_multi_tensor_optimizer_step(h, table, len(sizes), dt, B, ws, pdt=dt)
        else:                                      # one call per tensor
            for d, g, n in zip(dev, gd, sizes):
                L.qb_optimizer8bit_step(h, d[0], g, n, d[1], d[3] if two else None, d[2], d[4] if two else None, B)
        for hh, g in zip(host, gs):
            oracle.optim8bit_step(kind, hh[0], g, hh[1], hh[2], hh[3] if two else None, hh[4] if two else None, B,
                                  step=step, gdt=dt, pdt=dt, **hp)
        torch.cuda.synchronize()
        for i, (hh, d) in enumerate(zip(host, dev)):
            what = f"{name} dt={dt} step {step} tensor {i}"
            for k in ((1, 2, 3, 4) if two else (1, 2)):
                assert np.array_equal(host_bits(d[k]).view(np.uint8), hh[k].view(np.uint8)), f"{what}: state {k}"
            got = host_bits(d[0])
            check_params(got, hh[0], dt, exact, what)
            hh[0][:] = got          # each step is checked from the same parameters (one rounding per step)


def test_16bit_params_with_32bit_states():
    """The binary32-state fallback on bf16 parameters: states exact, parameters bit-exact (SGD)."""
    kind, hp, _ = KINDS["sgd"]
    L = qb()
    dt, n = oracle.BF16, 3000
    p = half(n, 1, 0.02, dt)
    s = np.zeros(n, np.float32)
    pd, sd = to_device(p, TORCH_DT[dt]), to_device(s)
    for step in range(1, 4):
        g = half(n, 50 + step, 1e-3, dt)
        L.qb_optimizer8bit_step(lib_hp(kind, hp, step), pd, to_device(g, TORCH_DT[dt]), n, sd, None, None, None,
                                2048)
        oracle.optim32_step(kind, p, g, s, step=step, gdt=dt, pdt=dt, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(pd), p) and np.array_equal(host_bits(sd).view(np.uint32), s.view(np.uint32))
