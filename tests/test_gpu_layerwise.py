"""GPU parity: the layer-wise 8-bit optimizers LAMB and LARS
(qb_multi_tensor_optimizer_step) against the CPU oracle, one oracle call per
tensor (one tensor = one layer).  State codes and absmax bit-exact; LARS
parameters bit-exact; LAMB parameters within 1e-6 relative of the parameter
scale (its states never read p, and its step takes hardware square root and
reciprocal, as AdamW's)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu

KINDS = {
    "lamb": (oracle.LAMB, dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, wd=0.01), False),
    "lars": (oracle.LARS, dict(lr=0.5, beta1=0.9, wd=5e-4, trust=0.001), True),
}


def lib_hp(kind, hp, step):
    h = dict(hp)
    wd = h.pop("wd", 0.0)
    trust = h.pop("trust", 0.0)
    return qb().optim_hparams(kind, weight_decay=wd, step=step, trust_coefficient=trust, **h)


def grad(n, seed, gdt, scale=1e-3):
    g = (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)
    if gdt == oracle.F32:
        return g
    return torch.from_numpy(g).to(TORCH_DT[gdt]).view(torch.int16).numpy().view(np.uint16).copy()


class Layer:
    """One tensor: host oracle state and its device copy (8-bit or binary32 states)."""

    def __init__(self, kind, n, B, seed, scale=0.02, eight=True):
        rng = np.random.default_rng(seed)
        nb = (n + B - 1) // B
        self.kind, self.n, self.B, self.eight, self.scale = kind, n, B, eight, scale
        self.two = oracle.OPTIMIZER_STATES[kind] == 2
        self.p = (rng.standard_normal(n) * scale).astype(np.float32)
        if eight:
            self.s1, self.a1 = np.full(n, 127, np.uint8), np.zeros(nb, np.float32)
            self.s2, self.a2 = np.full(n, 127, np.uint8), np.zeros(nb, np.float32)
        else:
            self.s1, self.a1 = np.zeros(n, np.float32), None
            self.s2, self.a2 = np.zeros(n, np.float32), None
        dev = lambda a: None if a is None else to_device(a if a.size else np.zeros(16, a.dtype))
        self.d = [dev(self.p), dev(self.s1), dev(self.a1), dev(self.s2) if self.two else None,
                  dev(self.a2) if self.two else None]

    def oracle_step(self, g, step, gdt, hp):
        if self.n == 0:
            return
        if self.eight:
            oracle.optim8bit_step(self.kind, self.p, g, self.s1, self.a1, self.s2 if self.two else None,
                                  self.a2 if self.two else None, self.B, step=step, gdt=gdt, **hp)
        else:
            oracle.optim32_step(self.kind, self.p, g, self.s1, self.s2 if self.two else None, step=step, gdt=gdt,
                                **hp)

    def check(self, exact_p, what):
        if self.n == 0:
            return
        p = host_bits(self.d[0])[:self.n]
        pairs = [(self.d[1], self.s1), (self.d[2], self.a1)]
        if self.two:
            pairs += [(self.d[3], self.s2), (self.d[4], self.a2)]
        for k, (dv, hv) in enumerate(pairs):
            if hv is None:
                continue
            got = host_bits(dv)[:hv.size]
            assert np.array_equal(got.view(np.uint8), hv.view(np.uint8)), \
                f"{what}: state array {k} differs at {np.flatnonzero(got != hv)[:8]}"
        if exact_p:
            assert np.array_equal(p.view(np.uint32), self.p.view(np.uint32)), \
                f"{what}: params differ at {np.flatnonzero(p != self.p)[:8]}"
        else:
            np.testing.assert_allclose(p, self.p, rtol=1e-6, atol=1e-6 * self.scale, err_msg=f"{what}: params")


def step_all(L, kind, hp, layers, step, gdt, B, seed):
    gs = [grad(max(l.n, 1), seed + 10 * i + step, gdt)[:l.n] for i, l in enumerate(layers)]
    gd = [to_device(g if g.size else np.zeros(8, g.dtype), TORCH_DT[gdt]) for g in gs]
    table = L.tensor_table([(l.d[0], g, l.d[1], l.d[3], l.d[2], l.d[4]) for l, g in zip(layers, gd)])
    for i, l in enumerate(layers):
        table[i].n = l.n
    h = lib_hp(kind, hp, step)
    ws = torch.empty(L.qb_optimizer_workspace_bytes(h, table, len(layers), B), dtype=torch.uint8, device=DEV)
    L.qb_multi_tensor_optimizer_step(h, table, len(layers), gdt, B, ws)
    for l, g in zip(layers, gs):
        l.oracle_step(g, step, gdt, hp)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", list(KINDS))
@pytest.mark.parametrize("B,gdt", [(2048, oracle.BF16), (256, oracle.F16), (64, oracle.F32), (4096, oracle.BF16)])
def test_layers_equal_oracle(name, B, gdt):
    kind, hp, exact_p = KINDS[name]
    L = qb()
    sizes = [1, 4096, 65, 2048 * 3 + 17, 300000, 0, 2048, 123457, 8]
    scales = [0.02, 0.5, 1e-3, 0.02, 0.05, 0.02, 3.0, 0.01, 0.02]
    layers = [Layer(kind, n, B, 40 + i, s) for i, (n, s) in enumerate(zip(sizes, scales))]
    for step in range(1, 5):
        step_all(L, kind, hp, layers, step, gdt, B, 5000)
        for i, l in enumerate(layers):
            l.check(exact_p, f"{name} B={B} step {step} layer {i}")


@pytest.mark.parametrize("name", list(KINDS))
def test_one_large_layer(name):
    kind, hp, exact_p = KINDS[name]
    L = qb()
    layers = [Layer(kind, (1 << 22) + 333, 2048, 7)]
    for step in range(1, 3):
        step_all(L, kind, hp, layers, step, oracle.BF16, 2048, 900)
        layers[0].check(exact_p, f"{name} step {step}")


@pytest.mark.parametrize("name", list(KINDS))
def test_mixed_8bit_and_32bit_layers(name):
    kind, hp, exact_p = KINDS[name]
    L = qb()
    sizes = [4096, 100, 2048 * 5 + 3, 4095, 1, 30000]
    eight = [True, False, True, False, False, True]
    layers = [Layer(kind, n, 2048, 60 + i, eight=e) for i, (n, e) in enumerate(zip(sizes, eight))]
    for step in range(1, 4):
        step_all(L, kind, hp, layers, step, oracle.BF16, 2048, 700)
        for i, l in enumerate(layers):
            l.check(exact_p, f"{name} step {step} layer {i}")


@pytest.mark.parametrize("name", list(KINDS))
def test_zero_layers_and_repeatability(name):
    """A layer of zeros takes ratio 1 (as the oracle); and the same step on the
    same inputs gives the same bits on every run (the norms add in a fixed order)."""
    kind, hp, exact_p = KINDS[name]
    L = qb()
    runs = []
    for _ in range(2):
        layers = [Layer(kind, 50000, 2048, 3), Layer(kind, 3000, 2048, 4, scale=0.0)]
        step_all(L, kind, hp, layers, 1, oracle.F32, 2048, 11)
        for i, l in enumerate(layers):
            l.check(exact_p, f"{name} layer {i}")
        runs.append([host_bits(a) for a in layers[0].d if a is not None])
    for a, b in zip(*runs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("name", list(KINDS))
def test_many_small_layers(name):
    """300 layers of 0 to 5,000 elements in one call: the coarse index of the
    tile and group maps spans many tensors per bucket; every layer against its
    own oracle call."""
    kind, hp, exact_p = KINDS[name]
    L = qb()
    rng = np.random.default_rng(77)
    sizes = [int(v) for v in rng.integers(0, 5000, 300)]
    sizes[::37] = [0] * len(sizes[::37])
    layers = [Layer(kind, n, 256, 1000 + i, scale=float(rng.uniform(0.005, 0.5))) for i, n in enumerate(sizes)]
    for step in range(1, 3):
        step_all(L, kind, hp, layers, step, oracle.BF16, 256, 3000)
        for i, l in enumerate(layers):
            l.check(exact_p, f"{name} step {step} layer {i}")
