"""GPU parity: libqb's fused 8-bit AdamW step (single tensor and multi-tensor)
against the CPU oracle.  State codes and absmax are compared bit-exact; the
parameters within 1e-6 relative (of the parameter scale)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
P_RTOL = 1e-6


def hparams(step):
    return qb().hparams(lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"], weight_decay=HP["wd"],
                        step=step)


class State:
    """Host state + device mirror of one tensor."""

    def __init__(self, n, B, seed):
        rng = np.random.default_rng(seed)
        self.n, self.B = n, B
        nb = (n + B - 1) // B
        self.p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        self.m = np.full(n, 127, np.uint8)
        self.v = np.full(n, 127, np.uint8)
        self.am = np.zeros(nb, np.float32)
        self.av = np.zeros(nb, np.float32)

    def device(self):
        return [to_device(a) for a in (self.p, self.m, self.v, self.am, self.av)]


def grad(n, seed, gdt):
    g = (np.random.default_rng(seed).standard_normal(n) * 1e-3).astype(np.float32)
    if gdt == oracle.F32:
        return g
    return torch.from_numpy(g).to(TORCH_DT[gdt]).view(torch.int16).numpy().view(np.uint16).copy()


def assert_state_equal(dev_state, st, what=""):
    p, m, v, am, av = (host_bits(t) for t in dev_state)
    assert np.array_equal(m, st.m), f"{what} m codes differ at {np.flatnonzero(m != st.m)[:8]}"
    assert np.array_equal(v, st.v), f"{what} v codes differ at {np.flatnonzero(v != st.v)[:8]}"
    assert np.array_equal(am.view(np.uint32), st.am.view(np.uint32)), f"{what} absmax_m"
    assert np.array_equal(av.view(np.uint32), st.av.view(np.uint32)), f"{what} absmax_v"
    np.testing.assert_allclose(p, st.p, rtol=P_RTOL, atol=P_RTOL * 0.02, err_msg=f"{what} params")


def run_steps(n, B, gdt, steps, seed, grad_fn=None):
    st = State(n, B, seed)
    d = st.device()
    L = qb()
    for step in range(1, steps + 1):
        g = grad_fn(step) if grad_fn else grad(n, seed * 1000 + step, gdt)
        gd = to_device(g, TORCH_DT[gdt])
        L.qb_adamw8bit_step(d[0], gd, n, d[1], d[2], d[3], d[4], B, hparams(step))
        oracle.adamw8bit_step(st.p, g, st.m, st.v, st.am, st.av, B, step=step, gdt=gdt, **HP)
        torch.cuda.synchronize()
        assert_state_equal(d, st, f"step {step}")
    return st, d


def test_config1_ten_steps_free_running():
    """1,048,576 fp32 params, fp32 grads, B = 2048, 10 steps."""
    run_steps(1 << 20, 2048, oracle.F32, 10, seed=1)


@pytest.mark.parametrize("B", [64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("gdt", [oracle.F32, oracle.F16, oracle.BF16])
def test_blocksizes_and_grad_dtypes(B, gdt):
    run_steps(3 * 4096 * 4 + 1234, B, gdt, 3, seed=B + 10 * gdt)


@pytest.mark.parametrize("n", [1, 3, 63, 64, 65, 2047, 2049, 4097])
def test_small_and_ragged(n):
    run_steps(n, 2048, oracle.BF16, 3, seed=n)


def test_zero_and_extreme_gradients():
    n, B = 2048 * 8, 2048

    def gfn(step):
        g = (np.random.default_rng(step).standard_normal(n) * 1e-3).astype(np.float32)
        g[0:B] = 0.0                                  # an all-zero block every step
        g[B:2 * B] *= np.float32(1e-25)               # moments far below 2^-60
        g[2 * B:3 * B] *= np.float32(1e12)            # moments far above 2^60
        g[3 * B + 5] = 3.0                            # one outlier
        if step == 2:
            g[4 * B:5 * B] = 0.0                      # a block that goes quiet
        return g

    run_steps(n, B, oracle.F32, 4, seed=7, grad_fn=gfn)


def test_multi_tensor_equals_loop_and_oracle():
    rng = np.random.default_rng(11)
    sizes = [1, 4096, 65, 2048 * 3 + 17, 300000, 4096, 2048, 123457, 0, 8]
    B, gdt = 2048, oracle.BF16
    L = qb()
    states = [State(n, B, 100 + i) for i, n in enumerate(sizes)]
    dm = [s.device() for s in states]                 # multi-tensor copies
    ds = [s.device() for s in states]                 # single-tensor copies
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    for step in range(1, 4):
        gs = [grad(max(n, 1), 7000 + 10 * i + step, gdt)[:n] for i, n in enumerate(sizes)]
        gd = [to_device(g if g.size else np.zeros(1, np.uint16), TORCH_DT[gdt]) for g in gs]
        table = L.tensor_table([(d[0], g, d[1], d[2], d[3], d[4]) for d, g in zip(dm, gd)])
        for i, n in enumerate(sizes):
            table[i].n = n
        L.qb_multi_tensor_step(table, len(sizes), L.QB_BF16, B, hparams(step), ws)
        for d, g, n in zip(ds, gd, sizes):
            L.qb_adamw8bit_step(d[0], g, n, d[1], d[2], d[3], d[4], B, hparams(step))
        for s, g in zip(states, gs):
            if s.n:
                oracle.adamw8bit_step(s.p, g, s.m, s.v, s.am, s.av, B, step=step, gdt=gdt, **HP)
        torch.cuda.synchronize()
        for a, b, s in zip(dm, ds, states):
            for x, y in zip(a, b):
                assert torch.equal(x, y), "multi-tensor differs from the single-tensor loop"
            assert_state_equal(a, s, f"step {step}")


@pytest.mark.parametrize("B", [256, 2048])
def test_multi_tensor_many_small_tensors(B):
    # far more tensors than tiles per bucket of the coarse tile index: buckets
    # that span many tensors, empty tensors between them, one-element tensors
    rng = np.random.default_rng(B)
    sizes = [int(x) for x in rng.integers(1, 5000, size=300)]
    for i in (0, 17, 150, 299):
        sizes[i] = 0
    sizes[5] = 1
    sizes[200] = 2048 * 40 + 3
    gdt = oracle.BF16
    L = qb()
    states = [State(n, B, 900 + i) for i, n in enumerate(sizes)]
    dm = [s.device() for s in states]
    ds = [s.device() for s in states]
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    for step in range(1, 3):
        gs = [grad(max(n, 1), 80000 + 10 * i + step, gdt)[:n] for i, n in enumerate(sizes)]
        gd = [to_device(g if g.size else np.zeros(1, np.uint16), TORCH_DT[gdt]) for g in gs]
        table = L.tensor_table([(d[0], g, d[1], d[2], d[3], d[4]) for d, g in zip(dm, gd)])
        for i, n in enumerate(sizes):
            table[i].n = n
        L.qb_multi_tensor_step(table, len(sizes), L.QB_BF16, B, hparams(step), ws)
        for d, g, n in zip(ds, gd, sizes):
            L.qb_adamw8bit_step(d[0], g, n, d[1], d[2], d[3], d[4], B, hparams(step))
        for s, g in zip(states, gs):
            if s.n:
                oracle.adamw8bit_step(s.p, g, s.m, s.v, s.am, s.av, B, step=step, gdt=gdt, **HP)
        torch.cuda.synchronize()
        for a, b, s in zip(dm, ds, states):
            for x, y in zip(a, b):
                assert torch.equal(x, y), "multi-tensor differs from the single-tensor loop"
            assert_state_equal(a, s, f"step {step}")


def test_resume_equals_straight_run():
    n, B, gdt = 2048 * 40 + 99, 2048, oracle.BF16
    L = qb()
    straight = State(n, B, 5).device()
    resumed = State(n, B, 5).device()
    for step in range(1, 11):
        g = to_device(grad(n, 555 + step, gdt), TORCH_DT[gdt])
        L.qb_adamw8bit_step(straight[0], g, n, straight[1], straight[2], straight[3], straight[4], B, hparams(step))
        L.qb_adamw8bit_step(resumed[0], g, n, resumed[1], resumed[2], resumed[3], resumed[4], B, hparams(step))
        if step == 5:                                  # checkpoint to host and back
            torch.cuda.synchronize()
            resumed = [t.cpu().clone().to(DEV) for t in resumed]
    torch.cuda.synchronize()
    for a, b in zip(straight, resumed):
        assert torch.equal(a, b)
