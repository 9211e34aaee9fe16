"""GPU parity: libqb's fused 8-bit Adam, Lion, SGD (momentum) and RMSprop
steps (qb_optimizer8bit_step, qb_multi_tensor_optimizer_step) against the CPU
oracle.  State codes and absmax bit-exact; parameters bit-exact too, except
for AdamW (within 1e-6 relative of the parameter scale), whose states never
read the parameters."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device

pytestmark = pytest.mark.gpu

# (oracle kind, hyperparameters, parameters bit-exact)
KINDS = {
    "adam": (oracle.ADAM, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01), True),
    "lion": (oracle.LION, dict(lr=1e-4, beta1=0.9, beta2=0.99, wd=0.1), True),
    "sgd": (oracle.SGD, dict(lr=1e-2, beta1=0.9, dampening=0.1, wd=1e-4), True),
    "sgd_nesterov": (oracle.SGD, dict(lr=1e-2, beta1=0.9, dampening=0.0, wd=1e-4, nesterov=True), True),
    "rmsprop": (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, eps=1e-8, wd=0.01), True),
    "adamw": (oracle.ADAMW, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01), False),
}


def lib_hp(kind, hp, step):
    h = dict(hp)
    wd = h.pop("wd", 0.0)
    return qb().optim_hparams(kind, weight_decay=wd, step=step, **h)


class State:
    def __init__(self, kind, n, B, seed):
        rng = np.random.default_rng(seed)
        nb = (n + B - 1) // B
        self.kind, self.n, self.B = kind, n, B
        self.two = oracle.OPTIMIZER_STATES[kind] == 2
        self.p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        self.c1 = np.full(n, 127, np.uint8)
        self.a1 = np.zeros(nb, np.float32)
        self.c2 = np.full(n, 127, np.uint8)
        self.a2 = np.zeros(nb, np.float32)

    def device(self):
        d = [to_device(a) for a in (self.p, self.c1, self.a1)]
        d += [to_device(self.c2), to_device(self.a2)] if self.two else [None, None]
        return d

    def oracle_step(self, g, step, gdt, hp):
        oracle.optim8bit_step(self.kind, self.p, g, self.c1, self.a1, self.c2 if self.two else None,
                              self.a2 if self.two else None, self.B, step=step, gdt=gdt, **hp)


def grad(n, seed, gdt):
    g = (np.random.default_rng(seed).standard_normal(n) * 1e-3).astype(np.float32)
    if gdt == oracle.F32:
        return g
    return torch.from_numpy(g).to(TORCH_DT[gdt]).view(torch.int16).numpy().view(np.uint16).copy()


def assert_equal_state(d, st, exact_p, what):
    p, c1, a1 = host_bits(d[0]), host_bits(d[1]), host_bits(d[2])
    assert np.array_equal(c1, st.c1), f"{what}: state-1 codes differ at {np.flatnonzero(c1 != st.c1)[:8]}"
    assert np.array_equal(a1.view(np.uint32), st.a1.view(np.uint32)), f"{what}: absmax 1"
    if st.two:
        c2, a2 = host_bits(d[3]), host_bits(d[4])
        assert np.array_equal(c2, st.c2), f"{what}: state-2 codes differ"
        assert np.array_equal(a2.view(np.uint32), st.a2.view(np.uint32)), f"{what}: absmax 2"
    if exact_p:
        assert np.array_equal(p.view(np.uint32), st.p.view(np.uint32)), f"{what}: params differ"
    else:
        np.testing.assert_allclose(p, st.p, rtol=1e-6, atol=1e-6 * 0.02, err_msg=f"{what}: params")


def run(name, n, B, gdt, steps, seed):
    kind, hp, exact_p = KINDS[name]
    L = qb()
    st = State(kind, n, B, seed)
    d = st.device()
    for step in range(1, steps + 1):
        g = grad(n, seed * 1000 + step, gdt)
        L.qb_optimizer8bit_step(lib_hp(kind, hp, step), d[0], to_device(g, TORCH_DT[gdt]), n, d[1], d[3], d[2],
                                d[4], B)
        st.oracle_step(g, step, gdt, hp)
        torch.cuda.synchronize()
        assert_equal_state(d, st, exact_p, f"{name} step {step}")


@pytest.mark.parametrize("name", list(KINDS))
def test_ten_steps_free_running(name):
    run(name, 2048 * 37 + 1000, 2048, oracle.F32, 10, seed=11)


@pytest.mark.parametrize("name", list(KINDS))
@pytest.mark.parametrize("B,gdt", [(64, oracle.BF16), (256, oracle.F16), (4096, oracle.BF16), (1024, oracle.F32)])
def test_blocksizes_and_grad_dtypes(name, B, gdt):
    run(name, B * 9 + 37, B, gdt, 3, seed=B + gdt)


@pytest.mark.parametrize("name", ["lion", "sgd", "rmsprop"])
@pytest.mark.parametrize("n", [1, 2, 3, 255, 2049])
def test_small_and_ragged(name, n):
    run(name, n, 2048, oracle.BF16, 3, seed=n)


def test_adamw_generic_entry_equals_adamw8bit_step():
    kind, hp, _ = KINDS["adamw"]
    L = qb()
    n, B = 2048 * 5 + 17, 2048
    a, b = State(kind, n, B, 3).device(), State(kind, n, B, 3).device()
    for step in range(1, 4):
        g = to_device(grad(n, 40 + step, oracle.BF16), torch.bfloat16)
        L.qb_optimizer8bit_step(lib_hp(kind, hp, step), a[0], g, n, a[1], a[3], a[2], a[4], B)
        L.qb_adamw8bit_step(b[0], g, n, b[1], b[3], b[2], b[4], B,
                            L.hparams(lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                      weight_decay=hp["wd"], step=step))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["adam", "lion", "sgd", "rmsprop"])
def test_multi_tensor_equals_loop_and_oracle(name):
    kind, hp, exact_p = KINDS[name]
    L = qb()
    sizes = [1, 4096, 65, 2048 * 3 + 17, 300000, 0, 2048, 123457, 8]
    B, gdt = 2048, oracle.BF16
    states = [State(kind, n, B, 100 + i) for i, n in enumerate(sizes)]
    dm = [s.device() for s in states]
    ds = [s.device() for s in states]
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    for step in range(1, 4):
        gs = [grad(max(n, 1), 7000 + 10 * i + step, gdt)[:n] for i, n in enumerate(sizes)]
        gd = [to_device(g if g.size else np.zeros(1, np.uint16), TORCH_DT[gdt]) for g in gs]
        table = L.tensor_table([(d[0], g, d[1], d[3], d[2], d[4]) for d, g in zip(dm, gd)])
        for i, n in enumerate(sizes):
            table[i].n = n
        L.qb_multi_tensor_optimizer_step(lib_hp(kind, hp, step), table, len(sizes), L.QB_BF16, B, ws)
        for d, g, n in zip(ds, gd, sizes):
            L.qb_optimizer8bit_step(lib_hp(kind, hp, step), d[0], g, n, d[1], d[3], d[2], d[4], B)
        for s, g in zip(states, gs):
            if s.n:
                s.oracle_step(g, step, gdt, hp)
        torch.cuda.synchronize()
        for a, b, s in zip(dm, ds, states):
            for x, y in zip(a, b):
                if x is not None:
                    assert torch.equal(x, y), f"{name}: multi-tensor differs from the single-tensor loop"
            if s.n:
                assert_equal_state(a, s, exact_p, f"{name} step {step}")


def test_sgd_first_step_ignores_stale_state():
    """At step 1 SGD's momentum buffer is the gradient, whatever the state held."""
    kind, hp, _ = KINDS["sgd"]
    L = qb()
    n, B = 4096 + 5, 2048
    st = State(kind, n, B, 9)
    st.c1 = np.random.default_rng(1).integers(0, 256, n).astype(np.uint8)
    st.a1 = np.full(st.a1.shape, 3.0, np.float32)
    d = st.device()
    g = grad(n, 5, oracle.F32)
    L.qb_optimizer8bit_step(lib_hp(kind, hp, 1), d[0], to_device(g), n, d[1], None, d[2], None, B)
    st.oracle_step(g, 1, oracle.F32, hp)
    torch.cuda.synchronize()
    assert_equal_state(d, st, True, "sgd step 1")


@pytest.mark.parametrize("name", ["adamw", "adam", "lion", "sgd", "rmsprop"])
def test_mixed_8bit_and_32bit_states_in_one_launch(name):
    """The 32-bit fallback: tensors under min_8bit_size (and one marked 32-bit)
    keep binary32 states in the same multi-tensor launch.  Their states and
    parameters are exactly the oracle's binary32 step (within 1e-6 for AdamW's
    parameters); the 8-bit tensors as before."""
    from bit_optimizer_states_amd import state as policy
    kind, hp, exact_p = KINDS[name]
    L = qb()
    sizes = [4096, 100, 2048 * 5 + 3, 4095, 1, 30000]
    B, gdt = 2048, oracle.BF16
    rng = np.random.default_rng(kind + 5)
    ps = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    pd = [to_device(p) for p in ps]
    states = policy.allocate(pd, kind, blocksize=B, min_8bit_size=4096, force_32bit={5})
    eight = [policy.uses_8bit(n, 4096, i == 5) for i, n in enumerate(sizes)]
    assert eight == [True, False, True, False, False, False]
    two = oracle.OPTIMIZER_STATES[kind] == 2
    host = []
    for n, e in zip(sizes, eight):
        nb = (n + B - 1) // B
        if e:
            host.append([np.full(n, 127, np.uint8), np.zeros(nb, np.float32), np.full(n, 127, np.uint8),
                         np.zeros(nb, np.float32)])
        else:
            host.append([np.zeros(n, np.float32), None, np.zeros(n, np.float32), None])
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    for step in range(1, 4):
        gs = [grad(n, 900 + 10 * i + step, gdt) for i, n in enumerate(sizes)]
        gd = [to_device(g, TORCH_DT[gdt]) for g in gs]
        table = L.tensor_table([(p, g, s1, s2, a1, a2) for p, g, (s1, s2, a1, a2) in zip(pd, gd, states)])
        L.qb_multi_tensor_optimizer_step(lib_hp(kind, hp, step), table, len(sizes), L.QB_BF16, B, ws)
        for p, g, h, e in zip(ps, gs, host, eight):
            if e:
                oracle.optim8bit_step(kind, p, g, h[0], h[1], h[2] if two else None, h[3] if two else None, B,
                                      step=step, gdt=gdt, **hp)
            else:
                oracle.optim32_step(kind, p, g, h[0], h[2] if two else None, step=step, gdt=gdt, **hp)
        torch.cuda.synchronize()
        for i, (p, h, e, (s1, s2, a1, a2)) in enumerate(zip(ps, host, eight, states)):
            got_p = host_bits(pd[i])
            if exact_p:
                assert np.array_equal(got_p.view(np.uint32), p.view(np.uint32)), (name, step, i)
            else:
                np.testing.assert_allclose(got_p, p, rtol=1e-6, atol=1e-6 * 0.02)
            assert np.array_equal(host_bits(s1).view(np.uint8), h[0].view(np.uint8)), (name, step, i, "state 1")
            if two:
                assert np.array_equal(host_bits(s2).view(np.uint8), h[2].view(np.uint8)), (name, step, i, "state 2")
            if e:
                assert np.array_equal(host_bits(a1).view(np.uint32), h[1].view(np.uint32))
                if two:
                    assert np.array_equal(host_bits(a2).view(np.uint32), h[3].view(np.uint32))
