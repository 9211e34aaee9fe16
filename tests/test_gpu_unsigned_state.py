"""GPU parity: the 8-bit steps with the never-negative state (v of AdamW, Adam
and LAMB; the state of RMSprop) held in the unsigned dynamic code
(qb_optim_hparams.v_code = QB_UDYN8), against the CPU oracle.  State codes and
absmax bit-exact; parameters bit-exact except AdamW and LAMB (1e-6 relative),
as for the signed code.  Ragged tensors cover partial tiles, whose missing
elements must count as the unsigned code of 0.0; one launch mixes 8-bit and
binary32 states; the paged step equals the device-resident one bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, host_bits, qb, to_device
from test_gpu_param_dtypes import KINDS, LAYERWISE, lib_hp

pytestmark = pytest.mark.gpu

NONNEG = ["adamw", "adam", "rmsprop", "lamb"]


def fresh(kind, n, B, seed, eight=True):
    """Host state of one tensor: p, then (s1, a1, s2, a2); 8-bit codes of 0.0
    (127 signed, 0 unsigned) or binary32 zeros."""
    p = (np.random.default_rng(seed).standard_normal(n) * 0.02).astype(np.float32)
    nb = -(-n // B)
    if not eight:
        return [p, np.zeros(n, np.float32), None, np.zeros(n, np.float32), None]
    z1 = 0 if kind == oracle.RMSPROP else 127
    return [p, np.full(n, z1, np.uint8), np.zeros(nb, np.float32), np.full(n, 0, np.uint8), np.zeros(nb, np.float32)]


def dev_of(h):
    return [None if a is None else to_device(a if a.size else np.zeros(16, a.dtype)) for a in h]


def oracle_step(kind, h, g, B, step, hp, gdt):
    two = oracle.OPTIMIZER_STATES[kind] == 2
    if h[0].size == 0:
        return
    if h[2] is None:
        oracle.optim32_step(kind, h[0], g, h[1], h[3] if two else None, step=step, gdt=gdt, **hp)
    else:
        oracle.optim8bit_step(kind, h[0], g, h[1], h[2], h[3] if two else None, h[4] if two else None, B,
                              step=step, gdt=gdt, vcode=oracle.UDYN8, **hp)


def check(kind, h, d, exact, what):
    two = oracle.OPTIMIZER_STATES[kind] == 2
    n = h[0].size
    if not n:
        return
    for k in ((1, 2, 3, 4) if two else (1, 2)):
        if h[k] is None:
            continue
        got = host_bits(d[k])[:h[k].size]
        assert np.array_equal(got.view(np.uint8), h[k].view(np.uint8)), \
            f"{what}: state array {k} differs at {np.flatnonzero(got != h[k])[:8]}"
    p = host_bits(d[0])[:n]
    if exact:
        assert np.array_equal(p.view(np.uint32), h[0].view(np.uint32)), f"{what}: params"
    else:
        np.testing.assert_allclose(p, h[0], rtol=1e-6, atol=2e-8, err_msg=f"{what}: params")
    h[0][:] = p          # the next step starts from the device's parameters


def grads(sizes, seed, gdt):
    rng = np.random.default_rng(seed)
    out = []
    for n in sizes:
        g = (rng.standard_normal(max(n, 1)) * 1e-3).astype(np.float32)[:n]
        if gdt != oracle.F32:
            g = torch.from_numpy(g).to(TORCH_DT[gdt]).view(torch.int16).numpy().view(np.uint16).copy()
        out.append(g)
    return out


def run(name, sizes, B, gdt, steps, multi, eight=None, seed=0):
    kind, hp, exact = KINDS[name]
    L = qb()
    two = oracle.OPTIMIZER_STATES[kind] == 2
    eight = eight or [True] * len(sizes)
    host = [fresh(kind, n, B, seed + i, e) for i, (n, e) in enumerate(zip(sizes, eight))]
    dev = [dev_of(h) for h in host]
    for step in range(1, steps + 1):
        gs = grads(sizes, seed * 100 + step, gdt)
        gd = [to_device(g if g.size else np.zeros(8, g.dtype), TORCH_DT[gdt]) for g in gs]
        h = lib_hp(kind, hp, step)
        h.v_code = qb().QB_UDYN8
        if multi:
            table = L.tensor_table([(d[0], g, d[1], d[3] if two else None, d[2], d[4] if two else None)
                                    for d, g in zip(dev, gd)])
            for i, n in enumerate(sizes):
                table[i].n = n
            ws = torch.empty(L.qb_optimizer_workspace_bytes(h, table, len(sizes), B), dtype=torch.uint8, device=DEV)
            L.qb_multi_tensor_optimizer_step(h, table, len(sizes), gdt, B, ws)
        else:
            for d, g, n in zip(dev, gd, sizes):
                L.qb_optimizer8bit_step(h, d[0], g, n, d[1], d[3] if two else None, d[2], d[4] if two else None, B)
        for hh, g in zip(host, gs):
            oracle_step(kind, hh, g, B, step, hp, gdt)
        torch.cuda.synchronize()
        for i, (hh, d) in enumerate(zip(host, dev)):
            check(kind, hh, d, exact, f"{name} B={B} multi={multi} step {step} tensor {i}")


SIZES = [1, 4096, 65, 2048 * 3 + 17, 300000, 0, 2048, 123457, 8]


@pytest.mark.parametrize("name", NONNEG)
@pytest.mark.parametrize("B,gdt", [(2048, oracle.BF16), (64, oracle.F32), (4096, oracle.F16), (256, oracle.BF16)])
def test_unsigned_state_free_running_equals_oracle(name, B, gdt):
    run(name, SIZES, B, gdt, 5, multi=True, seed=B + gdt)
    if name not in LAYERWISE:
        run(name, SIZES, B, gdt, 3, multi=False, seed=7 * B + gdt)


@pytest.mark.parametrize("name", NONNEG)
def test_unsigned_state_mixed_with_binary32_states(name):
    run(name, [4096, 100, 2048 * 5 + 3, 4095, 1, 30000], 2048, oracle.BF16, 3, multi=True,
        eight=[True, False, True, False, False, True], seed=50)


@pytest.mark.parametrize("name", ["adamw", "rmsprop"])
def test_paged_unsigned_state_equals_device_resident(name):
    """The paged step with the unsigned code equals the device-resident
    multi-tensor step on the same inputs, bit for bit (pages of 8 blocks)."""
    kind, hp, _ = KINDS[name]
    L = qb()
    two = oracle.OPTIMIZER_STATES[kind] == 2
    sizes, B, page = [1, 4096, 65, 2048 * 3 + 17, 300000, 0, 123457], 2048, 2048 * 8
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    dside, hside = [], []
    z1 = 0 if kind == oracle.RMSPROP else 127
    for n in sizes:
        nb = -(-n // B)
        p = (torch.randn(max(n, 1), device=DEV, generator=g) * 0.02)[:n].contiguous()
        st = [torch.full((max(n, 1),), z1, dtype=torch.uint8, device=DEV)[:n].contiguous(),
              torch.zeros(max(nb, 1), device=DEV)[:nb].contiguous()]
        if two:
            st += [torch.full((max(n, 1),), 0, dtype=torch.uint8, device=DEV)[:n].contiguous(),
                   torch.zeros(max(nb, 1), device=DEV)[:nb].contiguous()]
        dside.append([p.clone()] + [t.clone() for t in st])
        hside.append([p.clone()] + [torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t.cpu()) for t in st])
    ws_dev = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    ws_pg = torch.empty(L.qb_paged_workspace_bytes(page, B), dtype=torch.uint8, device=DEV)
    for step in range(1, 4):
        gr = [(torch.randn(max(n, 1), device=DEV, generator=g) * 1e-3).to(torch.bfloat16)[:n].contiguous()
              for n in sizes]
        h = lib_hp(kind, hp, step)
        h.v_code = L.QB_UDYN8

        def rows(side):
            return [(s[0], gg, s[1], s[3] if two else None, s[2], s[4] if two else None) for s, gg in zip(side, gr)]

        L.qb_multi_tensor_optimizer_step(h, L.tensor_table(rows(dside)), len(sizes), L.QB_BF16, B, ws_dev)
        L.qb_paged_optimizer_step(h, L.paged_tensor_table(rows(hside)), len(sizes), L.QB_BF16, B, page, ws_pg)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(dside, hside)):
            for k, (x, y) in enumerate(zip(a, b)):
                assert torch.equal(x.cpu().view(torch.uint8), y.cpu().view(torch.uint8)), (name, step, i, k)


def test_unsigned_v_keeps_small_v_closer_to_the_binary32_run():
    """Ten AdamW steps from the same start: the decoded v of the unsigned code
    tracks the binary32 optimizer's v more closely than the signed code's
    (mean relative error over elements with v above 1e-3 of the block absmax)."""
    kind, hp, _ = KINDS["adamw"]
    L = qb()
    n, B = 2048 * 64, 2048
    rng = np.random.default_rng(9)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(10)]
    p32, m32, v32 = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for step, g in enumerate(gs, 1):
        oracle.optim32_step(kind, p32, g, m32, v32, step=step, **hp)
    err = {}
    for code in (L.QB_DYN8, L.QB_UDYN8):
        d = [to_device(p0), to_device(np.full(n, 127, np.uint8)), to_device(np.zeros(n // B, np.float32)),
             to_device(np.full(n, 127 if code == L.QB_DYN8 else 0, np.uint8)), to_device(np.zeros(n // B, np.float32))]
        for step, g in enumerate(gs, 1):
            h = lib_hp(kind, hp, step)
            h.v_code = code
            L.qb_optimizer8bit_step(h, d[0], to_device(g), n, d[1], d[3], d[2], d[4], B)
        torch.cuda.synchronize()
        cb = np.array(L.qb_codebook(code), np.float32)
        av = host_bits(d[4])
        v8 = cb[host_bits(d[3])] * np.repeat(av, B)
        big = v32 > 1e-3 * np.repeat(av, B)
        err[code] = np.mean(np.abs(v8[big] - v32[big]) / v32[big])
    assert err[L.QB_UDYN8] < 0.75 * err[L.QB_DYN8], err
