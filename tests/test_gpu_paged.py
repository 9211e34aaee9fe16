"""GPU parity: the paged 8-bit optimizer step (states in pinned host memory,
stepped page by page) against the device-resident multi-tensor step on the
same inputs: parameters, state codes and absmax equal bit for bit after every
step (the device-resident step is itself checked against the oracle)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, qb

pytestmark = pytest.mark.gpu

KINDS = {
    "adamw": (oracle.ADAMW, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    "adam": (oracle.ADAM, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    "lion": (oracle.LION, dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)),
    "sgd": (oracle.SGD, dict(lr=1e-2, beta1=0.9, dampening=0.1, weight_decay=1e-4)),
    "rmsprop": (oracle.RMSPROP, dict(lr=1e-3, beta2=0.99, eps=1e-8, weight_decay=0.01)),
}


def make(sizes, B, two, seed, pdt=torch.float32):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    dev_side, host_side = [], []
    for n in sizes:
        p = (torch.randn(max(n, 1), device=DEV, generator=g) * 0.02).to(pdt)[:n].contiguous()
        nb = -(-n // B)
        st = [torch.full((max(n, 1),), 127, dtype=torch.uint8, device=DEV)[:n].contiguous(),
              torch.zeros(max(nb, 1), device=DEV)[:nb].contiguous()]
        if two:
            st += [torch.full((max(n, 1),), 127, dtype=torch.uint8, device=DEV)[:n].contiguous(),
                   torch.zeros(max(nb, 1), device=DEV)[:nb].contiguous()]
        dev_side.append([p.clone()] + [t.clone() for t in st])
        host_side.append([p.clone()] + [torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t.cpu())
                                        for t in st])
    return dev_side, host_side


def run(name, sizes, B, page, steps=3, pdt=torch.float32, seed=1):
    L = qb()
    kind, hp = KINDS[name]
    two = oracle.OPTIMIZER_STATES[kind] == 2
    gdt = torch.bfloat16 if pdt == torch.float32 else pdt
    dev_side, host_side = make(sizes, B, two, seed, pdt)
    ws_dev = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
    ws_pg = torch.empty(L.qb_paged_workspace_bytes(page, B), dtype=torch.uint8, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed + 100)
    for step in range(1, steps + 1):
        grads = [(torch.randn(max(n, 1), device=DEV, generator=gen) * 1e-3).to(gdt)[:n].contiguous() for n in sizes]
        h = L.optim_hparams(kind, step=step, **hp)

        def rows(side, grads):
            out = []
            for s, gr in zip(side, grads):
                m, am = s[1], s[2]
                v, av = (s[3], s[4]) if two else (None, None)
                out.append((s[0], gr, m, v, am, av))
            return out

        td = L.tensor_table(rows(dev_side, grads))
        L.qb_multi_tensor_optimizer_step(h, td, len(sizes), L._DTYPE[gdt], B, ws_dev, pdt=L._DTYPE[pdt])
        tp = L.paged_tensor_table(rows(host_side, grads))
        L.qb_paged_optimizer_step(h, tp, len(sizes), L._DTYPE[gdt], B, page, ws_pg, pdt=L._DTYPE[pdt])
        torch.cuda.synchronize()
        for i, (d, hs) in enumerate(zip(dev_side, host_side)):
            for k, (a, b) in enumerate(zip(d, hs)):
                assert torch.equal(a.cpu().view(torch.uint8), b.cpu().view(torch.uint8)), (name, step, i, k)


@pytest.mark.parametrize("name", list(KINDS))
def test_paged_equals_device_resident(name):
    # pages of 8 blocks: the 300,000- and 123,457-element tensors span many pages, ragged last pages
    run(name, [1, 4096, 65, 2048 * 3 + 17, 300000, 0, 2048, 123457], 2048, 2048 * 8)


def test_one_block_pages_and_small_blocks():
    run("adamw", [2048 * 20 + 5, 77], 2048, 2048)            # 21 pages of one block each
    run("lion", [64 * 1000 + 3, 5000], 64, 64 * 37)           # B = 64, pages of 37 blocks


def test_bf16_params_and_a_page_larger_than_every_tensor():
    run("adamw", [5000, 70000], 256, 1 << 20, pdt=torch.bfloat16)


def test_large_tensor_many_pages():
    run("adamw", [1 << 24], 2048, 1 << 20, steps=2)            # 16 pages, both slots reused
