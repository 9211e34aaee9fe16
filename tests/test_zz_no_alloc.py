"""GPU: the allocation-free multi-tensor AdamW step (qb_multi_tensor_step_noalloc,
the library's own device scratch in place of a workspace) equals
qb_multi_tensor_step on the same inputs, bit for bit, on two calls in a row,
the second with fewer and smaller tensors (so the scratch holds the first
call's longer table when the second one runs)."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, qb

pytestmark = pytest.mark.gpu


def state(sizes, B, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    out = []
    for n in sizes:
        nb = -(-n // B)
        p = (torch.randn(max(n, 1), device=DEV, generator=g) * 0.02)[:n].contiguous()
        grad = (torch.randn(max(n, 1), device=DEV, generator=g) * 1e-3).to(torch.bfloat16)[:n].contiguous()
        m = torch.randint(0, 256, (max(n, 1),), dtype=torch.uint8, device=DEV, generator=g)[:n].contiguous()
        v = torch.randint(127, 256, (max(n, 1),), dtype=torch.uint8, device=DEV, generator=g)[:n].contiguous()
        am = torch.rand(max(nb, 1), device=DEV, generator=g)[:nb].contiguous() * 1e-3
        av = torch.rand(max(nb, 1), device=DEV, generator=g)[:nb].contiguous() * 1e-6
        out.append([p, grad, m, v, am, av])
    return out


def clone(ts):
    return [[t.clone() for t in row] for row in ts]


def table_of(L, ts, sizes):
    table = L.tensor_table([(r[0], r[1], r[2], r[3], r[4], r[5]) for r in ts])
    for i, n in enumerate(sizes):
        table[i].n = n
    return table


@pytest.mark.parametrize("B", [2048, 256])
def test_noalloc_step_equals_workspace_step_twice(B):
    L = qb()
    calls = [([1, 4096, 65, B * 7 + 17, 300000, 0, 123457, 8, 2 * B], 11),
             ([B * 3 + 1, 5, 0, 4096], 12)]                     # second call: fewer, smaller tensors
    for step, (sizes, seed) in enumerate(calls, start=1):
        print(f"[no-alloc] B={B} call {step} tensors={len(sizes)}", flush=True)
        a = state(sizes, B, seed)
        b = clone(a)
        hp = L.hparams(step=step + 2)
        ta = table_of(L, a, sizes)
        ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(sizes)), dtype=torch.uint8, device=DEV)
        L.qb_multi_tensor_step(ta, len(sizes), L.QB_BF16, B, hp, ws)
        tb = table_of(L, b, sizes)
        L.qb_multi_tensor_step_noalloc(tb, len(sizes), L.QB_BF16, B, hp)
        torch.cuda.synchronize()
        for i, (ra, rb) in enumerate(zip(a, b)):
            for k in (0, 2, 3, 4, 5):
                assert torch.equal(ra[k].view(torch.uint8), rb[k].view(torch.uint8)), \
                    f"B={B} call {step} tensor {i} array {k} differs"
        # the step did run: the parameters moved
        assert any(not torch.equal(ra[0], s[0]) for ra, s in zip(a, state(sizes, B, seed)) if ra[0].numel())


def test_noalloc_rejects_more_tensors_than_its_scratch_holds():
    L = qb()
    p = torch.zeros(16, device=DEV)
    g = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    m = torch.full((16,), 127, dtype=torch.uint8, device=DEV)
    a = torch.zeros(1, device=DEV)
    table = L.tensor_table([(p, g, m, m.clone(), a, a.clone())] * 4097)
    with pytest.raises(L.QbError) as e:
        L.qb_multi_tensor_step_noalloc(table, 4097, L.QB_BF16, 2048, L.hparams())
    assert e.value.status == L.QB_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(p, torch.zeros(16, device=DEV))              # nothing ran
