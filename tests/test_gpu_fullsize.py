"""GPU parity at the workloads' full sizes, through the same C-ABI calls the
benchmark times.  The HIP path processes the whole tensor; the oracle
recomputes sampled blocks (blocks are independent, so a sampled block's
result is exact, not statistical) and, for nested quantization, the whole
state of the tensors it covers.

Workloads (seeded, synthetic; shapes of the pages' models):
  * 268,435,456 fp32 values, 0.02 * Student-t(3), dynamic 8-bit code at block
    sizes 256, 2048 and 4096 (quantize + dequantize round trip);
  * one flat buffer of 1,500,000,000 fp32 parameters, bf16 gradients, fused
    AdamW8bit at block 2048 (ragged last block of 1,792 elements), with v in
    the signed and in the unsigned dynamic code;
  * NF4 / FP4 block-64 quantization with nested quantization (block 256) and a
    bf16 dequantize of 7B-decoder-shaped fp16 weights, per tensor and with the
    grouped calls over all 225 tensors;
  * one multi-tensor AdamW8bit launch over the 291 tensors of a 7B decoder
    (6,738,415,616 parameters), with 10%-row-sparse embedding gradients;
  * beyond 32-bit offsets: an AdamW8bit step on 2^31 + 4097 parameters and an
    NF4 nested round trip on 2^32 + 131 weights.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_optimizer_states_amd import inputs
from gpu_helpers import DEV, host_bits, qb

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def hparams(step):
    return qb().hparams(lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"], weight_decay=HP["wd"],
                        step=step)


def block_rows(t, B, blocks):
    """Host copies of the listed blocks of flat device tensor t (last block may be partial)."""
    n = t.numel()
    out = []
    for b in blocks:
        lo, hi = int(b) * B, min(n, (int(b) + 1) * B)
        out.append(host_bits(t[lo:hi]))
    return out


@pytest.mark.parametrize("B", [256, 2048, 4096])
def test_quantize8_roundtrip_268M(B):
    n = 268_435_456
    L = qb()
    x = inputs.student_t3(n, 0.02, seed=20 + B, device=DEV)
    nb = n // B
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(nb, dtype=torch.float32, device=DEV)
    L.qb_quantize(x, n, qb().QB_DYN8, B, codes, absmax)
    y = torch.empty(n, dtype=torch.float32, device=DEV)
    L.qb_dequantize(codes, absmax, None, qb().QB_DYN8, B, n, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(B)
    blocks = np.unique(np.concatenate([rng.choice(nb, 2048, replace=False), [0, nb - 1]]))
    xs = np.concatenate(block_rows(x, B, blocks))
    want_c, want_a = oracle.quantize_blockwise(xs, oracle.DYN8, B)
    got_c = np.concatenate(block_rows(codes, B, blocks))
    got_a = absmax.cpu().numpy()[blocks]
    assert np.array_equal(got_c, want_c)
    assert np.array_equal(got_a.view(np.uint32), want_a.view(np.uint32))
    want_y = oracle.dequantize_blockwise(want_c, want_a, oracle.DYN8, B, xs.size)
    got_y = np.concatenate(block_rows(y, B, blocks))
    assert np.array_equal(got_y.view(np.uint32), want_y.view(np.uint32))
    # round-trip error per block over the whole tensor (reported, bounded)
    err = (y - x).abs().view(nb, B)
    blk_max = (err.max(dim=1).values / torch.where(absmax > 0, absmax, torch.ones_like(absmax))).max().item()
    print(f"\nB={B}: max |x - x^| / absmax over all blocks {blk_max:.6f}, "
          f"mean |x - x^| {err.mean().item():.3e}, max per-block mean {err.mean(dim=1).max().item():.3e}")
    assert blk_max <= 0.00703126 + 2 ** -22


def test_adamw8bit_flat_1p5B():
    n, B = 1_500_000_000, 2048
    L = qb()
    nb = (n + B - 1) // B
    assert n - (nb - 1) * B == 1792
    p = inputs.normal(n, 0.02, seed=31, device=DEV)
    m = torch.full((n,), 127, dtype=torch.uint8, device=DEV)
    v = torch.full((n,), 127, dtype=torch.uint8, device=DEV)
    am = torch.zeros(nb, device=DEV)
    av = torch.zeros(nb, device=DEV)
    rng = np.random.default_rng(3)
    blocks = np.unique(np.concatenate([rng.choice(nb - 1, 4096, replace=False), [0, nb - 1]]))
    # oracle state of the sampled blocks, free-running from the same initial state
    st = [[host_bits(p[b * B:min(n, (b + 1) * B)]), np.full(min(n, (b + 1) * B) - b * B, 127, np.uint8),
           np.full(min(n, (b + 1) * B) - b * B, 127, np.uint8), np.zeros(1, np.float32), np.zeros(1, np.float32)]
          for b in blocks]
    for step in range(1, 4):
        g = inputs.normal(n, 1e-3, seed=inputs.grad_seed(31, 0, step), device=DEV, dtype=torch.bfloat16)
        L.qb_adamw8bit_step(p, g, n, m, v, am, av, B, hparams(step))
        gs = block_rows(g, B, blocks)
        for s, gb in zip(st, gs):
            oracle.adamw8bit_step(s[0], gb, s[1], s[2], s[3], s[4], B, step=step, gdt=oracle.BF16, **HP)
        torch.cuda.synchronize()
        pm, mm, vm = block_rows(p, B, blocks), block_rows(m, B, blocks), block_rows(v, B, blocks)
        amh, avh = am.cpu().numpy()[blocks], av.cpu().numpy()[blocks]
        for k, s in enumerate(st):
            assert np.array_equal(mm[k], s[1]) and np.array_equal(vm[k], s[2]), (step, blocks[k])
            assert amh[k] == s[3][0] and avh[k] == s[4][0], (step, blocks[k])
            np.testing.assert_allclose(pm[k], s[0], rtol=1e-6, atol=2e-8)
        del g


def test_adamw8bit_flat_1p5B_unsigned_v():
    """The flat step of bench.py --flat --v-code udyn8: qb_optimizer8bit_step
    with v in the unsigned dynamic code (fresh v codes 0), sampled blocks
    against the oracle over three steps."""
    n, B = 1_500_000_000, 2048
    L = qb()
    nb = (n + B - 1) // B
    p = inputs.normal(n, 0.02, seed=37, device=DEV)
    m = torch.full((n,), 127, dtype=torch.uint8, device=DEV)
    v = torch.full((n,), 0, dtype=torch.uint8, device=DEV)
    am = torch.zeros(nb, device=DEV)
    av = torch.zeros(nb, device=DEV)
    rng = np.random.default_rng(4)
    blocks = np.unique(np.concatenate([rng.choice(nb - 1, 4096, replace=False), [0, nb - 1]]))
    st = [[host_bits(p[b * B:min(n, (b + 1) * B)]), np.full(min(n, (b + 1) * B) - b * B, 127, np.uint8),
           np.zeros(min(n, (b + 1) * B) - b * B, np.uint8), np.zeros(1, np.float32), np.zeros(1, np.float32)]
          for b in blocks]
    for step in range(1, 4):
        g = inputs.normal(n, 1e-3, seed=inputs.grad_seed(37, 0, step), device=DEV, dtype=torch.bfloat16)
        h = L.optim_hparams(L.QB_ADAMW, HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"],
                            weight_decay=HP["wd"], step=step, v_code=L.QB_UDYN8)
        L.qb_optimizer8bit_step(h, p, g, n, m, v, am, av, B)
        gs = block_rows(g, B, blocks)
        for s, gb in zip(st, gs):
            oracle.optim8bit_step(oracle.ADAMW, s[0], gb, s[1], s[3], s[2], s[4], B, step=step, gdt=oracle.BF16,
                                  vcode=oracle.UDYN8, **HP)
        torch.cuda.synchronize()
        pm, mm, vm = block_rows(p, B, blocks), block_rows(m, B, blocks), block_rows(v, B, blocks)
        amh, avh = am.cpu().numpy()[blocks], av.cpu().numpy()[blocks]
        for k, s in enumerate(st):
            assert np.array_equal(mm[k], s[1]) and np.array_equal(vm[k], s[2]), (step, blocks[k])
            assert amh[k] == s[3][0] and avh[k] == s[4][0], (step, blocks[k])
            np.testing.assert_allclose(pm[k], s[0], rtol=1e-6, atol=2e-8)
            s[0][:] = pm[k]          # each step from the device's parameters (AdamW's p is within 1e-6)
        del g


@pytest.mark.parametrize("code", [oracle.NF4, oracle.FP4])
def test_quantize4_nested_7b_shapes(code):
    L = qb()
    shapes = inputs.llama7b_weight_shapes()
    full_oracle = {"layers.0.attn.q", "layers.0.mlp.gate"}
    nested_checked = {name for name, _ in shapes if name == "embed" or name.startswith(("layers.0.", "layers.8.",
                                                                                           "layers.16.", "layers.24.", "layers.31."))}
    rng = np.random.default_rng(40 + code)
    for j, (name, shape) in enumerate(shapes):
        if name not in nested_checked:
            continue
        n = int(np.prod(shape))
        nb = (n + 63) // 64
        w = inputs.normal(n, 0.02, seed=7919 * 2024 + j, device=DEV, dtype=torch.float16)
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=DEV)
        c2 = torch.empty(nb, dtype=torch.uint8, device=DEV)
        a2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=DEV)
        off = torch.empty(4, dtype=torch.float32, device=DEV)
        ws = torch.empty(L.qb_dq_workspace_bytes(n, 64), dtype=torch.uint8, device=DEV)
        L.qb_quantize(w, n, code, 64, codes, None, L.make_dq(c2, a2, off, 256, ws))
        y = torch.empty(n, dtype=torch.bfloat16, device=DEV)
        L.qb_dequantize(codes, None, L.make_dq(c2, a2, off, 256), code, 64, n, y)
        torch.cuda.synchronize()
        wh = host_bits(w)
        if name in full_oracle:
            want_c, st = oracle.quantize(wh, code, 64, xdt=oracle.F16, double_quant=True)
            assert np.array_equal(codes.cpu().numpy(), want_c), name
            want_y = oracle.dequantize(want_c, st, code, 64, n, oracle.BF16)
            assert np.array_equal(host_bits(y), want_y), name
            a = st["absmax_fp32"]
        else:
            # absmax of every block (max of |x|, exact) for the nested state; sampled blocks for codes
            a = np.abs(wh.view(np.float16).astype(np.float32)).reshape(-1, 64).max(axis=1)
            blocks = rng.choice(nb, 512, replace=False)
            xs = np.concatenate([wh[b * 64:(b + 1) * 64] for b in blocks])
            want_c, _ = oracle.quantize_blockwise(xs, code, 64, oracle.F16)
            got_c = np.concatenate([codes[b * 32:(b + 1) * 32].cpu().numpy() for b in blocks])
            assert np.array_equal(got_c, want_c), name
        c2w, a2w, mu = oracle.dq_quantize(a, 256)
        assert np.float32(off[0].item()) == mu, name
        assert np.array_equal(c2.cpu().numpy(), c2w) and np.array_equal(a2.cpu().numpy(), a2w), name
        if name not in full_oracle:
            blocks = rng.choice(nb, 256, replace=False)
            ahat = oracle.dq_decode(c2w, a2w, mu)
            for b in blocks:
                want = oracle.dequantize_blockwise(codes[b * 32:(b + 1) * 32].cpu().numpy(), ahat[b:b + 1], code, 64,
                                                   64, oracle.BF16)
                assert np.array_equal(host_bits(y[b * 64:(b + 1) * 64]), want), (name, b)
        del w, codes, c2, a2, off, ws, y


def test_multi_tensor_7b_one_launch():
    L = qb()
    B = 2048
    shapes = inputs.llama7b_param_shapes()
    sizes = [int(np.prod(s)) for _, s in shapes]
    assert len(shapes) == 291 and sum(sizes) == 6_738_415_616
    params = []
    for i, n in enumerate(sizes):
        nb = (n + B - 1) // B
        params.append([inputs.normal(n, 0.02, seed=1000 + i, device=DEV),
                       torch.full((n,), 127, dtype=torch.uint8, device=DEV),
                       torch.full((n,), 127, dtype=torch.uint8, device=DEV),
                       torch.zeros(nb, device=DEV), torch.zeros(nb, device=DEV)])
    rng = np.random.default_rng(50)
    nbs = [(n + B - 1) // B for n in sizes]
    samples = set()
    for i, nb in enumerate(nbs):
        samples.add((i, nb - 1))                             # the (possibly partial) last block of every tensor
        samples.add((i, int(rng.integers(nb))))
    cum = np.cumsum([0] + nbs)
    for gb in rng.choice(cum[-1], 2048, replace=False):      # random blocks over the whole model
        i = int(np.searchsorted(cum, gb, side="right") - 1)
        samples.add((i, int(gb - cum[i])))
    embed = [k for k, (nm, _) in enumerate(shapes) if nm == "embed"][0]
    for b in rng.choice(nbs[embed], 256, replace=False):     # embedding blocks: most lie in zero-gradient rows
        samples.add((embed, int(b)))
    samples = sorted(samples)
    ws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(shapes)), dtype=torch.uint8, device=DEV)

    def slc(t, b, n):
        return t[b * B:min(n, (b + 1) * B)]

    state = {}
    for (i, b) in samples:
        n = sizes[i]
        k = min(n, (b + 1) * B) - b * B
        state[(i, b)] = [host_bits(slc(params[i][0], b, n)), np.full(k, 127, np.uint8), np.full(k, 127, np.uint8),
                         np.zeros(1, np.float32), np.zeros(1, np.float32)]
    zero_row_blocks = 0
    for step in range(1, 3):
        grads = []
        for i, (name, shape) in enumerate(shapes):
            gs = inputs.grad_seed(2024, i, step)
            if name == "embed":
                grads.append(inputs.sparse_row_grad(shape[0], shape[1], 0.10, 1e-3, gs, device=DEV).reshape(-1))
            else:
                grads.append(inputs.normal(sizes[i], 1e-3, gs, device=DEV, dtype=torch.bfloat16))
        table = L.tensor_table([(p, g, m, v, am, av) for (p, m, v, am, av), g in zip(params, grads)])
        L.qb_multi_tensor_step(table, len(shapes), L.QB_BF16, B, hparams(step), ws)
        for (i, b), s in state.items():
            gb = host_bits(slc(grads[i], b, sizes[i]))
            if i == embed and not np.any(gb):
                zero_row_blocks += 1
            oracle.adamw8bit_step(s[0], gb, s[1], s[2], s[3], s[4], B, step=step, gdt=oracle.BF16, **HP)
        torch.cuda.synchronize()
        for (i, b), s in state.items():
            p, m, v, am, av = params[i]
            n = sizes[i]
            assert np.array_equal(host_bits(slc(m, b, n)), s[1]), (step, shapes[i][0], b)
            assert np.array_equal(host_bits(slc(v, b, n)), s[2]), (step, shapes[i][0], b)
            assert am[b].item() == s[3][0] and av[b].item() == s[4][0], (step, shapes[i][0], b)
            np.testing.assert_allclose(host_bits(slc(p, b, n)), s[0], rtol=1e-6, atol=2e-8)
        del grads, table
    assert zero_row_blocks > 0, "the sample must include zero-gradient embedding blocks"


def test_grouped_4bit_7b_all_225_tensors():
    """The grouped NF4 calls the benchmark times, over all 225 7B weight
    tensors at once: every tensor's nested state (mean, codes, second-level
    absmax) exactly as the oracle computes it from that tensor's block absmax;
    sampled blocks of every tensor for the 4-bit codes and the bf16 output."""
    L = qb()
    code, B, B2 = oracle.NF4, 64, 256
    shapes = inputs.llama7b_weight_shapes()
    rng = np.random.default_rng(77)
    W = []
    for j, (name, shape) in enumerate(shapes):
        n = int(np.prod(shape))
        nb = (n + B - 1) // B
        w = inputs.normal(n, 0.02, seed=3331 + j, device=DEV, dtype=torch.float16)
        W.append((name, n, w, torch.empty((n + 1) // 2, dtype=torch.uint8, device=DEV),
                  torch.empty(nb, dtype=torch.uint8, device=DEV),
                  torch.empty((nb + B2 - 1) // B2, dtype=torch.float32, device=DEV),
                  torch.empty(4, dtype=torch.float32, device=DEV), torch.empty(n, dtype=torch.bfloat16, device=DEV)))
    dqs = [L.make_dq(c2, a2, off, B2) for (_, _, _, _, c2, a2, off, _) in W]
    qt = L.quant_table([(w, n, codes, None, dq) for (_, n, w, codes, *_), dq in zip(W, dqs)])
    qws = torch.empty(L.qb_multi_tensor_quantize_workspace_bytes(qt, len(W), B), dtype=torch.uint8, device=DEV)
    L.qb_multi_tensor_quantize(qt, len(W), L.QB_F16, code, B, B2, qws)
    dt = L.dequant_table([(codes, None, dq, n, y) for (_, n, _, codes, _, _, _, y), dq in zip(W, dqs)])
    dws = torch.empty(L.qb_multi_tensor_workspace_bytes(len(W)), dtype=torch.uint8, device=DEV)
    L.qb_multi_tensor_dequantize(dt, len(W), code, B, B2, L.QB_BF16, dws)
    torch.cuda.synchronize()
    del qws
    for (name, n, w, codes, c2, a2, off, y) in W:
        nb = n // B
        # block absmax (a maximum: exact whatever computes it) for the tensor's nested state
        a = w.abs().view(nb, B).amax(dim=1).float().cpu().numpy()
        c2w, a2w, mu = oracle.dq_quantize(a, B2)
        assert np.float32(off[0].item()) == mu, name
        assert np.array_equal(c2.cpu().numpy(), c2w) and np.array_equal(a2.cpu().numpy(), a2w), name
        blocks = np.unique(np.concatenate([rng.choice(nb, 48, replace=False), [0, nb - 1]]))
        idx = torch.from_numpy(blocks).to(DEV)
        xs = host_bits(w.view(nb, B).index_select(0, idx)).reshape(-1)
        want_c, _ = oracle.quantize_blockwise(xs, code, B, oracle.F16)
        got_c = codes.view(nb, B // 2).index_select(0, idx).cpu().numpy().reshape(-1)
        assert np.array_equal(got_c, want_c), name
        ahat = oracle.dq_decode(c2w, a2w, mu)[blocks]
        want_y = oracle.dequantize_blockwise(want_c, ahat, code, B, len(blocks) * B, oracle.BF16)
        got_y = host_bits(y.view(nb, B).index_select(0, idx)).reshape(-1)
        assert np.array_equal(got_y, want_y), name


def _sample_blocks(nb, around, rng, k=64):
    """Block indices: random ones, the first and last, and those around the given element offsets."""
    pick = set(rng.choice(nb, k, replace=False).tolist()) | {0, nb - 1}
    for e in around:
        b = e // 64
        pick |= {max(0, min(nb - 1, b + d)) for d in (-2, -1, 0, 1, 2)}
    return np.array(sorted(pick))


def test_adamw8bit_beyond_int32_elements():
    """One tensor of 2^31 + 4097 parameters: every element offset above 2^31
    (the ragged last block included) reaches the right place."""
    L = qb()
    n, B = (1 << 31) + 4097, 2048
    nb = (n + B - 1) // B
    p = inputs.normal(n, 0.02, seed=71, device=DEV)
    g = inputs.normal(n, 1e-3, seed=72, device=DEV, dtype=torch.bfloat16)
    m = torch.full((n,), 127, dtype=torch.uint8, device=DEV)
    v = torch.full((n,), 127, dtype=torch.uint8, device=DEV)
    am = torch.zeros(nb, device=DEV)
    av = torch.zeros(nb, device=DEV)
    rng = np.random.default_rng(73)
    blocks = np.unique(np.concatenate([rng.choice(nb, 96, replace=False), [0, nb - 2, nb - 1],
                                       np.arange((1 << 31) // B - 2, (1 << 31) // B + 3)]))
    p0 = block_rows(p, B, blocks)
    g0 = block_rows(g, B, blocks)
    L.qb_adamw8bit_step(p, g, n, m, v, am, av, B, hparams(1))
    torch.cuda.synchronize()
    pm, mm, vm = block_rows(p, B, blocks), block_rows(m, B, blocks), block_rows(v, B, blocks)
    amh, avh = am.cpu().numpy()[blocks], av.cpu().numpy()[blocks]
    for k, b in enumerate(blocks):
        ph = p0[k].copy()
        cm, cv = np.full(ph.size, 127, np.uint8), np.full(ph.size, 127, np.uint8)
        a1, a2 = np.zeros(1, np.float32), np.zeros(1, np.float32)
        oracle.adamw8bit_step(ph, g0[k], cm, cv, a1, a2, B, step=1, gdt=oracle.BF16, **HP)
        assert np.array_equal(mm[k], cm) and np.array_equal(vm[k], cv), b
        assert amh[k] == a1[0] and avh[k] == a2[0], b
        np.testing.assert_allclose(pm[k], ph, rtol=1e-6, atol=2e-8)


def test_nf4_nested_beyond_uint32_elements():
    """NF4 block-64 quantization with nesting and a bf16 dequantize of one
    tensor of 2^32 + 131 fp16 weights (odd length: the last byte's low nibble is
    0): sampled blocks around 2^31 and 2^32 against the oracle, and the whole
    nested state."""
    L = qb()
    n, B, B2 = (1 << 32) + 131, 64, 256
    nb = (n + B - 1) // B
    w = inputs.normal(n, 0.02, seed=74, device=DEV, dtype=torch.float16)
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=DEV)
    c2 = torch.empty(nb, dtype=torch.uint8, device=DEV)
    a2 = torch.empty((nb + B2 - 1) // B2, dtype=torch.float32, device=DEV)
    off = torch.empty(4, dtype=torch.float32, device=DEV)
    ws = torch.empty(L.qb_dq_workspace_bytes(n, B), dtype=torch.uint8, device=DEV)
    L.qb_quantize(w, n, qb().QB_NF4, B, codes, None, L.make_dq(c2, a2, off, B2, ws))
    del ws
    y = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    L.qb_dequantize(codes, None, L.make_dq(c2, a2, off, B2), qb().QB_NF4, B, n, y)
    torch.cuda.synchronize()
    full = n // B
    a = w[:full * B].abs().view(full, B).amax(dim=1).float().cpu().numpy()
    a = np.concatenate([a, [float(w[full * B:].abs().max())]]).astype(np.float32)
    c2w, a2w, mu = oracle.dq_quantize(a, B2)
    assert np.float32(off[0].item()) == mu
    assert np.array_equal(c2.cpu().numpy(), c2w) and np.array_equal(a2.cpu().numpy(), a2w)
    ahat = oracle.dq_decode(c2w, a2w, mu)
    rng = np.random.default_rng(75)
    for b in _sample_blocks(nb, [1 << 31, 1 << 32, n - 1], rng):
        lo, hi = int(b) * B, min(n, (int(b) + 1) * B)
        xs = host_bits(w[lo:hi])
        want_c, _ = oracle.quantize_blockwise(xs, oracle.NF4, B, oracle.F16)
        got_c = codes[lo // 2:(hi + 1) // 2].cpu().numpy()
        assert np.array_equal(got_c, want_c), b
        want_y = oracle.dequantize_blockwise(want_c, ahat[b:b + 1], oracle.NF4, B, hi - lo, oracle.BF16)
        assert np.array_equal(host_bits(y[lo:hi]), want_y), b
