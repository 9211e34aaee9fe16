#!/usr/bin/env python3
"""Benchmark of the block-wise quantization hot path on one MI355X.

One step = one pass of the whole hot path over synthetic inputs resident in HBM:
  1. one fused 8-bit AdamW step over a 7B decoder's 291 fp32 parameter tensors
     (6,738,415,616 parameters; bf16 gradients ~N(0, 1e-3), the embedding's
     gradient non-zero on a seeded 10% of its rows; int8 moments on the dynamic
     code; block size 2048) in ONE multi-tensor launch;
  2. 4-bit NF4 block-wise quantization (block 64) with nested quantization of
     the absmax (dynamic 8-bit code, block 256) of the 225 fp16 weight
     matrices of the same decoder (6,607,077,376 weights ~N(0, 0.02)), in one
     grouped call (qb_multi_tensor_quantize: four launches);
  3. dequantization of those 225 NF4 tensors to bf16 in one grouped launch
     (qb_multi_tensor_dequantize);
  4. a dynamic 8-bit round trip (quantize, then dequantize to fp32; block 2048)
     of 268,435,456 fp32 values ~0.02 * Student-t(3).
Two gradient sets alternate between steps (generated before timing).  After
the timed steps the two 4-bit sweeps are also timed with one qb_quantize /
qb_dequantize call per tensor (reported under "components", not in `value`).

Prints one JSON line (rank 0).  `value` is the whole step's algorithmic
traffic divided by its time; the per-part figures (AdamW GB/s and params/s,
4-bit dequantize GB/s) are under "components"; "roofline" reports the
dominant kernel (the multi-tensor AdamW step) against the 8 TB/s HBM peak.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused AdamW8bit step GB/s + params/s; 4-bit dequant GB/s (% of HBM peak)"
HBM_PEAK_GBS = 8000.0
ADAM_BLOCK = 2048
W4_BLOCK, W4_BLOCK2 = 64, 256
Q8_N, Q8_BLOCK = 268_435_456, 2048
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_optim8_adamw_multi.llama7b_step.traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def adam_bytes_per_param(grad_bytes=2, block=ADAM_BLOCK):
    # p read+write (8), grad read, m and v codes read+write (4), absmax m and v read+write per block
    return 8 + grad_bytes + 4 + 16.0 / block


def w4_bytes_per_weight():
    # dequantize: packed codes (0.5), nested codes (1/64), second absmax (4/(64*256)), bf16 out (2)
    return 0.5 + 1.0 / W4_BLOCK + 4.0 / (W4_BLOCK * W4_BLOCK2) + 2.0


def q8_bytes_per_elem(block=Q8_BLOCK):
    # quantize: fp32 in (4), code out (1), absmax out; dequantize: code and absmax in, fp32 out (4)
    return 5.0 + 4.0 / block


def q4_bytes_per_weight():
    # quantize: fp16 in (2), packed codes (0.5), nested codes and second absmax out
    return 2.0 + 0.5 + 1.0 / W4_BLOCK + 4.0 / (W4_BLOCK * W4_BLOCK2)


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_optimizer_states_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


def traffic_per_launch():
    """HBM bytes per AdamW launch from the committed counter summary, or None if
    it is missing or the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


class Model7B:
    """Device state of the multi-tensor AdamW step and the 4-bit sweep."""

    def __init__(self, torch, qb, inputs, dev, seed, with_w4=True, grad_sets=2):
        self.t = torch
        shapes = inputs.llama7b_param_shapes()
        self.names = [s[0] for s in shapes]
        self.sizes = [int(np.prod(s[1])) for s in shapes]
        self.params = []
        self.grads = [[] for _ in range(grad_sets)]
        log(f"allocating {len(shapes)} parameter tensors ({sum(self.sizes):,} params)")
        for i, (name, shape) in enumerate(shapes):
            n = self.sizes[i]
            nb = (n + ADAM_BLOCK - 1) // ADAM_BLOCK
            p = inputs.normal(n, 0.02, seed=seed * 1000 + i, device=dev)
            m = torch.full((n,), 127, dtype=torch.uint8, device=dev)
            v = torch.full((n,), 127, dtype=torch.uint8, device=dev)
            am = torch.zeros(nb, dtype=torch.float32, device=dev)
            av = torch.zeros(nb, dtype=torch.float32, device=dev)
            self.params.append((p, m, v, am, av))
            for k in range(grad_sets):
                gs = inputs.grad_seed(seed, i, k)
                if name == "embed":
                    g = inputs.sparse_row_grad(shape[0], shape[1], 0.10, 1e-3, gs, device=dev).reshape(-1)
                else:
                    g = inputs.normal(n, 1e-3, gs, device=dev, dtype=torch.bfloat16)
                self.grads[k].append(g)
        self.tables = [qb.tensor_table([(p, g, m, v, am, av) for (p, m, v, am, av), g in zip(self.params, gset)])
                       for gset in self.grads]
        self.ws = torch.empty(qb.qb_multi_tensor_workspace_bytes(len(shapes)), dtype=torch.uint8, device=dev)
        self.n_params = sum(self.sizes)
        self.w4 = []
        if with_w4:
            wshapes = inputs.llama7b_weight_shapes()
            log(f"allocating {len(wshapes)} fp16 weight tensors for the 4-bit sweep")
            wsmax = 0
            for j, (name, shape) in enumerate(wshapes):
                n = int(np.prod(shape))
                nb = (n + W4_BLOCK - 1) // W4_BLOCK
                w = inputs.normal(n, 0.02, seed=seed * 7919 + j, device=dev, dtype=torch.float16)
                codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev)
                c2 = torch.empty(nb, dtype=torch.uint8, device=dev)
                a2 = torch.empty((nb + W4_BLOCK2 - 1) // W4_BLOCK2, dtype=torch.float32, device=dev)
                off = torch.empty(4, dtype=torch.float32, device=dev)
                y = torch.empty(n, dtype=torch.bfloat16, device=dev)
                self.w4.append((n, w, codes, c2, a2, off, y))
                wsmax = max(wsmax, qb.qb_dq_workspace_bytes(n, W4_BLOCK))
            self.w4_ws = torch.empty(wsmax, dtype=torch.uint8, device=dev)
            self.dq_q = [qb.make_dq(c2, a2, off, W4_BLOCK2, self.w4_ws) for (_, _, _, c2, a2, off, _) in self.w4]
            self.dq_d = [qb.make_dq(c2, a2, off, W4_BLOCK2) for (_, _, _, c2, a2, off, _) in self.w4]
            # grouped calls: the whole sweep in one quantize call (4 launches) and one dequantize launch
            self.q_table = qb.quant_table([(w, n, codes, None, dq)
                                           for (n, w, codes, *_), dq in zip(self.w4, self.dq_d)])
            self.q_ws = torch.empty(qb.qb_multi_tensor_quantize_workspace_bytes(self.q_table, len(self.w4), W4_BLOCK),
                                    dtype=torch.uint8, device=dev)
            self.d_table = qb.dequant_table([(codes, None, dq, n, y)
                                             for (n, _, codes, _, _, _, y), dq in zip(self.w4, self.dq_d)])
            self.d_ws = torch.empty(qb.qb_multi_tensor_workspace_bytes(len(self.w4)), dtype=torch.uint8, device=dev)
        self.n_w4 = sum(e[0] for e in self.w4)
        self.q8 = None
        if with_w4:
            log(f"allocating the {Q8_N:,}-value fp32 tensor for the 8-bit round trip")
            x = inputs.student_t3(Q8_N, 0.02, seed=seed * 31 + 2, device=dev)
            self.q8 = (x, torch.empty(Q8_N, dtype=torch.uint8, device=dev),
                       torch.empty(Q8_N // Q8_BLOCK, dtype=torch.float32, device=dev), torch.empty_like(x))


def run_adam(qb, model, step):
    table = model.tables[(step - 1) % len(model.tables)]
    qb.qb_multi_tensor_step(table, len(table), qb.QB_BF16, ADAM_BLOCK, qb.hparams(step=step, **HP), model.ws)


def run_q4(qb, model):
    qb.qb_multi_tensor_quantize(model.q_table, len(model.w4), qb.QB_F16, qb.QB_NF4, W4_BLOCK, W4_BLOCK2, model.q_ws)


def run_dq4(qb, model):
    qb.qb_multi_tensor_dequantize(model.d_table, len(model.w4), qb.QB_NF4, W4_BLOCK, W4_BLOCK2, qb.QB_BF16,
                                  model.d_ws)


def run_q8(qb, model):
    x, codes, absmax, y = model.q8
    qb.qb_quantize(x, Q8_N, qb.QB_DYN8, Q8_BLOCK, codes, absmax)
    qb.qb_dequantize(codes, absmax, None, qb.QB_DYN8, Q8_BLOCK, Q8_N, y)


def run_q4_per_tensor(qb, model):
    for (n, w, codes, *_), dq in zip(model.w4, model.dq_q):
        qb.qb_quantize(w, n, qb.QB_NF4, W4_BLOCK, codes, None, dq)


def run_dq4_per_tensor(qb, model):
    for (n, _, codes, _, _, _, y), dq in zip(model.w4, model.dq_d):
        qb.qb_dequantize(codes, None, dq, qb.QB_NF4, W4_BLOCK, n, y)


def time_calls(torch, fn, reps=5):
    """Mean HIP-event time (ms) of fn() over reps calls after one warmup call."""
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def time_back_to_back(torch, fn, reps=20):
    """Mean time (ms) of one fn() call over reps calls run back to back between
    two HIP events (after one warmup call): for microsecond kernels, whose
    per-call events would otherwise weigh in."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, model, seconds_target, rng):
    """The oracle, single-threaded, on a bounded sample of the same workload:
    seeded full AdamW blocks of the 7B model (copied from the device), one
    4096x11008 weight quantized (NF4 + nested) and dequantized to bf16, and the
    8-bit round trip of the first 2^23 values of the Student-t tensor."""
    import oracle
    nblocks = 98304
    # sample full blocks in proportion to the tensors' block counts
    full_blocks = np.array([n // ADAM_BLOCK for n in model.sizes], dtype=np.int64)
    prob = full_blocks / full_blocks.sum()
    tensor_of = rng.choice(len(model.sizes), size=nblocks, p=prob)
    ps, gs, ms, vs, ams, avs = [], [], [], [], [], []
    for ti in np.unique(tensor_of):
        k = int(np.sum(tensor_of == ti))
        blk = torch.from_numpy(rng.choice(full_blocks[ti], size=k, replace=False)).to(model.params[ti][0].device)
        p, m, v, am, av = model.params[ti]
        g = model.grads[0][ti]
        B = ADAM_BLOCK
        ps.append(p[: full_blocks[ti] * B].view(-1, B).index_select(0, blk).cpu().numpy().reshape(-1))
        gs.append(g[: full_blocks[ti] * B].view(-1, B).index_select(0, blk).view(torch.int16).cpu().numpy()
                  .view(np.uint16).reshape(-1))
        ms.append(m[: full_blocks[ti] * B].view(-1, B).index_select(0, blk).cpu().numpy().reshape(-1))
        vs.append(v[: full_blocks[ti] * B].view(-1, B).index_select(0, blk).cpu().numpy().reshape(-1))
        ams.append(am.index_select(0, blk).cpu().numpy())
        avs.append(av.index_select(0, blk).cpu().numpy())
    p, g, m, v, am, av = (np.ascontiguousarray(np.concatenate(a)) for a in (ps, gs, ms, vs, ams, avs))
    n_adam = p.size
    t0 = time.perf_counter()
    oracle.adamw8bit_step(p, g, m, v, am, av, ADAM_BLOCK, lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"],
                          eps=HP["eps"], wd=HP["weight_decay"], step=3, gdt=oracle.BF16)
    t_adam = time.perf_counter() - t0
    n4 = 4096 * 11008
    w = next(e[1] for e in model.w4 if e[0] == n4).cpu().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    codes, st = oracle.quantize(w, oracle.NF4, W4_BLOCK, xdt=oracle.F16, double_quant=True)
    t_q4 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dequantize(codes, st, oracle.NF4, W4_BLOCK, n4, oracle.BF16)
    t_d4 = time.perf_counter() - t0
    n8 = 1 << 23
    x8 = model.q8[0][:n8].cpu().numpy()
    t0 = time.perf_counter()
    c8, a8 = oracle.quantize_blockwise(x8, oracle.DYN8, Q8_BLOCK)
    oracle.dequantize_blockwise(c8, a8, oracle.DYN8, Q8_BLOCK, n8, oracle.F32)
    t_q8 = time.perf_counter() - t0
    total_bytes = (n_adam * adam_bytes_per_param() + n4 * (q4_bytes_per_weight() + w4_bytes_per_weight()) +
                   n8 * 2 * q8_bytes_per_elem())
    total_t = t_adam + t_q4 + t_d4 + t_q8
    return {
        "value": total_bytes / total_t / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{nblocks} seeded full 2048-element AdamW blocks of the 7B model ({n_adam:,} params, "
                   f"{t_adam:.2f} s) + NF4 nested quantize ({t_q4:.2f} s) and bf16 dequantize ({t_d4:.2f} s) "
                   f"of one 4096x11008 fp16 weight + dynamic 8-bit round trip of the first {n8:,} fp32 values "
                   f"({t_q8:.2f} s); single-threaded C oracle"),
        "adamw_params_per_s": n_adam / t_adam,
        "dequant4_GBps": n4 * w4_bytes_per_weight() / t_d4 / 1e9,
        "host_cpus": os.cpu_count(),
        "host_cpu_model": host_cpu_model(),
    }


OPTIMIZERS = {  # name: (qb kind, hyperparameters, states)
    "adamw": (0, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), 2),
    "adam": (1, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), 2),
    "lion": (2, dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1), 1),
    "sgd": (3, dict(lr=1e-2, beta1=0.9, weight_decay=1e-4), 1),
    "rmsprop": (4, dict(lr=1e-3, beta2=0.99, eps=1e-8, weight_decay=0.0), 1),
    "lamb": (5, dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, weight_decay=0.01), 2),
    "lars": (6, dict(lr=0.5, beta1=0.9, weight_decay=5e-4, trust_coefficient=1e-3), 1),
}
LAYERWISE = ("lamb", "lars")
NONNEG_STATE = ("adamw", "adam", "rmsprop", "lamb")    # kinds whose v (RMSprop: its state) is never negative


def optim_bytes_per_param(states, grad_bytes=2, block=ADAM_BLOCK):
    # p read+write (8), grad read, each state's code read+write (2) and absmax read+write per block
    return 8 + grad_bytes + states * (2 + 8.0 / block)


def layerwise_extra_bytes_per_param(name, state_bits, grad_bytes=2, block=ADAM_BLOCK):
    # the norm pass before the step: p and g (LARS), plus the states read (LAMB)
    if name == "lars":
        return 4 + grad_bytes
    return 4 + grad_bytes + (2 * (1 + 4.0 / block) if state_bits == 8 else 8)


def bench_flat(torch, qb, inputs, dev, args):
    """Single-tensor fused 8-bit optimizer step (AdamW by default) on a flat
    1,500,000,000-parameter fp32 buffer (bf16 gradients ~N(0, 1e-3), two sets
    alternating; block 2048)."""
    n = 1_500_000_000
    nb = (n + ADAM_BLOCK - 1) // ADAM_BLOCK
    kind, hp, states = OPTIMIZERS[args.optimizer]
    uv = args.v_code == "udyn8"             # the never-negative state in the unsigned code
    if uv and args.optimizer not in NONNEG_STATE:
        raise SystemExit(f"--v-code udyn8 needs a kind with a never-negative state: {', '.join(NONNEG_STATE)}")
    z1 = 0 if uv and args.optimizer == "rmsprop" else 127       # codes of 0.0 of state 1 and state 2
    z2 = 0 if uv else 127
    log(f"allocating a flat buffer of {n:,} params ({args.optimizer}, {states} state(s))")
    pdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[args.param_dtype]
    gdt = torch.bfloat16 if args.param_dtype == "fp32" else pdt      # 16-bit params take grads of their dtype
    p = inputs.normal(n, 0.02, seed=args.seed, device=dev, dtype=pdt)
    if args.paged:                # states in pinned host memory, stepped page by page
        if args.state_bits != 8 or args.optimizer in LAYERWISE:
            raise SystemExit("--paged runs the element-wise kinds with 8-bit states")
        pin = lambda t: torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t)
        s1 = pin(torch.full((n,), z1, dtype=torch.uint8))
        a1 = pin(torch.zeros(nb))
        s2 = pin(torch.full((n,), z2, dtype=torch.uint8)) if states == 2 else None
        a2 = pin(torch.zeros(nb)) if states == 2 else None
    elif args.state_bits == 8:
        s1 = torch.full((n,), z1, dtype=torch.uint8, device=dev)
        a1 = torch.zeros(nb, device=dev)
        s2 = torch.full((n,), z2, dtype=torch.uint8, device=dev) if states == 2 else None
        a2 = torch.zeros(nb, device=dev) if states == 2 else None
    else:                       # the 32-bit fallback: binary32 states, no absmax
        s1 = torch.zeros(n, device=dev)
        s2 = torch.zeros(n, device=dev) if states == 2 else None
        a1 = a2 = None
    grads = [inputs.normal(n, 1e-3, inputs.grad_seed(args.seed, 0, k), device=dev, dtype=gdt) for k in range(2)]

    layerwise = args.optimizer in LAYERWISE
    if args.paged:
        tables = [qb.paged_tensor_table([(p, grads[j], s1, s2, a1, a2)]) for j in range(2)]
        ws = torch.empty(qb.qb_paged_workspace_bytes(args.page_params, ADAM_BLOCK), dtype=torch.uint8, device=dev)
    elif layerwise:             # one tensor = one layer, through the multi-tensor call (norm pass + step)
        tables = [qb.tensor_table([(p, grads[j], s1, s2, a1, a2)]) for j in range(2)]
        ws = torch.empty(qb.qb_optimizer_workspace_bytes(qb.optim_hparams(kind, **hp), tables[0], 1, ADAM_BLOCK),
                         dtype=torch.uint8, device=dev)

    def step(k):
        h = qb.optim_hparams(kind, step=k, v_code=qb.QB_UDYN8 if uv else qb.QB_DYN8, **hp)
        if args.paged:
            qb.qb_paged_optimizer_step(h, tables[k % 2], 1, qb._DTYPE[gdt], ADAM_BLOCK, args.page_params, ws,
                                       pdt=qb._DTYPE[pdt])
        elif layerwise:
            qb.qb_multi_tensor_optimizer_step(h, tables[k % 2], 1, qb._DTYPE[gdt], ADAM_BLOCK, ws,
                                              pdt=qb._DTYPE[pdt])
        else:
            qb.qb_optimizer8bit_step(h, p, grads[k % 2], n, s1, s2, a1, a2, ADAM_BLOCK)

    torch.cuda.synchronize()
    for k in range(1, args.warmup + 1):
        step(k)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        step(args.warmup + 1 + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[len(ms) // 2]
    bpp = optim_bytes_per_param(states) if args.state_bits == 8 else 8 + 2 + 8 * states
    if layerwise:
        bpp += layerwise_extra_bytes_per_param(args.optimizer, args.state_bits)
    if args.param_dtype != "fp32":
        bpp -= 4 if not layerwise else 6            # p read + written in 2 bytes (and read in the norm pass)
    nbytes = n * bpp
    call = "one-layer multi-tensor call (norm pass + step)" if layerwise else "single-tensor"
    extra = {}
    if args.paged:
        call = f"paged (states in pinned host memory, pages of {args.page_params:,} params)"
        state_bytes = n * states * (1 + 4.0 / ADAM_BLOCK)      # each way across PCIe
        extra = {"pcie_bytes_each_way": state_bytes, "pcie_GB/s_each_way": state_bytes / med / 1e6}
    print(json.dumps({"workload": f"flat 1.5e9 params, {args.param_dtype if args.param_dtype != 'fp32' else 'bf16'} "
                                  f"grads, block 2048, {call} {args.optimizer} "
                                  f"step, {args.state_bits}-bit states"
                                  f"{' (v in the unsigned dynamic code)' if uv else ''}, {args.param_dtype} params",
                      "optimizer": args.optimizer, "param_dtype": args.param_dtype, "v_code": args.v_code,
                      "state_bits": args.state_bits, "steps": args.steps, "median_ms": med,
                      "bytes_per_param": bpp, "GB/s": nbytes / med / 1e6,
                      "params_per_s": n / med * 1e3, "frac_of_hbm_peak": nbytes / med / 1e6 / HBM_PEAK_GBS,
                      "wall_ms_per_step": wall / args.steps * 1e3, **extra}), flush=True)


def bench_codes(torch, qb, inputs, dev, args):
    """User codes on the 268,435,456-value Student-t tensor (block 2048): the
    quantile code estimated from the data, then quantize + fp32 dequantize with
    it; the linear code's round trip for comparison."""
    n = Q8_N
    x = inputs.student_t3(n, 0.02, seed=args.seed * 31 + 2, device=dev)
    codes = torch.empty(n, dtype=torch.uint8, device=dev)
    absmax = torch.empty(n // Q8_BLOCK, device=dev)
    y = torch.empty_like(x)
    tq = torch.empty(qb.qb_code_table_bytes(), dtype=torch.uint8, device=dev)
    tl = torch.empty_like(tq)
    qb.qb_prepare_code(qb.qb_linear_code(), tl)
    ws = torch.empty(qb.qb_quantile_workspace_bytes(n), dtype=torch.uint8, device=dev)
    parts = {
        "estimate_quantiles": (lambda: qb.qb_estimate_quantiles(x, n, tq, ws), n * 4.0),
        "quantize_quantile_code": (lambda: qb.qb_quantize_code(x, n, tq, Q8_BLOCK, codes, absmax), n * (5 + 4 / Q8_BLOCK)),
        "dequantize_quantile_code": (lambda: qb.qb_dequantize_code(codes, absmax, tq, Q8_BLOCK, n, y),
                                     n * (5 + 4 / Q8_BLOCK)),
        "quantize_linear_code": (lambda: qb.qb_quantize_code(x, n, tl, Q8_BLOCK, codes, absmax), n * (5 + 4 / Q8_BLOCK)),
    }
    out = {"workload": "268,435,456 fp32 values ~0.02 * Student-t(3), block 2048, user codes", "n": n}
    for name, (fn, nbytes) in parts.items():
        ms = time_calls(torch, fn, reps=args.steps)
        out[name] = {"ms": ms, "GB/s": nbytes / ms / 1e6, "frac_of_hbm_peak": nbytes / ms / 1e6 / HBM_PEAK_GBS,
                     "elements_per_s": n / ms * 1e3}
    print(json.dumps(out), flush=True)


def roundtrip_error_stats(torch, x, y, block):
    """Per-block max and mean |x - y| of a round trip, summarised over the
    blocks (max, mean, p99), absolute and relative to the block's absmax."""
    nb = x.numel() // block
    e = (x[:nb * block] - y[:nb * block]).abs().view(nb, block)
    a = x[:nb * block].abs().view(nb, block).amax(1)
    bmax, bmean = e.amax(1), e.mean(1, dtype=torch.float64)
    ok = a > 0
    rmax = (bmax[ok].double() / a[ok].double())
    rmean = (bmean[ok] / a[ok].double())

    def summary(t):
        t = t.double()
        k = max(1, int(round(0.99 * t.numel())))
        return {"max": t.max().item(), "mean": t.mean().item(), "p99": t.kthvalue(k).values.item()}

    return {"blocks": nb, "block_max_abs_err": summary(bmax), "block_mean_abs_err": summary(bmean),
            "block_max_rel_err": summary(rmax), "block_mean_rel_err": summary(rmean)}


def bench_roundtrip8(torch, qb, inputs, dev, args):
    """Dynamic 8-bit quantize + fp32 dequantize of 268,435,456 values
    ~0.02 * Student-t(3) at block sizes 256, 2048 and 4096: kernel times
    (HIP events), codes/s and GB/s, and the distribution over blocks of the
    per-block max and mean |x - x_hat|."""
    n = Q8_N
    x = inputs.student_t3(n, 0.02, seed=args.seed * 31 + 2, device=dev)
    codes = torch.empty(n, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    out = {"workload": "268,435,456 fp32 values ~0.02 * Student-t(3), dynamic 8-bit code, quantize + fp32 dequantize",
           "n": n, "blocks": []}
    for B in (256, 2048, 4096):
        absmax = torch.empty(n // B, device=dev)
        tq = time_calls(torch, lambda: qb.qb_quantize(x, n, qb.QB_DYN8, B, codes, absmax), reps=args.steps)
        td = time_calls(torch, lambda: qb.qb_dequantize(codes, absmax, None, qb.QB_DYN8, B, n, y), reps=args.steps)
        nbytes = n * q8_bytes_per_elem(B)                      # one pass: 4 + 1 + 4/B bytes per element
        torch.cuda.synchronize()
        out["blocks"].append({"B": B, "quantize_ms": tq, "dequantize_ms": td, "codes_per_s": n / tq * 1e3,
                              "quantize_GB/s": nbytes / tq / 1e6, "dequantize_GB/s": nbytes / td / 1e6,
                              "quantize_frac_of_hbm_peak": nbytes / tq / 1e6 / HBM_PEAK_GBS,
                              "dequantize_frac_of_hbm_peak": nbytes / td / 1e6 / HBM_PEAK_GBS,
                              **roundtrip_error_stats(torch, x, y, B)})
        log(f"B={B}: quantize {tq:.3f} ms, dequantize {td:.3f} ms")
    print(json.dumps(out), flush=True)


MM_SHAPES = [(4096, 4096), (11008, 4096), (4096, 11008)]      # (N, K) of the 7B projections
MM_ROWS = [1, 16, 64, 256, 4096]
MFMA_BF16_PEAK_TFLOPS = 2500.0


def dq4_matmul_bytes(M, N, K, block=W4_BLOCK, block2=W4_BLOCK2):
    """Algorithmic HBM bytes of one fused call: NF4 codes, nested constants
    (one code byte per block, fp32 second-level absmax, the mean), x and y (bf16)."""
    nb = -(-N * K // block)
    return N * K / 2 + nb + 4 * -(-nb // block2) + 4 + 2 * M * K + 2 * M * N


def bench_matmul(torch, qb, inputs, dev, args):
    """The 4-bit layer product in bf16: qb_dequant_matmul (NF4, nested, B = 64)
    against the unfused route (qb_dequantize to bf16, then torch's matmul) on the
    7B decoder's projection shapes, for M = 1 .. 4096 rows of activations.
    Codes are uniform random bytes and the nested constants fixed values (the
    kernels have no data-dependent work)."""
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    out = {"workload": "y = x W^T, W NF4 (B = 64, nested B2 = 256), bf16 compute, 7B projection shapes",
           "shapes": []}
    for N, K in MM_SHAPES:
        nb = N * K // W4_BLOCK
        codes = torch.randint(0, 256, (N * K // 2,), dtype=torch.uint8, device=dev, generator=g)
        c2 = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=dev, generator=g)
        a2 = torch.full((-(-nb // W4_BLOCK2),), 0.02, device=dev)
        mu = torch.full((4,), 0.03, device=dev)
        dq = qb.make_dq(c2, a2, mu, W4_BLOCK2)
        w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        for M in MM_ROWS:
            x = inputs.normal(M * K, 1.0, seed=args.seed + M, device=dev, dtype=torch.bfloat16).view(M, K)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fused = time_back_to_back(torch, lambda: qb.qb_dequant_matmul(x, codes, None, 1, W4_BLOCK, N, y, dq=dq),
                                      reps=args.steps)

            def unfused():
                qb.qb_dequantize(codes, None, dq, 1, W4_BLOCK, N * K, w)
                torch.matmul(x, w.t(), out=y)

            ref = time_back_to_back(torch, unfused, reps=args.steps)
            nbytes = dq4_matmul_bytes(M, N, K)
            flops = 2.0 * M * N * K
            out["shapes"].append({"N": N, "K": K, "M": M, "fused_us": fused * 1e3, "unfused_us": ref * 1e3,
                                  "speedup": ref / fused, "GB/s": nbytes / fused / 1e6,
                                  "frac_of_hbm_peak": nbytes / fused / 1e6 / HBM_PEAK_GBS,
                                  "TFLOP/s": flops / fused / 1e9,
                                  "frac_of_bf16_mfma_peak": flops / fused / 1e9 / MFMA_BF16_PEAK_TFLOPS})
            log(f"N={N} K={K} M={M}: fused {fused * 1e3:.1f} us, unfused {ref * 1e3:.1f} us")
    print(json.dumps(out), flush=True)


def copy_calibration(torch, dev):
    """Five device-to-device copies of exactly 1 GiB: 1,073,741,824 bytes read and
    written per dispatch.  Profiling this under FETCH_SIZE / WRITE_SIZE gives the
    factor that turns those counters into HBM bytes for the kernels above."""
    a = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": 1 << 30, "dispatches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=2024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--adam-only", action="store_true", help="time only the multi-tensor AdamW step")
    ap.add_argument("--flat", action="store_true",
                    help="time the single-tensor AdamW step on a flat 1.5e9-parameter buffer instead")
    ap.add_argument("--paged", action="store_true",
                    help="--flat with the optimizer states in pinned host memory (qb_paged_optimizer_step)")
    ap.add_argument("--page-params", type=int, default=1 << 26, help="parameters per page of the --paged run")
    ap.add_argument("--param-dtype", choices=["fp32", "bf16", "fp16"], default="fp32",
                    help="parameter dtype of the --flat run (16-bit parameters take gradients of their dtype)")
    ap.add_argument("--optimizer", choices=sorted(OPTIMIZERS), default="adamw",
                    help="optimizer of the --flat run (the 8-bit states of each kind)")
    ap.add_argument("--v-code", choices=["dyn8", "udyn8"], default="dyn8",
                    help="code of the never-negative state of the --flat run (udyn8: the unsigned dynamic code)")
    ap.add_argument("--state-bits", type=int, choices=(8, 32), default=8,
                    help="state width of the --flat run (32: the binary32 fallback of small or chosen tensors)")
    ap.add_argument("--codes", action="store_true",
                    help="time the user-code calls (quantile estimation, quantile and linear codes) instead")
    ap.add_argument("--roundtrip8", action="store_true",
                    help="time the dynamic 8-bit round trip at B = 256, 2048, 4096 and report per-block errors")
    ap.add_argument("--matmul", action="store_true",
                    help="time the fused 4-bit dequantize + product on the 7B projection shapes instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device five times (the reference kernel for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    from bit_optimizer_states_amd import binding as qb
    from bit_optimizer_states_amd import inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = "cuda:0"
    if args.copy_calibration:
        return copy_calibration(torch, dev)
    qb.lib()
    rng = np.random.default_rng(args.seed)
    if args.flat:
        return bench_flat(torch, qb, inputs, dev, args)
    if args.codes:
        return bench_codes(torch, qb, inputs, dev, args)
    if args.matmul:
        return bench_matmul(torch, qb, inputs, dev, args)
    if args.roundtrip8:
        return bench_roundtrip8(torch, qb, inputs, dev, args)
    model = Model7B(torch, qb, inputs, dev, args.seed, with_w4=not args.adam_only)
    torch.cuda.synchronize()
    log(f"setup done; warmup {args.warmup} steps")

    def step(k, ev=None):
        if ev is not None:
            ev[0].record()
        run_adam(qb, model, k)
        if ev is not None:
            ev[1].record()
        if not args.adam_only:
            run_q4(qb, model)
            if ev is not None:
                ev[2].record()
            run_dq4(qb, model)
            if ev is not None:
                ev[3].record()
            run_q8(qb, model)
            if ev is not None:
                ev[4].record()

    for k in range(1, args.warmup + 1):
        step(k)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + 1 + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")

    adam_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    adam_bytes = model.n_params * adam_bytes_per_param()
    comps = {"adamw8bit_multi_tensor": {
        "ms": adam_ms, "GB/s": adam_bytes / adam_ms / 1e6, "params_per_s": model.n_params / adam_ms * 1e3,
        "frac_of_hbm_peak": adam_bytes / adam_ms / 1e6 / HBM_PEAK_GBS, "launches_per_step": 1}}
    step_bytes = adam_bytes
    if not args.adam_only:
        q4_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        d4_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        q4_bytes = model.n_w4 * q4_bytes_per_weight()
        d4_bytes = model.n_w4 * w4_bytes_per_weight()
        comps["quantize4_nf4_nested"] = {"ms": q4_ms, "GB/s": q4_bytes / q4_ms / 1e6,
                                         "frac_of_hbm_peak": q4_bytes / q4_ms / 1e6 / HBM_PEAK_GBS,
                                         "launches_per_step": 4, "call": "qb_multi_tensor_quantize"}
        comps["dequant4_nf4_nested_bf16"] = {"ms": d4_ms, "GB/s": d4_bytes / d4_ms / 1e6,
                                             "frac_of_hbm_peak": d4_bytes / d4_ms / 1e6 / HBM_PEAK_GBS,
                                             "launches_per_step": 1, "call": "qb_multi_tensor_dequantize"}
        q8_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
        q8_bytes = Q8_N * 2 * q8_bytes_per_elem()
        comps["roundtrip8_dyn8_fp32"] = {"ms": q8_ms, "GB/s": q8_bytes / q8_ms / 1e6,
                                         "frac_of_hbm_peak": q8_bytes / q8_ms / 1e6 / HBM_PEAK_GBS,
                                         "elements_per_s": Q8_N / q8_ms * 1e3, "launches_per_step": 2,
                                         "call": "qb_quantize + qb_dequantize",
                                         "error": roundtrip_error_stats(torch, model.q8[0], model.q8[3], Q8_BLOCK)}
        step_bytes += q4_bytes + d4_bytes + q8_bytes
    ms_per_step = wall / args.steps * 1e3
    if not args.adam_only:
        # the same sweeps with one qb_quantize / qb_dequantize call per tensor (outside the timed step)
        q1 = time_calls(torch, lambda: run_q4_per_tensor(qb, model))
        d1 = time_calls(torch, lambda: run_dq4_per_tensor(qb, model))
        comps["quantize4_nf4_nested_per_tensor_calls"] = {
            "ms": q1, "GB/s": q4_bytes / q1 / 1e6, "frac_of_hbm_peak": q4_bytes / q1 / 1e6 / HBM_PEAK_GBS,
            "launches": 4 * len(model.w4), "call": "qb_quantize"}
        comps["dequant4_nf4_nested_bf16_per_tensor_calls"] = {
            "ms": d1, "GB/s": d4_bytes / d1 / 1e6, "frac_of_hbm_peak": d4_bytes / d1 / 1e6 / HBM_PEAK_GBS,
            "launches": len(model.w4), "call": "qb_dequantize"}
    traffic = traffic_per_launch()
    achieved = adam_bytes / adam_ms / 1e6
    out = {
        "metric": METRIC,
        "value": step_bytes / ms_per_step / 1e6,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("7B decoder (291 tensors, 6,738,415,616 fp32 params, bf16 grads, 10% sparse embedding "
                         "rows): one multi-tensor fused AdamW8bit step, block 2048" +
                         ("" if args.adam_only else
                          "; + NF4 nested quantize and bf16 dequantize of its 225 fp16 weights "
                          "(6,607,077,376), block 64 / 256; + dynamic 8-bit quantize and fp32 dequantize of "
                          "268,435,456 Student-t(3) values, block 2048")),
            "params": model.n_params,
            "weights_4bit": model.n_w4,
            "adam_blocksize": ADAM_BLOCK,
            "w4_blocksize": W4_BLOCK,
            "w4_blocksize2": W4_BLOCK2,
            "parallelism": "single GPU",
        },
        "components": comps,
        "roofline": {
            "kernel": "k_optim8<AdamW, 2048, bf16, multi-tensor>",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": adam_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(torch, model, 10.0, rng)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
