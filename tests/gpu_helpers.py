"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
bring results back to the host; the oracle runs on host copies of the same
input bytes."""
import os

import numpy as np
import torch

import oracle

DEV = "cuda:0"
IN_TREE_LIB = os.path.realpath(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                            "bit_optimizer_states_amd", "libqb.so"))
TORCH_DT = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}


def qb():
    """The binding, with the in-tree libqb.so loaded (asserted: the parity
    evidence must come from the library built from these sources)."""
    from bit_optimizer_states_amd import binding
    binding.lib()
    assert binding.loaded_path() == IN_TREE_LIB, f"loaded {binding.loaded_path()}, expected {IN_TREE_LIB}"
    return binding


def host_bits(t):
    """Host numpy copy of a device tensor: fp32 as float32, 16-bit types as uint16 bits."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def to_device(a, dtype=None):
    """Device tensor from a host numpy array (uint16 bits reinterpreted as dtype)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(dtype)
    return t.to(DEV)


def packed_len(code, n):
    return (n + 1) // 2 if code in (oracle.NF4, oracle.FP4) else n


def gpu_quantize(x, code, B, double_quant=False, B2=256):
    """Quantize device tensor x with libqb; returns host arrays."""
    L = qb()
    n = x.numel()
    nb = (n + B - 1) // B
    codes = torch.full((max(packed_len(code, n), 1),), 0xAB, dtype=torch.uint8, device=DEV)
    if not double_quant:
        absmax = torch.full((max(nb, 1),), -7.0, dtype=torch.float32, device=DEV)
        L.qb_quantize(x, n, code, B, codes, absmax)
        torch.cuda.synchronize()
        return codes.cpu().numpy()[:packed_len(code, n)], absmax.cpu().numpy()[:nb]
    c2 = torch.full((max(nb, 1),), 0xAB, dtype=torch.uint8, device=DEV)
    a2 = torch.full(((nb + B2 - 1) // B2 + 1,), -7.0, dtype=torch.float32, device=DEV)
    off = torch.full((4,), -7.0, dtype=torch.float32, device=DEV)
    ws = torch.full((L.qb_dq_workspace_bytes(n, B),), 0xCD, dtype=torch.uint8, device=DEV)
    dq = L.make_dq(c2, a2, off, B2, ws)
    L.qb_quantize(x, n, code, B, codes, None, dq)
    torch.cuda.synchronize()
    return codes.cpu().numpy()[:packed_len(code, n)], {
        "c2": c2.cpu().numpy()[:nb], "absmax2": a2.cpu().numpy()[:(nb + B2 - 1) // B2],
        "mu": np.float32(off.cpu().numpy()[0]), "a2_tail": a2.cpu().numpy()[(nb + B2 - 1) // B2:]}


def gpu_dequantize(codes, state, code, B, n, ydt, B2=256):
    """Dequantize host codes/state with libqb; returns host output (bits for 16-bit)."""
    L = qb()
    y = torch.empty(max(n, 1), dtype=TORCH_DT[ydt], device=DEV)
    cd = to_device(codes if codes.size else np.zeros(1, np.uint8))
    if isinstance(state, dict):
        dq = L.make_dq(to_device(state["c2"]), to_device(state["absmax2"]),
                       to_device(np.array([state["mu"], 0, 0, 0], np.float32)), B2)
        keep = dq
        L.qb_dequantize(cd, None, dq, code, B, n, y)
    else:
        keep = to_device(state if state.size else np.zeros(1, np.float32))
        L.qb_dequantize(cd, keep, None, code, B, n, y)
    torch.cuda.synchronize()
    del keep
    return host_bits(y)[:n]


def decorate(x, B, dt, rng):
    """Overwrite a few whole blocks with special cases: all zeros, one nonzero,
    a negative maximum, tiny and huge scales, subnormals (fp32 only where the
    type cannot hold them)."""
    x = x.copy()
    nb = (x.size + B - 1) // B
    if nb < 8:
        return x
    blocks = rng.choice(nb - 1, size=7, replace=False)   # never the ragged last block
    sl = [slice(b * B, (b + 1) * B) for b in blocks]
    x[sl[0]] = 0.0
    x[sl[1]] = 0.0
    x[sl[1].start + B // 3] = 0.25
    x[sl[2]] = -np.abs(x[sl[2]])
    if dt == oracle.F32:
        x[sl[3]] *= np.float32(1e-30)           # absmax below 2^-60: the IEEE-division path
        x[sl[4]] *= np.float32(1e25)            # absmax above 2^60
        x[sl[5]] = (x[sl[5]] * np.float32(1e-37)).astype(np.float32)   # subnormals
        x[sl[6]] *= np.float32(2.0 ** 40)
    else:
        x[sl[3]] *= np.float32(1e-3)
        x[sl[4]] *= np.float32(100.0)
    return x.astype(np.float32)
