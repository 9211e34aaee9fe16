"""Optimizer state buffers with the pages' bit-width policy.

8-bit optimizers keep 32-bit state for tensors with fewer than min_8bit_size
elements (4096 by default) and for tensors the caller marks 32-bit (page
"Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略", sections
如果需要高精度的参数 and 更改单个参数的位数).  This module only allocates the
zero-initialised buffers of each tensor; the step itself runs in libqb
(qb_optimizer8bit_step / qb_multi_tensor_optimizer_step take a tensor with no
absmax buffers as one with binary32 states).
"""
import torch

TWO_STATE_KINDS = (0, 1, 5)     # QB_ADAMW, QB_ADAM, QB_LAMB
RMSPROP = 4                     # QB_RMSPROP: its one state is never negative
DYN8, UDYN8 = 0, 3              # QB_DYN8, QB_UDYN8
ZERO_CODE = {DYN8: 127, UDYN8: 0}


def uses_8bit(numel, min_8bit_size=4096, force_32bit=False):
    """8-bit state unless the tensor is smaller than min_8bit_size (strictly)
    or marked 32-bit."""
    return not force_32bit and numel >= min_8bit_size


def allocate(params, kind, blocksize=2048, min_8bit_size=4096, force_32bit=(), v_code=DYN8):
    """Fresh state for each parameter tensor: a tuple (s1, s2, a1, a2) per
    tensor, the argument order of tensor_table's (m, v, absmax_m, absmax_v).
    8-bit: uint8 codes of 0.0 and zero fp32 absmax per block; 32-bit: zero
    float32 states and a1 = a2 = None.  s2 / a2 are None for the one-state
    kinds.  force_32bit: indices of tensors kept 32-bit.  v_code: the code of
    the never-negative state (v; RMSprop's state), whose 0.0 is code 0 in
    UDYN8 and 127 in DYN8."""
    two = kind in TWO_STATE_KINDS
    zero = [ZERO_CODE[v_code] if kind == RMSPROP else 127, ZERO_CODE[v_code]]
    out = []
    for i, p in enumerate(params):
        n = p.numel()
        if uses_8bit(n, min_8bit_size, i in force_32bit):
            nb = (n + blocksize - 1) // blocksize
            s = [torch.full((n,), zero[k], dtype=torch.uint8, device=p.device) for k in range(2 if two else 1)]
            a = [torch.zeros(nb, dtype=torch.float32, device=p.device) for _ in range(2 if two else 1)]
            out.append((s[0], s[1] if two else None, a[0], a[1] if two else None))
        else:
            s = [torch.zeros(n, dtype=torch.float32, device=p.device) for _ in range(2 if two else 1)]
            out.append((s[0], s[1] if two else None, None, None))
    return out
