"""CPU oracle for block-wise dynamic quantization and the 8-bit AdamW step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP library
(`bit_optimizer_states_amd`), and neither imports the other.

The arithmetic lives in `oracle.c` (plain C, one thread, every binary32 operation
rounded on its own); this module marshals numpy arrays and holds the two steps
that are clearest in exact integer arithmetic: exact rounding of a rational to
binary32 and the exact mean used by nested quantization.

Every array argument is a numpy array on the host.  bfloat16 / float16 data
travel as uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

DYN8, NF4, FP4, UDYN8 = 0, 1, 2, 3
F32, F16, BF16 = 0, 1, 2
CODE_SIZE = {DYN8: 256, NF4: 16, FP4: 16, UDYN8: 256}

_lib = None


def lib():
    """Load liboracle.so, building it from oracle.c if it is missing or stale."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        i64, i32, vp, fp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_double
        sig = {
            "orc_dyn8_codebook": [vp],
            "orc_udyn8_codebook": [vp],
            "orc_nf4_codebook": [vp],
            "orc_fp4_codebook": [vp],
            "orc_encode": [i32, vp, i64, vp],
            "orc_quantize_blockwise": [vp, i32, i64, i32, i32, vp, vp],
            "orc_dequantize_blockwise": [vp, vp, i32, i32, i64, vp, i32],
            "orc_dq_quantize": [vp, i64, fp, i32, vp, vp],
            "orc_dq_decode": [vp, vp, fp, i32, i64, vp],
            "orc_adamw32_step": [vp, vp, i32, i64, vp, vp, dp, dp, dp, dp, dp, i32],
            "orc_adamw8bit_step": [vp, vp, i32, i64, vp, vp, vp, vp, i32, dp, dp, dp, dp, dp, i32],
            "orc_adam_scalars": [dp, dp, dp, dp, dp, i32, vp],
            "orc_optim32_step": [i32, vp, i32, vp, vp, i32, i64, vp, vp],
            "orc_convert": [vp, i32, vp, i32, i64],
            "orc_linear_codebook": [vp],
            "orc_quantize_custom": [vp, i32, i64, vp, i32, vp, vp],
            "orc_dequantize_custom": [vp, vp, vp, i32, i64, vp, i32],
            "orc_estimate_quantiles": [vp, i32, i64, i32, vp],
            "orc_quantile_averages": [vp, i32, i64, i32, vp],
            "orc_optim8bit_step": [i32, vp, i32, vp, vp, i32, i64, vp, vp, vp, vp, i32, i32],
        }
        for name, argtypes in sig.items():
            f = getattr(L, name)
            f.argtypes = argtypes
            f.restype = ctypes.c_int
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_id(a):
    """numpy dtype of an element array -> oracle dtype id; uint16 arrays are
    ambiguous, so callers pass the id explicitly for them."""
    if a.dtype == np.float32:
        return F32
    raise TypeError("pass float16/bfloat16 data as uint16 bits with an explicit dtype id")


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed ({rc})")


# --------------------------------------------------------------------------
# codebooks and encoder
# --------------------------------------------------------------------------

def codebook(code):
    """Decode table indexed by the stored code (DYN8, UDYN8: 256, NF4/FP4: 16 entries)."""
    out = np.zeros(CODE_SIZE[code], dtype=np.float32)
    fn = {DYN8: lib().orc_dyn8_codebook, NF4: lib().orc_nf4_codebook, FP4: lib().orc_fp4_codebook,
          UDYN8: lib().orc_udyn8_codebook}[code]
    _check(fn(_p(out)), "codebook")
    return out


def encode(code, x):
    """Nearest code of every value of x (float32), ties toward zero."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.size, dtype=np.uint8)
    _check(lib().orc_encode(code, _p(x), x.size, _p(out)), "encode")
    return out


# --------------------------------------------------------------------------
# block-wise quantize / dequantize
# --------------------------------------------------------------------------

def packed_len(code, n):
    return (n + 1) // 2 if code in (NF4, FP4) else n


def quantize_blockwise(x, code, blocksize, xdt=None):
    """x: float32 array, or uint16 bits with xdt in (F16, BF16).
    Returns (codes uint8, absmax float32[ceil(n/B)])."""
    x = np.ascontiguousarray(x)
    if xdt is None:
        xdt = _dtype_id(x)
    n = x.size
    nb = (n + blocksize - 1) // blocksize
    codes = np.zeros(packed_len(code, n), dtype=np.uint8)
    absmax = np.zeros(nb, dtype=np.float32)
    _check(lib().orc_quantize_blockwise(_p(x), xdt, n, code, blocksize, _p(codes), _p(absmax)), "quantize")
    return codes, absmax


def dequantize_blockwise(codes, scale, code, blocksize, n, ydt=F32):
    """Returns float32 (ydt=F32) or uint16 bits (F16/BF16) of length n."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.zeros(n, dtype=np.float32 if ydt == F32 else np.uint16)
    _check(lib().orc_dequantize_blockwise(_p(codes), _p(scale), code, blocksize, n, _p(y), ydt), "dequantize")
    return y


# --------------------------------------------------------------------------
# exact rounding and the exact mean of nested quantization
# --------------------------------------------------------------------------

def _scaled(num, den, e):
    """num / (den * 2^e) as an exact pair (numerator, denominator) of integers."""
    return (num << -e, den) if e < 0 else (num, den << e)


def rn32_rational(num, den):
    """Round the non-negative rational num/den to the nearest binary32
    (ties to even), exactly, with Python integers.  Result as np.float32."""
    num, den = int(num), int(den)
    if num < 0 or den <= 0:
        raise ValueError("non-negative rational expected")
    if num == 0:
        return np.float32(0.0)
    # Pick e with 2^23 <= num / (den * 2^e) < 2^24: q = floor of that is a 24-bit
    # significand and the result is q * 2^e after rounding.
    e = num.bit_length() - den.bit_length() - 24
    while True:
        a, b = _scaled(num, den, e)
        if a >= (b << 24):
            e += 1
        elif a < (b << 23):
            e -= 1
        else:
            break
    e = max(e, -149)                     # subnormal range: the quantum stays 2^-149
    a, b = _scaled(num, den, e)
    q, r = divmod(a, b)
    if 2 * r > b or (2 * r == b and (q & 1)):
        q += 1
    if e + q.bit_length() > 128:
        raise OverflowError("value overflows binary32")
    return np.float32(np.ldexp(np.float64(q), e))   # q <= 2^24, e >= -149: exact


def exact_mean_f32(a):
    """Mean of non-negative finite binary32 values, computed exactly and rounded
    once to binary32.

    Reading (nested quantization centres the absmax values on their mean; the
    pages give no precision): the exact rational sum / count, rounded to the
    nearest binary32.  Every value is m * 2^(e-150) with an integer significand
    m < 2^24, so the sum is an exact integer multiple of 2^-149; significands are
    summed per exponent in int64 (exact) and combined with Python integers."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    nb = a.size
    if nb == 0:
        return np.float32(0.0)
    bits = a.view(np.uint32).astype(np.int64)
    if np.any(bits >> 31):
        raise ValueError("absmax values must be non-negative")
    ex = (bits >> 23) & 0xFF
    if np.any(ex == 0xFF):
        raise ValueError("absmax values must be finite")
    man = np.where(ex > 0, (bits & 0x7FFFFF) | 0x800000, bits & 0x7FFFFF)
    ex = np.maximum(ex, 1)                      # value = man * 2^(ex - 150)
    total = 0                                   # sum scaled by 2^149
    for e in np.unique(ex):
        total += int(man[ex == e].sum()) << int(e - 1)
    return rn32_rational(total, nb << 149)


# --------------------------------------------------------------------------
# nested (double) quantization
# --------------------------------------------------------------------------

def dq_quantize(absmax, blocksize2=256):
    """Nested quantization of fp32 absmax: returns (c2 uint8[nb], absmax2, mu)."""
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = absmax.size
    mu = exact_mean_f32(absmax)
    c2 = np.zeros(nb, dtype=np.uint8)
    a2 = np.zeros((nb + blocksize2 - 1) // blocksize2, dtype=np.float32)
    _check(lib().orc_dq_quantize(_p(absmax), nb, ctypes.c_float(mu), blocksize2, _p(c2), _p(a2)), "dq_quantize")
    return c2, a2, mu


def dequant_matmul(x, xdt, codes, scale, code, blocksize, N):
    """The product of a 4-bit layer in its compute dtype xdt ("Bitsandbytes",
    section QLoRA: Hesaplama veri türü): W [N, K] = the block-wise dequantized
    weights in xdt (dequantize_blockwise, per-block scale = absmax or the
    decoded nested constants), then y = x W^T with x [M, K] (float32, or uint16
    bits of xdt).  Returns (s, a): s [M, N] the product in binary64 (every
    product of two xdt values is exact there; the sum's own rounding is far
    below binary32's), a [M, N] = sum_k |x_mk w_nk| (for error bounds)."""
    M, K = x.shape
    w = dequantize_blockwise(codes, scale, code, blocksize, N * K, ydt=xdt)
    xf = (x if xdt == F32 else convert(x.reshape(-1), xdt, F32).reshape(M, K)).astype(np.float64)
    wf = (w if xdt == F32 else convert(w, xdt, F32)).astype(np.float64).reshape(N, K)
    return xf @ wf.T, np.abs(xf) @ np.abs(wf).T


def dq_decode(c2, absmax2, mu, blocksize2=256):
    c2 = np.ascontiguousarray(c2, dtype=np.uint8)
    absmax2 = np.ascontiguousarray(absmax2, dtype=np.float32)
    out = np.zeros(c2.size, dtype=np.float32)
    _check(lib().orc_dq_decode(_p(c2), _p(absmax2), ctypes.c_float(mu), blocksize2, c2.size, _p(out)), "dq_decode")
    return out


def quantize(x, code, blocksize, xdt=None, double_quant=False, blocksize2=256):
    """Full quantize: codes, and either absmax (no nesting) or the nested state
    dict(c2, absmax2, mu, absmax_fp32)."""
    codes, absmax = quantize_blockwise(x, code, blocksize, xdt)
    if not double_quant:
        return codes, absmax
    c2, a2, mu = dq_quantize(absmax, blocksize2)
    return codes, {"c2": c2, "absmax2": a2, "mu": mu, "absmax_fp32": absmax}


def dequantize(codes, state, code, blocksize, n, ydt=F32, blocksize2=256):
    """Inverse of quantize(); state is absmax or the nested dict."""
    if isinstance(state, dict):
        scale = dq_decode(state["c2"], state["absmax2"], state["mu"], blocksize2)
    else:
        scale = state
    return dequantize_blockwise(codes, scale, code, blocksize, n, ydt)


# --------------------------------------------------------------------------
# AdamW
# --------------------------------------------------------------------------

def adam_scalars(lr, beta1, beta2, eps, wd, step):
    out = np.zeros(8, dtype=np.float32)
    _check(lib().orc_adam_scalars(lr, beta1, beta2, eps, wd, step, _p(out)), "adam_scalars")
    return dict(zip(["b1", "ob1", "b2", "ob2", "s1", "s2", "dec", "eps"], out))


def adamw32_step(p, g, m, v, lr, beta1, beta2, eps, wd, step, gdt=None):
    """In-place AdamW step with binary32 state (p, m, v float32 arrays)."""
    if gdt is None:
        gdt = _dtype_id(g)
    _check(lib().orc_adamw32_step(_p(p), _p(g), gdt, p.size, _p(m), _p(v),
                                  lr, beta1, beta2, eps, wd, step), "adamw32")


def adamw8bit_step(p, g, cm, cv, am, av, blocksize, lr, beta1, beta2, eps, wd, step, gdt=None):
    """In-place 8-bit AdamW step: p float32, g float32 (or uint16 bits with gdt),
    cm/cv uint8 codes, am/av float32 block absmax."""
    for arr, dt in ((p, np.float32), (cm, np.uint8), (cv, np.uint8), (am, np.float32), (av, np.float32)):
        if arr.dtype != dt or not arr.flags.c_contiguous:
            raise TypeError("contiguous arrays of the documented dtypes expected")
    if gdt is None:
        gdt = _dtype_id(g)
    g = np.ascontiguousarray(g)
    _check(lib().orc_adamw8bit_step(_p(p), _p(g), gdt, p.size, _p(cm), _p(cv), _p(am), _p(av), blocksize,
                                    lr, beta1, beta2, eps, wd, step), "adamw8bit")


# user codes (oracle.c, section "user codes")
QUANTILE_CHUNK = 4096


def linear_codebook():
    out = np.zeros(256, dtype=np.float32)
    _check(lib().orc_linear_codebook(_p(out)), "linear_codebook")
    return out


def quantize_custom(x, cb, blocksize, xdt=None):
    """Block-wise quantization of x with the 256-entry ascending code cb."""
    x = np.ascontiguousarray(x)
    if xdt is None:
        xdt = _dtype_id(x)
    cb = np.ascontiguousarray(cb, dtype=np.float32)
    n = x.size
    codes = np.zeros(n, dtype=np.uint8)
    absmax = np.zeros((n + blocksize - 1) // blocksize, dtype=np.float32)
    _check(lib().orc_quantize_custom(_p(x), xdt, n, _p(cb), blocksize, _p(codes), _p(absmax)), "quantize_custom")
    return codes, absmax


def dequantize_custom(codes, scale, cb, blocksize, n, ydt=F32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    cb = np.ascontiguousarray(cb, dtype=np.float32)
    out = np.zeros(n, dtype=np.float32 if ydt == F32 else np.uint16)
    _check(lib().orc_dequantize_custom(_p(codes), _p(scale), _p(cb), blocksize, n, _p(out), ydt), "dequantize_custom")
    return out


def quantile_averages(x, chunk=QUANTILE_CHUNK, xdt=None):
    """The 257 quantile estimates A_j of x (binary64): the exact mean over the
    chunks of each chunk's order statistic at floor(j L / 257), rounded once."""
    x = np.ascontiguousarray(x)
    if xdt is None:
        xdt = _dtype_id(x)
    out = np.zeros(257, dtype=np.float64)
    _check(lib().orc_quantile_averages(_p(x), xdt, x.size, chunk, _p(out)), "quantile_averages")
    return out


def estimate_quantiles(x, chunk=QUANTILE_CHUNK, xdt=None):
    """The estimated quantile code of x (256 ascending entries, max |entry| 1)."""
    x = np.ascontiguousarray(x)
    if xdt is None:
        xdt = _dtype_id(x)
    out = np.zeros(256, dtype=np.float32)
    _check(lib().orc_estimate_quantiles(_p(x), xdt, x.size, chunk, _p(out)), "estimate_quantiles")
    return out


# the sibling optimizers (oracle.c, section "the sibling 8-bit optimizers")
ADAMW, ADAM, LION, SGD, RMSPROP, LAMB, LARS = 0, 1, 2, 3, 4, 5, 6
OPTIMIZER_STATES = {ADAMW: 2, ADAM: 2, LION: 1, SGD: 1, RMSPROP: 1, LAMB: 2, LARS: 1}


def _optim_hp(lr, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, dampening=0.0, nesterov=False, trust=0.0):
    return np.array([lr, beta1, beta2, eps, wd, dampening, 1.0 if nesterov else 0.0, trust], dtype=np.float64)


def convert(x, xdt, ydt):
    """x (float32, or uint16 bits of F16/BF16) converted to dtype ydt: widening
    exact, narrowing to nearest even."""
    x = np.ascontiguousarray(x)
    y = np.empty(x.size, np.float32 if ydt == F32 else np.uint16)
    _check(lib().orc_convert(_p(x), xdt, _p(y), ydt, x.size), "convert")
    return y


class _Params16:
    """A 16-bit parameter array as binary32 for the duration of a step: widened
    exactly on entry, rounded once to nearest even into the caller's array on
    exit (the update itself is the binary32 one)."""

    def __init__(self, p, pdt):
        self.p, self.pdt = p, pdt

    def __enter__(self):
        if self.pdt == F32:
            return self.p
        if self.p.dtype != np.uint16 or not self.p.flags.c_contiguous:
            raise TypeError("16-bit parameters are contiguous uint16 bit patterns")
        self.w = convert(self.p, self.pdt, F32)
        return self.w

    def __exit__(self, *exc):
        if self.pdt != F32 and exc[0] is None:
            self.p[:] = convert(self.w, F32, self.pdt)
        return False


def optim32_step(kind, p, g, x1, x2=None, step=1, gdt=None, pdt=F32, **hp):
    """In-place step of optimizer `kind` with binary32 states x1 (and x2 for the
    two-state kinds); hp: lr, beta1, beta2, eps, wd, dampening, nesterov, trust
    (the layer-wise kinds take one call per layer).  pdt: the parameters'
    dtype (F16 / BF16 parameters are uint16 bit patterns)."""
    if gdt is None:
        gdt = _dtype_id(g)
    g = np.ascontiguousarray(g)
    h = _optim_hp(**hp)
    with _Params16(p, pdt) as pw:
        _check(lib().orc_optim32_step(kind, _p(h), step, _p(pw), _p(g), gdt, pw.size, _p(x1),
                                      _p(x2) if x2 is not None else None), "optim32")


def optim8bit_step(kind, p, g, c1, a1, c2=None, a2=None, blocksize=2048, step=1, gdt=None, pdt=F32, vcode=DYN8,
                   **hp):
    """In-place 8-bit step of optimizer `kind`: states as dynamic 8-bit codes
    c1 (and c2) with block absmax a1 (and a2); pdt as for optim32_step.  vcode:
    the code of the never-negative state (v of the two-state kinds, the state
    of RMSprop), DYN8 or UDYN8."""
    two = OPTIMIZER_STATES[kind] == 2
    arrs = [(p, np.float32 if pdt == F32 else np.uint16), (c1, np.uint8), (a1, np.float32)]
    arrs += [(c2, np.uint8), (a2, np.float32)] if two else []
    for arr, dt in arrs:
        if arr.dtype != dt or not arr.flags.c_contiguous:
            raise TypeError("contiguous arrays of the documented dtypes expected")
    if gdt is None:
        gdt = _dtype_id(g)
    g = np.ascontiguousarray(g)
    h = _optim_hp(**hp)
    with _Params16(p, pdt) as pw:
        _check(lib().orc_optim8bit_step(kind, _p(h), step, _p(pw), _p(g), gdt, pw.size, _p(c1),
                                        _p(c2) if two else None, _p(a1), _p(a2) if two else None, blocksize,
                                        vcode),
               "optim8bit")


def f32_to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return np.array([lib().orc_f32_to_bf16(float(v)) for v in x], dtype=np.uint16)


def f32_to_f16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return np.array([lib().orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


def f16_bits_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return np.array([lib().orc_f16_to_f32(int(v)) for v in h], dtype=np.float32)
