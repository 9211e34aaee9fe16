"""ctypes binding of libqb (include/qb.h): same names, argument marshalling only.

Device buffers are torch tensors (contiguous, on the GPU); the binding passes
their data pointers and the current HIP stream of torch, checks the returned
status and raises `QbError` on anything but QB_OK.  Every computation runs in
the library's kernels; nothing here computes on the CPU.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# always the in-tree build: no environment variable can point the binding at
# another library
LIB_PATH = os.path.join(_HERE, "libqb.so")

QB_OK, QB_EINVAL, QB_EALIGN, QB_EUNSUPPORTED, QB_EHIP, QB_EWORKSPACE, QB_EINIT = range(7)
QB_F32, QB_F16, QB_BF16 = 0, 1, 2
QB_DYN8, QB_NF4, QB_FP4, QB_UDYN8 = 0, 1, 2, 3
QB_ADAMW, QB_ADAM, QB_LION, QB_SGD, QB_RMSPROP, QB_LAMB, QB_LARS = range(7)

_DTYPE = {torch.float32: QB_F32, torch.float16: QB_F16, torch.bfloat16: QB_BF16}


class QbError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {qb_status_string(status)} ({status})")


class qb_dq(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax2", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("blocksize2", ctypes.c_int32), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


class qb_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int32)]


class qb_optim_hparams(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("dampening", ctypes.c_double), ("nesterov", ctypes.c_int32), ("step", ctypes.c_int32),
                ("trust_coefficient", ctypes.c_double), ("v_code", ctypes.c_int)]


class qb_tensor(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("absmax_m", ctypes.c_void_p), ("absmax_v", ctypes.c_void_p), ("n", ctypes.c_int64)]


class qb_quant_tensor(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("c2", ctypes.c_void_p), ("absmax2", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("n", ctypes.c_int64)]


class qb_dequant_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p), ("c2", ctypes.c_void_p),
                ("absmax2", ctypes.c_void_p), ("offset", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64)]


class qb_matmul_weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p), ("c2", ctypes.c_void_p),
                ("absmax2", ctypes.c_void_p), ("offset", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64)]


QB_MATMUL_GROUP_MAX = 8

_lib = None


def loaded_path():
    """Real path of the shared object the binding has loaded (None before lib())."""
    return None if _lib is None else os.path.realpath(_lib._name)


def lib():
    """The loaded libqb.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with bit_optimizer_states_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.qb_quantize.argtypes = [vp, i32, i64, i32, i32, vp, vp, ctypes.POINTER(qb_dq), vp]
        L.qb_dequantize.argtypes = [vp, vp, ctypes.POINTER(qb_dq), i32, i32, i64, vp, i32, vp]
        L.qb_adamw8bit_step.argtypes = [vp, vp, i32, i64, vp, vp, vp, vp, i32, ctypes.POINTER(qb_adamw_hparams), vp]
        L.qb_multi_tensor_step_noalloc.argtypes = [ctypes.POINTER(qb_tensor), i32, i32, i32,
                                                   ctypes.POINTER(qb_adamw_hparams), vp]
        L.qb_multi_tensor_step.argtypes = [ctypes.POINTER(qb_tensor), i32, i32, i32, ctypes.POINTER(qb_adamw_hparams),
                                           vp, sz, vp]
        L.qb_multi_tensor_dequantize.argtypes = [ctypes.POINTER(qb_dequant_tensor), i32, i32, i32, i32, i32, vp, sz,
                                                 vp]
        L.qb_optimizer8bit_step.argtypes = [ctypes.POINTER(qb_optim_hparams), vp, i32, vp, i32, i64, vp, vp, vp, vp,
                                            i32, vp]
        L.qb_multi_tensor_optimizer_step.argtypes = [ctypes.POINTER(qb_optim_hparams), ctypes.POINTER(qb_tensor), i32,
                                                     i32, i32, i32, vp, sz, vp]
        L.qb_optimizer_workspace_bytes.argtypes = [ctypes.POINTER(qb_optim_hparams), ctypes.POINTER(qb_tensor), i32,
                                                   i32]
        L.qb_optimizer_workspace_bytes.restype = sz
        L.qb_paged_optimizer_step.argtypes = [ctypes.POINTER(qb_optim_hparams), ctypes.POINTER(qb_tensor), i32, i32,
                                              i32, i32, i64, vp, sz, vp]
        L.qb_paged_optimizer_step.restype = ctypes.c_int
        L.qb_paged_workspace_bytes.argtypes = [i64, i32]
        L.qb_paged_workspace_bytes.restype = sz
        L.qb_dequant_matmul.argtypes = [vp, i32, i64, i64, vp, vp, ctypes.POINTER(qb_dq), i32, i32, i64, vp, vp]
        L.qb_dequant_matmul.restype = ctypes.c_int
        L.qb_dequant_matmul_grouped.argtypes = [vp, i32, i64, i64, ctypes.POINTER(qb_matmul_weight), i32, i32, i32,
                                                i32, vp]
        L.qb_dequant_matmul_grouped.restype = ctypes.c_int
        L.qb_code_table_bytes.argtypes = []
        L.qb_code_table_bytes.restype = sz
        L.qb_linear_code.argtypes = [vp]
        L.qb_linear_code.restype = i32
        L.qb_prepare_code.argtypes = [vp, vp, vp]
        L.qb_normalize.argtypes = [vp, i32, i64, vp, i32, vp, vp]
        L.qb_quantile_workspace_bytes.argtypes = [i64]
        L.qb_quantile_workspace_bytes.restype = sz
        L.qb_estimate_quantiles.argtypes = [vp, i32, i64, vp, vp, vp, sz, vp]
        L.qb_quantize_code.argtypes = [vp, i32, i64, vp, i32, vp, vp, vp]
        L.qb_dequantize_code.argtypes = [vp, vp, vp, i32, i64, vp, i32, vp]
        L.qb_multi_tensor_quantize.argtypes = [ctypes.POINTER(qb_quant_tensor), i32, i32, i32, i32, i32, vp, sz, vp]
        L.qb_multi_tensor_quantize_workspace_bytes.argtypes = [ctypes.POINTER(qb_quant_tensor), i32, i32]
        L.qb_multi_tensor_quantize_workspace_bytes.restype = sz
        for f in (L.qb_quantize, L.qb_dequantize, L.qb_adamw8bit_step, L.qb_multi_tensor_step,
                  L.qb_multi_tensor_step_noalloc,
                  L.qb_multi_tensor_dequantize, L.qb_multi_tensor_quantize, L.qb_optimizer8bit_step,
                  L.qb_multi_tensor_optimizer_step, L.qb_prepare_code, L.qb_estimate_quantiles, L.qb_quantize_code,
                  L.qb_dequantize_code, L.qb_normalize):
            f.restype = ctypes.c_int
        L.qb_dq_workspace_bytes.argtypes = [i64, i32]
        L.qb_dq_workspace_bytes.restype = sz
        L.qb_multi_tensor_workspace_bytes.argtypes = [i32]
        L.qb_multi_tensor_workspace_bytes.restype = sz
        L.qb_codebook.argtypes = [i32, vp]
        L.qb_codebook.restype = i32
        L.qb_encoder_table.argtypes = [i32, vp, i32]
        L.qb_encoder_table.restype = i32
        L.qb_status_string.argtypes = [ctypes.c_int]
        L.qb_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    """Data pointer of a device tensor, or None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("torch tensor expected")
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _pinned_ptr(t):
    """Data pointer of a pinned host tensor, or None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.is_cuda or (t.numel() > 0 and not t.is_pinned()):
        raise ValueError("pinned host tensor expected")      # (an empty tensor has no storage to pin)
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status, where):
    if status != QB_OK:
        raise QbError(status, where)


def _dtype(t):
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def qb_status_string(status):
    return lib().qb_status_string(int(status)).decode()


def qb_dq_workspace_bytes(n, blocksize):
    return lib().qb_dq_workspace_bytes(int(n), int(blocksize))


def qb_multi_tensor_workspace_bytes(count):
    return lib().qb_multi_tensor_workspace_bytes(int(count))


def make_dq(codes, absmax2, offset, blocksize2, ws=None):
    """qb_dq from device tensors (ws may be None for dequantize)."""
    return qb_dq(_ptr(codes), _ptr(absmax2), _ptr(offset), int(blocksize2), _ptr(ws),
                 0 if ws is None else ws.numel() * ws.element_size())


def qb_quantize(x, n, code, blocksize, codes, absmax=None, dq=None, stream=None):
    _check(lib().qb_quantize(_ptr(x), _dtype(x), int(n), int(code), int(blocksize), _ptr(codes), _ptr(absmax),
                             ctypes.byref(dq) if dq is not None else None, _stream(stream)), "qb_quantize")


def qb_dequantize(codes, absmax, dq, code, blocksize, n, y, stream=None):
    _check(lib().qb_dequantize(_ptr(codes), _ptr(absmax), ctypes.byref(dq) if dq is not None else None, int(code),
                               int(blocksize), int(n), _ptr(y), _dtype(y), _stream(stream)), "qb_dequantize")


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1):
    return qb_adamw_hparams(lr, beta1, beta2, eps, weight_decay, int(step))


def qb_adamw8bit_step(p, g, n, m, v, absmax_m, absmax_v, blocksize, hp, stream=None):
    _check(lib().qb_adamw8bit_step(_ptr(p), _ptr(g), _dtype(g), int(n), _ptr(m), _ptr(v), _ptr(absmax_m),
                                   _ptr(absmax_v), int(blocksize), ctypes.byref(hp), _stream(stream)),
           "qb_adamw8bit_step")


def qb_dequant_matmul(x, codes, absmax, code, blocksize, N, y, dq=None, stream=None):
    """y [M, N] = x [M, K] W^T with W [N, K] as 4-bit codes (absmax, or the
    nested constants in dq); x and y of the compute dtype."""
    M, K = x.shape
    _check(lib().qb_dequant_matmul(_ptr(x), _dtype(x), int(M), int(K), _ptr(codes), _ptr(absmax),
                                   ctypes.byref(dq) if dq is not None else None, int(code), int(blocksize), int(N),
                                   _ptr(y), _stream(stream)), "qb_dequant_matmul")


def matmul_weights(weights):
    """ctypes array of qb_matmul_weight from (codes, absmax, dq, N, y) tuples
    (absmax None with a qb_dq, dq None without)."""
    arr = (qb_matmul_weight * max(len(weights), 1))()
    for i, (codes, absmax, dq, N, y) in enumerate(weights):
        arr[i] = qb_matmul_weight(_ptr(codes), _ptr(absmax), dq.codes if dq is not None else None,
                                  dq.absmax2 if dq is not None else None, dq.offset if dq is not None else None,
                                  _ptr(y), int(N))
    return arr


def qb_dequant_matmul_grouped(x, table, count, code, blocksize, blocksize2=256, stream=None):
    """y_i = x W_i^T for the `count` weights of `table` (matmul_weights) in one
    launch; x [M, K] of the compute dtype."""
    M, K = x.shape
    _check(lib().qb_dequant_matmul_grouped(_ptr(x), _dtype(x), int(M), int(K), table, int(count), int(code),
                                           int(blocksize), int(blocksize2), _stream(stream)),
           "qb_dequant_matmul_grouped")


def optim_hparams(kind, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, dampening=0.0, nesterov=False,
                  step=1, trust_coefficient=0.0, v_code=QB_DYN8):
    """v_code: the code of the never-negative state (QB_DYN8 or QB_UDYN8)."""
    return qb_optim_hparams(int(kind), lr, beta1, beta2, eps, weight_decay, dampening, 1 if nesterov else 0,
                            int(step), trust_coefficient, int(v_code))


def qb_optimizer8bit_step(hp, p, g, n, state1, state2, absmax1, absmax2, blocksize, stream=None):
    """state2 / absmax2 may be None for the one-state kinds; the parameter and
    gradient dtypes are those of p and g."""
    _check(lib().qb_optimizer8bit_step(ctypes.byref(hp), _ptr(p), _dtype(p), _ptr(g), _dtype(g), int(n), _ptr(state1),
                                       _ptr(state2), _ptr(absmax1), _ptr(absmax2), int(blocksize), _stream(stream)),
           "qb_optimizer8bit_step")


def tensor_table(tensors):
    """ctypes array of qb_tensor from tuples (p, g, m, v, absmax_m, absmax_v);
    v and absmax_v may be None for the one-state optimizers."""
    arr = (qb_tensor * len(tensors))()
    for i, (p, g, m, v, am, av) in enumerate(tensors):
        arr[i] = qb_tensor(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(am), _ptr(av), p.numel())
    return arr


def qb_optimizer_workspace_bytes(hp, table, count, blocksize):
    return lib().qb_optimizer_workspace_bytes(ctypes.byref(hp), table, int(count), int(blocksize))


def qb_multi_tensor_optimizer_step(hp, table, count, gdt, blocksize, ws, stream=None, pdt=QB_F32):
    _check(lib().qb_multi_tensor_optimizer_step(ctypes.byref(hp), table, int(count), int(pdt), int(gdt),
                                                int(blocksize), _ptr(ws), ws.numel() * ws.element_size(),
                                                _stream(stream)),
           "qb_multi_tensor_optimizer_step")


def paged_tensor_table(tensors):
    """ctypes array of qb_tensor for the paged step from tuples (p, g, m, v,
    absmax_m, absmax_v): p, g device tensors; the states pinned host tensors
    (v and absmax_v may be None for the one-state optimizers)."""
    arr = (qb_tensor * len(tensors))()
    for i, (p, g, m, v, am, av) in enumerate(tensors):
        arr[i] = qb_tensor(_ptr(p), _ptr(g), _pinned_ptr(m), _pinned_ptr(v), _pinned_ptr(am), _pinned_ptr(av),
                           p.numel())
    return arr


def qb_paged_workspace_bytes(page_params, blocksize):
    return lib().qb_paged_workspace_bytes(int(page_params), int(blocksize))


def qb_paged_optimizer_step(hp, table, count, gdt, blocksize, page_params, ws, stream=None, pdt=QB_F32):
    """table: tensor_table() rows with p, g on the device and the states in
    pinned host memory (torch pin_memory=True)."""
    _check(lib().qb_paged_optimizer_step(ctypes.byref(hp), table, int(count), int(pdt), int(gdt), int(blocksize),
                                         int(page_params), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "qb_paged_optimizer_step")


def qb_multi_tensor_step(table, count, gdt, blocksize, hp, ws, stream=None):
    """table: result of tensor_table(); gdt: QB_F32/QB_F16/QB_BF16; ws: device byte tensor."""
    _check(lib().qb_multi_tensor_step(table, int(count), int(gdt), int(blocksize), ctypes.byref(hp), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)), "qb_multi_tensor_step")


def qb_multi_tensor_step_noalloc(table, count, gdt, blocksize, hp, stream=None):
    """qb_multi_tensor_step with the library's own scratch in place of ws."""
    _check(lib().qb_multi_tensor_step_noalloc(table, int(count), int(gdt), int(blocksize), ctypes.byref(hp),
                                              _stream(stream)), "qb_multi_tensor_step_noalloc")


def quant_table(entries):
    """Host array of qb_quant_tensor from (x, n, codes, absmax, dq) tuples;
    absmax is None for a nested tensor, whose dq is a qb_dq (make_dq; its ws
    is not used)."""
    arr = (qb_quant_tensor * len(entries))()
    for i, (x, n, codes, absmax, dq) in enumerate(entries):
        arr[i] = qb_quant_tensor(_ptr(x), _ptr(codes), _ptr(absmax), dq.codes if dq is not None else None,
                                 dq.absmax2 if dq is not None else None, dq.offset if dq is not None else None, int(n))
    return arr


def qb_multi_tensor_quantize_workspace_bytes(table, count, blocksize):
    return lib().qb_multi_tensor_quantize_workspace_bytes(table, int(count), int(blocksize))


def qb_multi_tensor_quantize(table, count, xdt, code, blocksize, blocksize2, ws, stream=None):
    """table: result of quant_table(); xdt: QB_F32/QB_F16/QB_BF16; ws: device byte tensor."""
    _check(lib().qb_multi_tensor_quantize(table, int(count), int(xdt), int(code), int(blocksize), int(blocksize2),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qb_multi_tensor_quantize")


def dequant_table(entries):
    """Host array of qb_dequant_tensor from (codes, absmax, dq, n, y) tuples;
    absmax is None for a nested tensor, whose dq is a qb_dq (make_dq)."""
    arr = (qb_dequant_tensor * len(entries))()
    for i, (codes, absmax, dq, n, y) in enumerate(entries):
        arr[i] = qb_dequant_tensor(_ptr(codes), _ptr(absmax), dq.codes if dq is not None else None,
                                   dq.absmax2 if dq is not None else None, dq.offset if dq is not None else None,
                                   _ptr(y), int(n))
    return arr


def qb_multi_tensor_dequantize(table, count, code, blocksize, blocksize2, ydt, ws, stream=None):
    """table: result of dequant_table(); ydt: QB_F32/QB_F16/QB_BF16; ws: device byte tensor."""
    _check(lib().qb_multi_tensor_dequantize(table, int(count), int(code), int(blocksize), int(blocksize2), int(ydt),
                                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qb_multi_tensor_dequantize")


def qb_code_table_bytes():
    return lib().qb_code_table_bytes()


def qb_linear_code():
    """Host list of the linear code's 256 entries."""
    out = (ctypes.c_float * 256)()
    lib().qb_linear_code(out)
    return list(out)


def qb_prepare_code(values, table, stream=None):
    """values: 256 host floats (ascending); table: device byte tensor of qb_code_table_bytes()."""
    arr = (ctypes.c_float * 256)(*[float(v) for v in values])
    _check(lib().qb_prepare_code(arr, _ptr(table), _stream(stream)), "qb_prepare_code")


def qb_normalize(x, n, absmax, blocksize, out, stream=None):
    _check(lib().qb_normalize(_ptr(x), _dtype(x), int(n), _ptr(absmax), int(blocksize), _ptr(out), _stream(stream)),
           "qb_normalize")


def qb_quantile_workspace_bytes(n):
    return lib().qb_quantile_workspace_bytes(int(n))


def qb_estimate_quantiles(x, n, table, ws, averages=None, stream=None):
    _check(lib().qb_estimate_quantiles(_ptr(x), _dtype(x), int(n), _ptr(table), _ptr(averages), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)), "qb_estimate_quantiles")


def qb_quantize_code(x, n, table, blocksize, codes, absmax, stream=None):
    _check(lib().qb_quantize_code(_ptr(x), _dtype(x), int(n), _ptr(table), int(blocksize), _ptr(codes), _ptr(absmax),
                                  _stream(stream)), "qb_quantize_code")


def qb_dequantize_code(codes, absmax, table, blocksize, n, y, stream=None):
    _check(lib().qb_dequantize_code(_ptr(codes), _ptr(absmax), _ptr(table), int(blocksize), int(n), _ptr(y),
                                    _dtype(y), _stream(stream)), "qb_dequantize_code")


def qb_codebook(code):
    """Host decode table of `code` as a list of floats."""
    out = (ctypes.c_float * 256)()
    k = lib().qb_codebook(int(code), out)
    if k < 0:
        raise QbError(QB_EINIT, "qb_codebook")
    return list(out[:k])


def qb_encoder_table(code):
    """Host encoder bucket table as a list of (threshold bits, payload) pairs."""
    k = lib().qb_encoder_table(int(code), None, 0)
    if k < 0:
        raise QbError(QB_EINIT, "qb_encoder_table")
    out = (ctypes.c_uint32 * (2 * k))()
    lib().qb_encoder_table(int(code), out, k)
    return [(out[2 * i], out[2 * i + 1]) for i in range(k)]
