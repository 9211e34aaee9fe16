"""Host-side checks of the HIP library (no GPU needed, no kernel runs).

  * libqb.so loads and exports every function include/qb.h declares;
  * its constant tables (built independently of the oracle) equal the oracle's;
  * the bucketed encoder the kernels run, emulated here in numpy from the
    library's own tables, equals the oracle's exact nearest-code encoder on
    every binary32 value tried (all thresholds and their neighbours included);
  * invalid arguments are rejected before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def qb():
    from bit_optimizer_states_amd import binding
    binding.lib()
    return binding


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qb_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(qb):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(qb.lib(), name), name


def test_stream_library_exports_its_header():
    """libqb_stream.so (the benchmark's HBM reference streams) exports every
    function include/qb_stream.h declares."""
    text = open(os.path.join(ROOT, "include", "qb_stream.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(qbs_[a-z0-9_]+)\s*\(", text)))
    assert names == ["qbs_adamw_pattern", "qbs_copy", "qbs_dequant4_pattern", "qbs_read", "qbs_write"]
    L = ctypes.CDLL(os.path.join(ROOT, "bit_optimizer_states_amd", "libqb_stream.so"))
    for name in names:
        assert hasattr(L, name), name


def test_binding_declares_argument_types_of_every_entry_point(qb):
    """Without argtypes ctypes passes a Python int as a 32-bit C int, which
    truncates a device pointer: every declared function must have them."""
    L = qb.lib()
    for name in declared_functions():
        f = getattr(L, name)
        assert f.argtypes is not None, f"{name}: no argtypes in the binding"


def test_binding_loads_the_in_tree_library_whatever_the_environment(qb):
    in_tree = os.path.realpath(os.path.join(ROOT, "bit_optimizer_states_amd", "libqb.so"))
    assert qb.loaded_path() == in_tree
    # a stray variable naming another build does not redirect the binding
    code = ("import bit_optimizer_states_amd.binding as b; b.lib(); print(b.loaded_path())")
    env = dict(os.environ, QB_LIBRARY="/nonexistent/libqb.so")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == in_tree


@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_codebooks_equal_oracle(qb, code):
    lib_cb = np.array(qb.qb_codebook(code), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), oracle.codebook(code).view(np.uint32))


def emulate_dyn8(table, x):
    """The kernels' dynamic-code encoder, from the library's bucket table."""
    assert len(table) == 2 * 1409
    t = np.array([e[0] for e in table], dtype=np.uint32).view(np.float32)
    pay = np.array([e[1] for e in table], dtype=np.int64)
    x = x.astype(np.float32)
    bits = x.view(np.uint32)
    mag = bits & np.uint32(0x7FFFFFFF)
    low, one = np.uint32(105 << 23), np.uint32(0x3F800000)
    cl = np.minimum(np.maximum(mag, low), one)
    b = (cl >> np.uint32(17)).astype(np.int64) - (105 << 6) + 1409 * (bits >> np.uint32(31)).astype(np.int64)
    return (pay[b] + (x >= t[b])).astype(np.uint8)


def emulate_udyn8(table, x):
    """The kernels' unsigned dynamic-code encoder (x >= 0), from the library's bucket table."""
    assert len(table) == 2817
    t = np.array([e[0] for e in table], dtype=np.uint32).view(np.float32)
    pay = np.array([e[1] for e in table], dtype=np.int64)
    x = x.astype(np.float32)
    low, one = np.uint32(105 << 23), np.uint32(0x3F800000)
    cl = np.minimum(np.maximum(x.view(np.uint32), low), one)
    b = (cl >> np.uint32(16)).astype(np.int64) - (105 << 7)
    return (pay[b] + (x >= t[b])).astype(np.uint8)


def emulate_4bit(table, x, code):
    """The documented 4-bit encoder: bucket 16 x + 16 rounded to nearest even
    (exact in binary64 before the rounding), then NF4: payload + (x >= threshold);
    FP4: byte 0 of the payload below the threshold, byte 1 from it on."""
    t = np.array([e[0] for e in table], dtype=np.uint32).view(np.float32)
    pay = np.array([e[1] for e in table], dtype=np.int64)
    x = x.astype(np.float32)
    b = np.clip(np.rint(x.astype(np.float64) * 16.0 + 16.0).astype(np.int64), 0, 32)
    if code == oracle.NF4:
        return (pay[b] + (x >= t[b])).astype(np.uint8)
    return np.where(x >= t[b], (pay[b] >> 8) & 0xFF, pay[b] & 0xFF).astype(np.uint8)


def probe_values(code, rng):
    cb = oracle.codebook(code)
    vals = [rng.uniform(-1, 1, 200000), rng.standard_normal(50000) * 1e-3,
            np.exp(rng.uniform(np.log(1e-9), 0, 100000)) * rng.choice([-1, 1], 100000)]
    srt = np.sort(np.unique(np.abs(cb) if code == oracle.FP4 else cb))
    mids = ((srt[:-1].astype(np.float64) + srt[1:]) / 2).astype(np.float32)
    near = [mids]
    for _ in range(3):
        near.append(np.nextafter(near[-1], np.float32(2)))
    down = [mids]
    for _ in range(3):
        down.append(np.nextafter(down[-1], np.float32(-2)))
    # bucket edges of the 4-bit encoder: 16 x + 16 at k + 1/2 (a tie) and one ulp either side
    ties = ((np.arange(33) - 15.5) / 16).astype(np.float32)
    edges = np.concatenate(near + down + [cb, ties, np.nextafter(ties, np.float32(2)), np.nextafter(ties, np.float32(-2))])
    x = np.concatenate(vals + [edges, -edges, [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 2.0 ** -22, -(2.0 ** -22)]])
    x = x.astype(np.float32)
    return x[np.abs(x) <= 1]


def test_dyn8_bucket_encoder_equals_oracle(qb):
    x = probe_values(oracle.DYN8, np.random.default_rng(31))
    assert np.array_equal(emulate_dyn8(qb.qb_encoder_table(0), x), oracle.encode(oracle.DYN8, x))


def test_dyn8_bucket_encoder_all_floats_in_a_binade(qb):
    # every binary32 in [0.5, 1] and [-1, -0.5]: the densest thresholds
    x = np.arange(0x3F000000, 0x3F800001, dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(emulate_dyn8(qb.qb_encoder_table(0), x), oracle.encode(oracle.DYN8, x))


def test_udyn8_bucket_encoder_equals_oracle(qb):
    """Every binary32 in [0.25, 1] (the densest thresholds) and probes down to
    the smallest entries, non-negative as the state it serves."""
    dense = np.arange(0x3E800000, 0x3F800001, dtype=np.uint32).view(np.float32)
    x = np.abs(probe_values(oracle.UDYN8, np.random.default_rng(33)))
    x = np.concatenate([dense, x, np.float32([0.0, 1e-45, 2.0 ** -23, 2.0 ** -22, 1.625e-7, 3.25e-7, 2.4e-7,
                                              5.5e-7])]).astype(np.float32)
    assert np.array_equal(emulate_udyn8(qb.qb_encoder_table(3), x), oracle.encode(oracle.UDYN8, x))


@pytest.mark.parametrize("code", [1, 2])
def test_4bit_bucket_encoder_equals_oracle(qb, code):
    x = probe_values(code, np.random.default_rng(32 + code))
    assert np.array_equal(emulate_4bit(qb.qb_encoder_table(code), x, code), oracle.encode(code, x))


def test_workspace_sizes(qb):
    bins = 64 * 256 * 8                    # 64 copies of 256 uint64 exponent bins
    assert qb.qb_dq_workspace_bytes(64 * 1000, 64) == bins + 4096
    assert qb.qb_dq_workspace_bytes(0, 64) == bins
    assert qb.qb_dq_workspace_bytes(100, 63) == 0
    assert qb.qb_multi_tensor_workspace_bytes(291) == 291 * 64 + 292 * 8 + (2 * 291 + 64 + 1) * 4
    assert qb.qb_multi_tensor_workspace_bytes(0) == 0


def test_invalid_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000  # an aligned fake device address: validation must fail before any use
    hp = qb.hparams(step=1)
    assert L.qb_quantize(A, 0, -1, 0, 256, A, A, None, None) == qb.QB_EINVAL         # n < 0
    assert L.qb_quantize(A, 0, 0, 0, 256, A, A, None, None) == qb.QB_OK              # n == 0: no-op
    assert L.qb_quantize(A, 0, 100, 0, 100, A, A, None, None) == qb.QB_EINVAL        # blocksize not a power of 2
    assert L.qb_quantize(A, 0, 100, 0, 8192, A, A, None, None) == qb.QB_EINVAL       # blocksize too large
    assert L.qb_quantize(A, 7, 100, 0, 256, A, A, None, None) == qb.QB_EINVAL        # bad dtype
    assert L.qb_quantize(A, 0, 100, 5, 256, A, A, None, None) == qb.QB_EINVAL        # bad code
    assert L.qb_quantize(A, 0, 100, 3, 256, A, A, None, None) == qb.QB_EINVAL        # the unsigned code: states only
    assert L.qb_dequantize(A, A, None, 3, 256, 100, A, 0, None) == qb.QB_EINVAL
    assert L.qb_quantize(None, 0, 100, 0, 256, A, A, None, None) == qb.QB_EINVAL     # null input
    assert L.qb_quantize(A + 4, 0, 100, 0, 256, A, A, None, None) == qb.QB_EALIGN    # misaligned
    assert L.qb_quantize(A, 0, 100, 0, 256, A, None, None, None) == qb.QB_EINVAL     # no absmax, no dq
    dq = qb.qb_dq(A, A, A, 256, A, 16)
    assert L.qb_quantize(A, 0, 100, 1, 64, A, A, ctypes.byref(dq), None) == qb.QB_EINVAL        # absmax and dq
    assert L.qb_quantize(A, 0, 6400, 1, 64, A, None, ctypes.byref(dq), None) == qb.QB_EWORKSPACE
    dq_bad = qb.qb_dq(A, A, A, 100, A, 1 << 20)
    assert L.qb_quantize(A, 0, 6400, 1, 64, A, None, ctypes.byref(dq_bad), None) == qb.QB_EINVAL
    assert L.qb_dequantize(A, None, None, 0, 256, 100, A, 0, None) == qb.QB_EINVAL   # no scale at all
    assert L.qb_dequantize(A, A, None, 0, 256, 100, A + 2, 2, None) == qb.QB_EALIGN
    assert L.qb_adamw8bit_step(A, A, 2, 100, A, A, A, A, 2048, ctypes.byref(hp), None) == qb.QB_EINVAL  # p aliases g
    A2 = A + 0x10000
    assert L.qb_adamw8bit_step(A, A2, 2, 100, A, A, A, A, 2048, None, None) == qb.QB_EINVAL
    for bad in (qb.hparams(step=0), qb.hparams(beta1=1.0), qb.hparams(eps=0.0), qb.hparams(lr=float("nan"))):
        assert L.qb_adamw8bit_step(A, A2, 2, 100, A, A, A, A, 2048, ctypes.byref(bad), None) == qb.QB_EINVAL
    assert L.qb_adamw8bit_step(A, A2, 2, 0, A, A, A, A, 2048, ctypes.byref(hp), None) == qb.QB_OK
    tab = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2, A, A, A, A, 100))
    assert L.qb_multi_tensor_step(tab, 1, 2, 2048, ctypes.byref(hp), A, 10, None) == qb.QB_EWORKSPACE
    assert L.qb_multi_tensor_step(tab, 0, 2, 2048, ctypes.byref(hp), A, 0, None) == qb.QB_OK
    tab_bad = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2 + 8, A, A, A, A, 100))
    assert L.qb_multi_tensor_step(tab_bad, 1, 2, 2048, ctypes.byref(hp), A, L.qb_multi_tensor_workspace_bytes(1), None) == qb.QB_EALIGN


def test_grouped_dequantize_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    ws = L.qb_multi_tensor_workspace_bytes(2)
    plain = qb.qb_dequant_tensor(A, A, None, None, None, A, 1000)
    nested = qb.qb_dequant_tensor(A, None, A, A, A, A, 1000)
    both = qb.qb_dequant_tensor(A, A, A, A, A, A, 1000)
    tab = lambda *e: (qb.qb_dequant_tensor * len(e))(*e)
    f = L.qb_multi_tensor_dequantize
    assert f(tab(plain), -1, 0, 64, 256, 2, A, ws, None) == qb.QB_EINVAL              # count < 0
    assert f(tab(plain), 0, 0, 64, 256, 2, A, 0, None) == qb.QB_OK                    # count == 0: no-op
    assert f(tab(plain), 1, 0, 64, 256, 2, A, 10, None) == qb.QB_EWORKSPACE
    assert f(tab(plain), 1, 0, 64, 256, 2, A + 8, ws, None) == qb.QB_EALIGN
    assert f(tab(plain), 1, 0, 100, 256, 2, A, ws, None) == qb.QB_EINVAL             # blocksize
    assert f(tab(plain), 1, 5, 64, 256, 2, A, ws, None) == qb.QB_EINVAL               # code
    assert f(tab(plain), 1, 0, 64, 256, 9, A, ws, None) == qb.QB_EINVAL               # dtype
    assert f(tab(plain, nested), 2, 0, 64, 256, 2, A, ws, None) == qb.QB_EUNSUPPORTED # mixed nesting
    assert f(tab(both), 1, 0, 64, 256, 2, A, ws, None) == qb.QB_EINVAL                # absmax and nested state
    assert f(tab(nested), 1, 0, 64, 100, 2, A, ws, None) == qb.QB_EINVAL              # blocksize2
    bad = qb.qb_dequant_tensor(A, A, None, None, None, A + 2, 1000)
    assert f(tab(bad), 1, 0, 64, 256, 2, A, ws, None) == qb.QB_EALIGN                 # misaligned output
    neg = qb.qb_dequant_tensor(A, A, None, None, None, A, -5)
    assert f(tab(neg), 1, 0, 64, 256, 2, A, ws, None) == qb.QB_EINVAL


def test_grouped_quantize_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    plain = qb.qb_quant_tensor(A, A, A, None, None, None, 1000)
    nested = qb.qb_quant_tensor(A, A, None, A, A, A, 1000)
    tab = lambda *e: (qb.qb_quant_tensor * len(e))(*e)
    wsz = L.qb_multi_tensor_quantize_workspace_bytes
    # workspace: tables only without nesting; with nesting two table regions,
    # 128 KiB of bins per tensor and the fp32 absmax (256-byte rounded)
    region = -(-(2 * 64 + 3 * 8 + (2 * 2 + 64 + 1) * 4) // 256) * 256
    assert wsz(tab(plain, plain), 2, 64) == region
    assert wsz(tab(nested, nested), 2, 64) == 2 * region + 2 * 131072 + 2 * (-(-16 * 4 // 256) * 256)
    assert wsz(tab(plain), 1, 100) == 0
    ws = wsz(tab(nested, nested), 2, 64)
    f = L.qb_multi_tensor_quantize
    assert f(tab(plain), -1, 0, 0, 64, 256, A, ws, None) == qb.QB_EINVAL               # count < 0
    assert f(tab(plain), 0, 0, 0, 64, 256, A, 0, None) == qb.QB_OK                     # count == 0: no-op
    assert f(tab(nested), 1, 0, 0, 64, 256, A, 100, None) == qb.QB_EWORKSPACE
    assert f(tab(plain), 1, 0, 0, 64, 256, A + 8, ws, None) == qb.QB_EALIGN
    assert f(tab(plain), 1, 0, 0, 100, 256, A, ws, None) == qb.QB_EINVAL              # blocksize
    assert f(tab(plain), 1, 0, 7, 64, 256, A, ws, None) == qb.QB_EINVAL               # code
    assert f(tab(plain), 1, 5, 0, 64, 256, A, ws, None) == qb.QB_EINVAL               # dtype
    assert f(tab(plain, nested), 2, 0, 0, 64, 256, A, ws, None) == qb.QB_EUNSUPPORTED  # mixed nesting
    both = qb.qb_quant_tensor(A, A, A, A, A, A, 1000)
    assert f(tab(both), 1, 0, 0, 64, 256, A, ws, None) == qb.QB_EINVAL                # absmax and nested state
    assert f(tab(nested), 1, 0, 0, 64, 100, A, ws, None) == qb.QB_EINVAL              # blocksize2
    bad = qb.qb_quant_tensor(A + 4, A, A, None, None, None, 1000)
    assert f(tab(bad), 1, 0, 0, 64, 256, A, ws, None) == qb.QB_EALIGN                 # misaligned input
    neg = qb.qb_quant_tensor(A, A, A, None, None, None, -1)
    assert f(tab(neg), 1, 0, 0, 64, 256, A, ws, None) == qb.QB_EINVAL


def test_optimizer_hyperparameters_rejected_before_launch(qb):
    L = qb.lib()
    A, A2 = 0x100000, 0x200000
    f = L.qb_optimizer8bit_step

    def call(hp, s2=A, a2=A, n=100):
        return f(ctypes.byref(hp), A, 0, A2, 2, n, A, s2, A, a2, 2048, None)

    H = qb.optim_hparams
    bad = [H(qb.QB_SGD, 0.1, beta1=0.0),                              # SGD needs momentum
           H(qb.QB_SGD, 0.1, beta1=0.9, dampening=0.1, nesterov=True), # Nesterov needs zero dampening
           H(qb.QB_SGD, 0.1, beta1=0.9, dampening=1.5),
           H(qb.QB_RMSPROP, 0.1, beta2=0.99, eps=0.0),
           H(qb.QB_RMSPROP, 0.1, beta2=1.0),
           H(qb.QB_LION, 0.1, beta1=1.0),
           H(qb.QB_ADAM, 0.1, eps=-1.0),
           H(qb.QB_ADAM, -0.1),                                        # lr < 0
           H(qb.QB_LION, 0.1, weight_decay=-1.0),
           H(qb.QB_LION, 0.1, step=0),
           H(7, 0.1),
           # the unsigned code only for a never-negative state, and only codes 0 and 3
           H(qb.QB_LION, 0.1, v_code=qb.QB_UDYN8),
           H(qb.QB_SGD, 0.1, beta1=0.9, v_code=qb.QB_UDYN8),
           H(qb.QB_ADAM, 0.1, v_code=qb.QB_NF4),
           H(qb.QB_ADAM, 0.1, v_code=7)]
    for hp in bad:
        assert call(hp) == qb.QB_EINVAL, (hp.kind, hp.beta1, hp.beta2, hp.eps, hp.dampening, hp.nesterov)
    assert f(None, A, 0, A2, 2, 100, A, A, A, A, 2048, None) == qb.QB_EINVAL
    # two-state kinds need state 2; zero length is a no-op for every kind
    assert call(H(qb.QB_ADAM, 1e-3), s2=None) == qb.QB_EINVAL
    assert call(H(qb.QB_ADAM, 1e-3), a2=A + 4) == qb.QB_EALIGN
    for k in (qb.QB_ADAMW, qb.QB_ADAM, qb.QB_LION, qb.QB_SGD, qb.QB_RMSPROP):
        assert call(H(k, 1e-3), s2=None, a2=None, n=0) == qb.QB_OK
    tab = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2, A, None, A, None, 100))
    m = L.qb_multi_tensor_optimizer_step
    assert m(ctypes.byref(H(qb.QB_ADAM, 1e-3)), tab, 1, 0, 2, 2048, A, L.qb_multi_tensor_workspace_bytes(1),
             None) == qb.QB_EINVAL                                     # Adam without state 2
    assert m(ctypes.byref(H(qb.QB_SGD, 1e-3, beta1=0.0)), tab, 1, 0, 2, 2048, A,
             L.qb_multi_tensor_workspace_bytes(1), None) == qb.QB_EINVAL
    assert m(ctypes.byref(H(qb.QB_LION, 1e-3)), tab, 1, 0, 2, 2048, A, 8, None) == qb.QB_EWORKSPACE
    # 32-bit fallback (absmax NULL): both absmax pointers NULL or neither for the two-state kinds
    assert f(ctypes.byref(H(qb.QB_ADAMW, 1e-3)), A, 0, A2, 2, 100, A, A, None, A, 2048, None) == qb.QB_EINVAL
    assert f(ctypes.byref(H(qb.QB_ADAMW, 1e-3)), A, 0, A2, 2, 100, A, A, A, None, 2048, None) == qb.QB_EINVAL
    assert f(ctypes.byref(H(qb.QB_ADAM, 1e-3)), A, 0, A2, 2, 100, A, None, None, None, 2048, None) == qb.QB_EINVAL
    assert f(ctypes.byref(H(qb.QB_SGD, 1e-3)), A, 0, A2, 2, 100, A + 4, None, None, None, 2048, None) == qb.QB_EALIGN


def test_layerwise_arguments_and_workspace(qb):
    L = qb.lib()
    A, A2 = 0x100000, 0x200000
    H = qb.optim_hparams
    f = L.qb_optimizer8bit_step
    bad = [H(qb.QB_LARS, 0.1, beta1=0.9),                                       # no trust coefficient
           H(qb.QB_LARS, 0.1, beta1=1.0, trust_coefficient=1e-3),
           H(qb.QB_LARS, 0.1, beta1=0.9, trust_coefficient=float("inf")),
           H(qb.QB_LAMB, 0.1, eps=0.0),
           H(qb.QB_LAMB, 0.1, beta2=1.0)]
    for hp in bad:
        assert f(ctypes.byref(hp), A, 0, A2, 2, 100, A, A, A, A, 2048, None) == qb.QB_EINVAL
    # valid, but the norms need a workspace: the single-tensor call refuses them
    for hp in (H(qb.QB_LAMB, 1e-3), H(qb.QB_LARS, 0.1, beta1=0.9, trust_coefficient=1e-3)):
        assert f(ctypes.byref(hp), A, 0, A2, 2, 100, A, A, A, A, 2048, None) == qb.QB_EUNSUPPORTED
    # workspace: two tensor tables, 16 bytes per group of 32 tiles (tiles of max(B, 1024) elements),
    # 4 per tensor
    tab = (qb.qb_tensor * 3)(qb.qb_tensor(A, A2, A, A, A, A, 5000), qb.qb_tensor(A, A2, A, A, A, A, 0),
                             qb.qb_tensor(A, A2, A, A, A, A, 2048 * 3 + 1))
    assert L.qb_multi_tensor_workspace_bytes(3) == 3 * 64 + 4 * 8 + (2 * 3 + 64 + 1) * 4   # 508
    region = 2 * 512                                   # two map regions, each rounded up to 256 bytes
    lamb = H(qb.QB_LAMB, 1e-3)
    assert L.qb_optimizer_workspace_bytes(ctypes.byref(lamb), tab, 3, 2048) == region + 256 + 256    # 2 groups
    assert L.qb_optimizer_workspace_bytes(ctypes.byref(lamb), tab, 3, 256) == region + 256 + 256
    assert L.qb_optimizer_workspace_bytes(ctypes.byref(H(qb.QB_ADAMW, 1e-3)), tab, 3, 2048) == 508
    big = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2, A, A, A, A, 2048 * 32 * 20 + 1))   # 641 tiles: 21 groups
    assert L.qb_optimizer_workspace_bytes(ctypes.byref(lamb), big, 1, 2048) == 2 * 512 + 512 + 256
    assert L.qb_optimizer_workspace_bytes(None, tab, 3, 2048) == 0
    assert L.qb_optimizer_workspace_bytes(ctypes.byref(lamb), tab, 3, 100) == 0
    # the step checks the larger workspace before touching the device
    m = L.qb_multi_tensor_optimizer_step
    assert m(ctypes.byref(lamb), tab, 3, 0, 2, 2048, A, region, None) == qb.QB_EWORKSPACE
    assert m(ctypes.byref(lamb), tab, 3, 0, 2, 2048, A, region + 511, None) == qb.QB_EWORKSPACE
    assert m(ctypes.byref(lamb), tab, 3, 0, 2, 2048, A, 512, None) == qb.QB_EWORKSPACE


def test_linear_code_equals_oracle(qb):
    got = np.array(qb.qb_linear_code(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.linear_codebook().view(np.uint32))
    assert qb.qb_code_table_bytes() == 6160          # entries, thresholds, bucket index


def test_normalize_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    assert L.qb_normalize(A, 0, 0, A, 64, A, None) == qb.QB_OK            # n == 0: nothing runs
    assert L.qb_normalize(A, 0, -1, A, 64, A, None) == qb.QB_EINVAL
    assert L.qb_normalize(A, 0, 100, A, 0, A, None) == qb.QB_EINVAL        # blocksize < 1
    assert L.qb_normalize(A, 7, 100, A, 64, A, None) == qb.QB_EINVAL       # dtype
    assert L.qb_normalize(A, 0, 100, None, 64, A, None) == qb.QB_EINVAL
    assert L.qb_normalize(A, 0, 100, A, 64, None, None) == qb.QB_EINVAL
    assert L.qb_normalize(A + 4, 0, 100, A, 64, A, None) == qb.QB_EALIGN
    assert L.qb_normalize(A, 0, 100, A, 64, A + 8, None) == qb.QB_EALIGN


def test_noalloc_step_arguments_rejected_before_launch(qb):
    L = qb.lib()
    hp = qb.hparams()
    assert L.qb_multi_tensor_step_noalloc(None, 0, 2, 2048, ctypes.byref(hp), None) == qb.QB_OK
    assert L.qb_multi_tensor_step_noalloc(None, -1, 2, 2048, ctypes.byref(hp), None) == qb.QB_EINVAL
    assert L.qb_multi_tensor_step_noalloc(None, 1, 2, 2048, None, None) == qb.QB_EINVAL
    # beyond the 4096 tensors its scratch holds
    assert L.qb_multi_tensor_step_noalloc(None, 4097, 2, 2048, ctypes.byref(hp), None) == qb.QB_EWORKSPACE


def test_user_code_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    good = (ctypes.c_float * 256)(*[k / 255.0 for k in range(256)])
    bad_order = (ctypes.c_float * 256)(*([0.5] + [k / 255.0 for k in range(1, 256)]))
    bad_nan = (ctypes.c_float * 256)(*([float("nan")] + [k / 255.0 for k in range(1, 256)]))
    assert L.qb_prepare_code(bad_order, A, None) == qb.QB_EINVAL
    assert L.qb_prepare_code(bad_nan, A, None) == qb.QB_EINVAL
    assert L.qb_prepare_code(good, A + 4, None) == qb.QB_EALIGN
    assert L.qb_prepare_code(None, A, None) == qb.QB_EINVAL
    assert L.qb_quantize_code(A, 0, 0, A, 256, A, A, None) == qb.QB_OK          # n == 0
    assert L.qb_quantize_code(A, 0, 100, None, 256, A, A, None) == qb.QB_EINVAL  # no table
    assert L.qb_quantize_code(A, 0, 100, A, 100, A, A, None) == qb.QB_EINVAL    # blocksize
    assert L.qb_quantize_code(A, 0, 100, A + 8, 256, A, A, None) == qb.QB_EALIGN
    assert L.qb_quantize_code(A, 0, 100, A, 256, A, None, None) == qb.QB_EINVAL  # no absmax
    assert L.qb_dequantize_code(A, A, A, 256, 0, A, 2, None) == qb.QB_OK
    assert L.qb_dequantize_code(A, None, A, 256, 100, A, 2, None) == qb.QB_EINVAL
    assert L.qb_dequantize_code(A, A, A, 256, 100, A + 2, 2, None) == qb.QB_EALIGN
    ws = L.qb_quantile_workspace_bytes(10000)
    assert ws == -(-(3 * 257 * 4) // 256) * 256 + 257 * 8
    assert L.qb_estimate_quantiles(A, 0, 0, A, None, A, ws, None) == qb.QB_EINVAL      # n < 1
    assert L.qb_estimate_quantiles(A, 0, 10000, A, None, A, ws - 8, None) == qb.QB_EWORKSPACE
    assert L.qb_estimate_quantiles(A, 5, 10000, A, None, A, ws, None) == qb.QB_EINVAL
    assert L.qb_estimate_quantiles(A, 0, 10000, A + 4, None, A, ws, None) == qb.QB_EALIGN
    assert L.qb_estimate_quantiles(A, 0, 10000, A, A + 8, A, ws, None) == qb.QB_EALIGN   # averages
    assert L.qb_quantile_workspace_bytes(4096 * 300) == -(-(300 * 257 * 4) // 256) * 256 + 257 * 8   # no group sums


def test_status_strings(qb):
    assert qb.qb_status_string(0) == "ok"
    assert "workspace" in qb.qb_status_string(5)


def test_parameter_dtype_pairs(qb):
    """16-bit parameters need gradients of the same dtype; fp32 parameters take any."""
    L = qb.lib()
    A, A2 = 0x100000, 0x200000
    f, m = L.qb_optimizer8bit_step, L.qb_multi_tensor_optimizer_step
    hp = ctypes.byref(qb.optim_hparams(qb.QB_ADAMW, 1e-3))
    F32, F16, BF16 = qb.QB_F32, qb.QB_F16, qb.QB_BF16
    for pdt, gdt, want in [(BF16, F16, qb.QB_EUNSUPPORTED), (F16, BF16, qb.QB_EUNSUPPORTED),
                           (BF16, F32, qb.QB_EUNSUPPORTED), (9, F32, qb.QB_EINVAL), (F32, 9, qb.QB_EINVAL),
                           (BF16, BF16, qb.QB_OK), (F16, F16, qb.QB_OK), (F32, BF16, qb.QB_OK)]:
        assert f(hp, A, pdt, A2, gdt, 0, A, A, A, A, 2048, None) == want, (pdt, gdt)   # n = 0: no launch
        assert m(hp, None, 0, pdt, gdt, 2048, None, 0, None) == want, (pdt, gdt)       # count = 0: no launch


def test_dequant_matmul_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    f = L.qb_dequant_matmul
    dq = qb.qb_dq(A, A, A, 256, None, 0)
    BF16, NF4, DYN8 = qb.QB_BF16, 1, 0
    assert f(A, BF16, 0, 64, A, A, None, NF4, 64, 10, A, None) == qb.QB_OK        # M = 0: no-op
    assert f(A, BF16, 4, 64, A, A, None, NF4, 64, 0, A, None) == qb.QB_OK         # N = 0: no-op
    assert f(A, BF16, 4, 48, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL    # K not a multiple of 32
    assert f(A, BF16, 4, 0, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL
    assert f(A, BF16, 4, 1 << 24, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL  # K too large
    assert f(A, BF16, -1, 64, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL
    assert f(A, BF16, 4, 64, A, A, None, DYN8, 64, 10, A, None) == qb.QB_EINVAL   # 4-bit codes only
    assert f(A, 9, 4, 64, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL
    assert f(A, BF16, 4, 64, A, A, None, NF4, 100, 10, A, None) == qb.QB_EINVAL   # block size
    assert f(A, BF16, 4, 64, A, None, None, NF4, 64, 10, A, None) == qb.QB_EINVAL  # no absmax
    assert f(A, BF16, 4, 64, A, A, ctypes.byref(dq), NF4, 64, 10, A, None) == qb.QB_EINVAL   # both
    assert f(None, BF16, 4, 64, A, A, None, NF4, 64, 10, A, None) == qb.QB_EINVAL
    assert f(A + 8, BF16, 4, 64, A, A, None, NF4, 64, 10, A, None) == qb.QB_EALIGN
    assert f(A, BF16, 4, 64, A + 8, A, None, NF4, 64, 10, A, None) == qb.QB_EALIGN
    assert f(A, BF16, 4, 64, A, A, None, NF4, 64, 10, A + 4, None) == qb.QB_EALIGN


def test_grouped_matmul_arguments_rejected_before_launch(qb):
    L = qb.lib()
    A = 0x100000
    W = qb.qb_matmul_weight
    plain = W(A, A, None, None, None, A, 64)
    nested = W(A, None, A, A, A, A, 64)
    tab = lambda *e: (W * len(e))(*e)
    f = L.qb_dequant_matmul_grouped
    assert f(A, 2, 1, 256, tab(plain), -1, 1, 64, 256, None) == qb.QB_EINVAL                 # count < 0
    assert f(A, 2, 1, 256, tab(*[plain] * 9), 9, 1, 64, 256, None) == qb.QB_EINVAL          # above the group limit
    assert f(A, 2, 1, 256, tab(plain), 0, 1, 64, 256, None) == qb.QB_OK                     # count == 0: no-op
    assert f(A, 2, 0, 256, tab(plain), 1, 1, 64, 256, None) == qb.QB_OK                     # M == 0: no-op
    assert f(A, 2, 1, 100, tab(plain), 1, 1, 64, 256, None) == qb.QB_EINVAL                 # K not a multiple of 32
    assert f(A, 2, 1, 256, tab(plain), 1, 0, 64, 256, None) == qb.QB_EINVAL                 # 8-bit code
    assert f(A, 2, 1, 256, tab(plain), 1, 1, 100, 256, None) == qb.QB_EINVAL                # blocksize
    assert f(A, 9, 1, 256, tab(plain), 1, 1, 64, 256, None) == qb.QB_EINVAL                 # dtype
    assert f(None, 2, 1, 256, tab(plain), 1, 1, 64, 256, None) == qb.QB_EINVAL              # no x
    assert f(A + 2, 2, 1, 256, tab(plain), 1, 1, 64, 256, None) == qb.QB_EALIGN             # misaligned x
    assert f(A, 2, 1, 256, tab(plain, nested), 2, 1, 64, 256, None) == qb.QB_EUNSUPPORTED   # mixed nesting
    assert f(A, 2, 1, 256, tab(nested), 1, 1, 64, 100, None) == qb.QB_EINVAL                # blocksize2
    assert f(A, 2, 1, 256, tab(W(A, A, None, None, None, A + 8, 64)), 1, 1, 64, 256, None) == qb.QB_EALIGN
    assert f(A, 2, 1, 256, tab(W(A, A, None, None, None, A, -1)), 1, 1, 64, 256, None) == qb.QB_EINVAL
    assert f(A, 2, 1, 256, tab(W(None, A, None, None, None, A, 64)), 1, 1, 64, 256, None) == qb.QB_EINVAL
    assert f(A, 2, 1, 256, tab(W(None, None, None, None, None, None, 0)), 1, 1, 64, 256, None) == qb.QB_OK  # N == 0


def test_paged_step_arguments_and_workspace(qb):
    L = qb.lib()
    A, A2 = 0x100000, 0x200000
    # two slots: two code pages (page_params bytes each) and two absmax pages, 256-byte aligned
    assert L.qb_paged_workspace_bytes(16384, 2048) == 2 * (2 * 16384 + 2 * 256)
    assert L.qb_paged_workspace_bytes(2048 * 100, 2048) == 2 * (2 * 204800 + 2 * 512)
    assert L.qb_paged_workspace_bytes(1000, 2048) == 0 and L.qb_paged_workspace_bytes(4096, 100) == 0
    f = L.qb_paged_optimizer_step
    H = qb.optim_hparams
    tab = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2, A, A, A, A, 5000))
    ws = L.qb_paged_workspace_bytes(16384, 2048)
    adamw = ctypes.byref(H(qb.QB_ADAMW, 1e-3))
    assert f(adamw, tab, 0, 0, 2, 2048, 16384, A, ws, None) == qb.QB_OK                 # count 0: no-op
    assert f(adamw, tab, 1, 0, 2, 2048, 1000, A, ws, None) == qb.QB_EINVAL              # page not a block multiple
    assert f(adamw, tab, 1, 0, 2, 2048, 16384, A, ws - 1, None) == qb.QB_EWORKSPACE
    assert f(adamw, tab, 1, 0, 2, 2048, 16384, A + 8, ws, None) == qb.QB_EALIGN
    assert f(ctypes.byref(H(qb.QB_LAMB, 1e-3)), tab, 1, 0, 2, 2048, 16384, A, ws, None) == qb.QB_EUNSUPPORTED
    s32 = (qb.qb_tensor * 1)(qb.qb_tensor(A, A2, A, A, None, None, 5000))           # binary32 states
    assert f(adamw, s32, 1, 0, 2, 2048, 16384, A, ws, None) == qb.QB_EUNSUPPORTED
    # states that are not pinned host memory are refused before anything is enqueued
    assert f(adamw, tab, 1, 0, 2, 2048, 16384, A, ws, None) == qb.QB_EINVAL
