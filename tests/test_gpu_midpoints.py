"""GPU parity where a code can hinge on the last bit of the quotient.

A value's code depends on n = x / a (binary32, correctly rounded) only through
comparisons with the code's decision points, the midpoints of adjacent
entries.  An error of one ulp in n changes a code only when n lies within an
ulp of such a midpoint.  Random data lands there rarely (about 1e-6 of
elements), so these tests plant values exactly there:

  * the kernels' quotient (qb_normalize runs the quantize kernels' own
    reciprocal-multiply-correct sequence) against host IEEE division for every
    binary32 significand of the absmax at exponents inside and outside the
    range of the fast path, and for subnormal absmax;
  * every binary32 (or 16-bit input) value next to RN(m a), for every midpoint
    m of DYN8, NF4 and FP4, in blocks whose absmax is not a power of two (so
    the division is not exact), including absmax outside 2^-60 .. 2^60 where
    the kernels fall back to IEEE division: codes and absmax against the oracle;
  * the optimizer's encoders (signed DYN8 state of SGD with momentum, whose
    first state is the gradient itself; unsigned v of AdamW) with states
    steered next to every midpoint.

Each test counts the planted values whose normalized value lies within one
binary32 ulp of a midpoint and prints the count; every one of them must get
the oracle's code (none may differ)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TORCH_DT, gpu_quantize, host_bits, qb, to_device
from test_gpu_param_dtypes import lib_hp

pytestmark = pytest.mark.gpu


def midpoints(code):
    """Decision points of a code: midpoints of adjacent distinct entries (exact in binary64)."""
    v = np.unique(oracle.codebook(code).astype(np.float64))
    return (v[:-1] + v[1:]) / 2


def near_midpoint(nv, mids):
    """Mask of binary32 values within one ulp (of the midpoint) of a midpoint."""
    nv = nv.astype(np.float64)
    k = np.clip(np.searchsorted(mids, nv), 1, mids.size - 1)
    d = np.minimum(np.abs(nv - mids[k - 1]), np.abs(nv - mids[k]))
    m = np.where(np.abs(nv - mids[k - 1]) <= np.abs(nv - mids[k]), mids[k - 1], mids[k])
    return d <= np.spacing(np.abs(m).astype(np.float32)).astype(np.float64)


def f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# the quotient itself
# ---------------------------------------------------------------------------

SIG = np.arange(1 << 23, dtype=np.uint32)


@pytest.mark.parametrize("e", [-60, -20, -1, 0, 1, 20, 59, 60, -61, 61, -100, 100, -126, "subnormal"])
def test_quotient_is_ieee_for_every_significand(e):
    """n = x / a for all 2^23 significands of a at one exponent: x = 2^e (so n
    = RN(1 / significand)) and x random in [-a, a], against numpy's IEEE
    binary32 division.  Exponents -61, 61, +-100 and -126 and the subnormal
    absmax run the IEEE-division fallback; 60 and -60 are the fast range's ends."""
    L = qb()
    rng = np.random.default_rng(1000 + (e if isinstance(e, int) else 999))
    if e == "subnormal":
        a = f32(SIG[1:])                                   # every positive subnormal
        x1 = a.copy()                                      # n = 1
    else:
        a = f32(((e + 127) << 23) | SIG)
        x1 = np.full(a.size, np.float32(2.0 ** e), np.float32)
    x2 = (a.astype(np.float64) * rng.uniform(-1.0, 1.0, a.size)).astype(np.float32)
    x = np.concatenate([x1, x2])
    aa = np.concatenate([a, a])
    assert np.all(np.abs(x) <= aa)
    out = torch.empty(x.size, dtype=torch.float32, device=DEV)
    print(f"[midpoints] quotient e={e} n={x.size}", flush=True)
    L.qb_normalize(to_device(x), x.size, to_device(aa), 1, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    with np.errstate(all="ignore"):
        want = x / aa                                      # IEEE binary32 division, round to nearest even
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"e={e}: {bad.size} quotients differ, first a={aa[bad[:4]]} x={x[bad[:4]]}"


def test_normalize_follows_blocks_and_zero_absmax():
    L = qb()
    B, nb = 64, 37
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, B * nb - 5) * 0.02).astype(np.float32)
    x[3 * B:4 * B] = 0.0                                   # a zero block: n = 0
    x[5 * B + 7] = np.float32(-0.0)                        # a zero keeps its sign, as IEEE division gives it
    x[6 * B:7 * B] *= np.float32(1e-30)                    # absmax below 2^-60: the IEEE-division path
    x[6 * B + 3] = np.float32(-0.0)
    a = np.abs(np.pad(x, (0, 5)).reshape(nb, B)).max(1).astype(np.float32)
    out = torch.full((x.size + 4,), -3.0, dtype=torch.float32, device=DEV)
    L.qb_normalize(to_device(x), x.size, to_device(a), B, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    with np.errstate(all="ignore"):
        want = np.where(np.repeat(a, B)[:x.size] > 0, x / np.repeat(a, B)[:x.size], 0.0).astype(np.float32)
    assert np.array_equal(got[:x.size].view(np.uint32), want.view(np.uint32))
    assert np.all(got[x.size:] == -3.0)                    # nothing written past n


# ---------------------------------------------------------------------------
# codes of values planted next to every midpoint
# ---------------------------------------------------------------------------

def absmax_set(dt, rng):
    """Block absmax values: mostly random significands (not powers of two) over
    the fast range, its ends, all-ones significands, and values outside the
    range (IEEE-division fallback), for the input dtype."""
    if dt == oracle.F32:
        a = [f32(((int(e) + 127) << 23) | int(s)) for e, s in zip(rng.integers(-60, 60, 300),
                                                                   rng.integers(1, 1 << 23, 300))]
        a += [np.float32(2.0 ** 60), np.float32(2.0 ** -60), f32(((59 + 127) << 23) | 0x7FFFFF),
              f32(((-60 + 127) << 23) | 1)]
        a += [f32(((e + 127) << 23) | 0x7FFFFF) for e in (-40, -1, 0, 7, 33)]
        a += [np.float32(1.5 * 2.0 ** -61), np.float32(1.3 * 2.0 ** 61), np.float32(1.7 * 2.0 ** -100),
              np.float32(1.1 * 2.0 ** 100), np.float32(1.5 * 2.0 ** -126), np.float32(3e-42)]
        return np.array(a, dtype=np.float32)
    # 16-bit inputs: absmax values the dtype holds (every fp16 / bf16 value widens exactly)
    if dt == oracle.F16:
        bits = np.concatenate([rng.integers(0x0400, 0x7BFF, 200), [0x0001, 0x0003, 0x03FF, 0x7BFF, 0x3FFF]])
        bits = bits[(bits & 0x3FF) != 0]                   # not a power of two
        return bits.astype(np.uint16).view(np.float16).astype(np.float32)
    bits = np.concatenate([rng.integers(0x0080, 0x7F7F, 200), [0x0001, 0x007F, 0x7F7F, 0x4FFF, 0x2C01]])
    bits = bits[(bits & 0x7F) != 0]
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to(v, dt):
    """Round binary64 values to the input dtype (nearest even), as binary32 holders."""
    if dt == oracle.F32:
        return v.astype(np.float32)
    if dt == oracle.F16:
        return v.astype(np.float16).astype(np.float32)
    # via binary32 (a second rounding can land one bf16 step off RN(v); the
    # planted neighbours cover that step)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def neighbours(x, dt, k):
    """x and its k nearest representable neighbours of dtype dt on each side."""
    out = [x]
    if dt == oracle.F32:
        up, dn = x.copy(), x.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            out += [up.copy(), dn.copy()]
        return np.concatenate(out)
    if dt == oracle.F16:
        h = x.astype(np.float16)
        up, dn = h.copy(), h.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float16(np.inf))
            dn = np.nextafter(dn, np.float16(-np.inf))
            out += [up.astype(np.float32), dn.astype(np.float32)]
        return np.concatenate(out)
    u = (x.view(np.uint32) >> 16).astype(np.int64)         # bf16 patterns (x is bf16-exact)
    sign = u >> 15
    mag = u & 0x7FFF
    for d in range(1, k + 1):
        for s in (1, -1):
            m = np.clip(mag + s * d, 0, 0x7F7F)
            out.append(((((sign << 15) | m).astype(np.uint32)) << 16).view(np.float32))
    return np.concatenate(out)


def planted_blocks(code, dt, B, rng, k=2):
    """One block per absmax a: a itself first, then every value of dtype dt
    within k steps of RN(m a) for every midpoint m (both signs for FP4's
    magnitudes), |x| <= a, zero-filled."""
    mids = midpoints(code)
    A = absmax_set(dt, rng)
    blocks = []
    for a in A:
        x0 = round_to(mids * np.float64(a), dt)            # m a is exact in binary64
        v = neighbours(x0, dt, k)
        v = v[np.isfinite(v) & (np.abs(v) <= a)]
        v = np.unique(v)
        assert v.size < B, (code, dt, v.size)
        blk = np.zeros(B, np.float32)
        blk[0] = a
        blk[1:1 + v.size] = rng.permutation(v)
        blocks.append(blk)
    return np.concatenate(blocks), A


def as_input(x, dt):
    if dt == oracle.F32:
        return x, x
    host = torch.from_numpy(x).to(TORCH_DT[dt]).view(torch.int16).numpy().view(np.uint16).copy()
    return host, host


@pytest.mark.parametrize("code", [oracle.DYN8, oracle.NF4, oracle.FP4])
@pytest.mark.parametrize("dt", [oracle.F32, oracle.F16, oracle.BF16])
def test_codes_next_to_every_midpoint_equal_oracle(code, dt):
    L = qb()
    rng = np.random.default_rng(100 * code + dt)
    B = 4096 if code == oracle.DYN8 else 256
    x, A = planted_blocks(code, dt, B, rng)
    host, _ = as_input(x, dt)
    n = x.size
    print(f"[midpoints] code={code} dt={dt} blocks={A.size} n={n}", flush=True)
    codes, absmax = gpu_quantize(to_device(host, TORCH_DT[dt]), code, B)
    want_c, want_a = oracle.quantize_blockwise(host, code, B, xdt=dt)
    assert np.array_equal(absmax.view(np.uint32), want_a.view(np.uint32))
    assert np.array_equal(absmax, A)
    bad = np.flatnonzero(codes != want_c)
    # the normalized values the oracle encodes, and those within an ulp of a midpoint
    with np.errstate(all="ignore"):
        nv = np.where(np.repeat(A, B) > 0, x / np.repeat(A, B), 0.0).astype(np.float32)
    near = near_midpoint(nv, midpoints(code))
    print(f"[midpoints] code={code} dt={dt}: {int(near.sum())} of {n} normalized values within 1 ulp of a "
          f"midpoint; codes differing from the oracle: {bad.size}", flush=True)
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:8]}"
    if dt == oracle.F32:                                   # 16-bit inputs are coarser than an ulp of n
        assert near.sum() >= A.size, "the planted values must reach the midpoints"
    # the GPU's own quotient equals the oracle's IEEE quotient on every planted value
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    L.qb_normalize(to_device(host, TORCH_DT[dt]), n, to_device(A), B, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), nv.view(np.uint32))


# ---------------------------------------------------------------------------
# the optimizer's encoders
# ---------------------------------------------------------------------------

def test_sgd_state_next_to_every_dynamic_midpoint():
    """SGD with momentum (no decay): the first state is the gradient itself, so
    the signed dynamic code of g / absmax is planted exactly, one 2048-block
    per absmax."""
    L = qb()
    rng = np.random.default_rng(21)
    B = 2048
    mids = midpoints(oracle.DYN8)
    blocks, A = [], []
    for a in absmax_set(oracle.F32, rng)[:150]:
        v = neighbours(round_to(mids * np.float64(a), oracle.F32), oracle.F32, 1)
        v = np.unique(v[np.isfinite(v) & (np.abs(v) <= a)])
        blk = np.zeros(B, np.float32)
        blk[0] = -a if len(A) % 2 else a                   # the block max with either sign
        blk[1:1 + v.size] = rng.permutation(v)
        blocks.append(blk)
        A.append(a)
    g = np.concatenate(blocks)
    n = g.size
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(lr=1e-2, beta1=0.9, dampening=0.0)
    s = np.full(n, 127, np.uint8)
    am = np.zeros(n // B, np.float32)
    dp, ds, da = to_device(p), to_device(s), to_device(am)
    print(f"[midpoints] sgd state n={n}", flush=True)
    L.qb_optimizer8bit_step(lib_hp(oracle.SGD, hp, 1), dp, to_device(g), n, ds, None, da, None, B)
    oracle.optim8bit_step(oracle.SGD, p, g, s, am, None, None, B, step=1, gdt=oracle.F32, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(da).view(np.uint32), am.view(np.uint32))
    assert np.array_equal(am, np.array(A, np.float32))
    got = host_bits(ds)
    with np.errstate(all="ignore"):
        nv = (g / np.repeat(am, B)).astype(np.float32)
    near = near_midpoint(nv, mids)
    bad = np.flatnonzero(got != s)
    print(f"[midpoints] sgd state: {int(near.sum())} of {n} within 1 ulp of a midpoint; differing codes: "
          f"{bad.size}", flush=True)
    assert bad.size == 0 and near.sum() >= len(A)
    assert np.array_equal(host_bits(dp).view(np.uint32), p.view(np.uint32))


def test_adamw_unsigned_v_next_to_every_midpoint():
    """AdamW from zero state with v in the unsigned dynamic code: v' =
    RN((1 - beta2) RN(g g)), steered next to every unsigned-code midpoint
    times the block's absmax by gradients on a fine grid around the target."""
    L = qb()
    rng = np.random.default_rng(22)
    B = 2048
    ob2 = np.float32(1.0 - 0.999)                          # the library's and the oracle's rounded 1 - beta2
    mids = midpoints(oracle.UDYN8)
    blocks, AV = [], []
    for gmax in (rng.uniform(1e-4, 1e-2, 40) * rng.choice([-1, 1], 40)).astype(np.float32):
        av = np.float32(ob2 * np.float32(gmax * gmax))
        target = mids * np.float64(av)
        g0 = np.sqrt(target / np.float64(ob2)).astype(np.float32)
        g = neighbours(g0, oracle.F32, 3)
        g = g[np.isfinite(g) & (np.abs(g) <= np.abs(gmax)) & (g > 0)]
        g = g[np.float32(ob2 * (g * g)) <= av]
        g = np.unique(g)
        if g.size >= B:
            g = rng.choice(g, B - 1, replace=False)
        blk = np.zeros(B, np.float32)
        blk[0] = gmax
        blk[1:1 + g.size] = rng.permutation(g) * rng.choice([-1, 1], g.size).astype(np.float32)
        blocks.append(blk)
        AV.append(av)
    g = np.concatenate(blocks)
    n = g.size
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
    m, v = np.full(n, 127, np.uint8), np.zeros(n, np.uint8)
    am, av = np.zeros(n // B, np.float32), np.zeros(n // B, np.float32)
    d = [to_device(a) for a in (p, m, v, am, av)]
    h = lib_hp(oracle.ADAMW, hp, 1)
    h.v_code = L.QB_UDYN8
    print(f"[midpoints] adamw unsigned v n={n}", flush=True)
    L.qb_optimizer8bit_step(h, d[0], to_device(g), n, d[1], d[2], d[3], d[4], B)
    oracle.optim8bit_step(oracle.ADAMW, p, g, m, am, v, av, B, step=1, gdt=oracle.F32, vcode=oracle.UDYN8, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(d[4]).view(np.uint32), av.view(np.uint32))
    assert np.array_equal(av, np.array(AV, np.float32))
    vp = (ob2 * (g * g)).astype(np.float32)                # v' as both sides compute it from zero state
    with np.errstate(all="ignore"):
        nv = (vp / np.repeat(av, B)).astype(np.float32)
    near = near_midpoint(nv, mids)
    bad_v = np.flatnonzero(host_bits(d[2]) != v)
    bad_m = np.flatnonzero(host_bits(d[1]) != m)
    print(f"[midpoints] adamw unsigned v: {int(near.sum())} of {n} within 1 ulp of a midpoint; differing codes: "
          f"v {bad_v.size}, m {bad_m.size}", flush=True)
    assert bad_v.size == 0 and bad_m.size == 0
    assert np.array_equal(host_bits(d[3]).view(np.uint32), am.view(np.uint32))
    assert near.sum() >= 40
