"""Pins of the oracle's layer-wise 8-bit optimizers, LAMB and LARS (CPU only).

The pages list 8-bit LARS and LAMB among the 8-bit optimizers ("Py之bitsandbytes",
section 1) without formulas; the oracle follows their published definitions
(LAMB: You et al., 2019, bias-corrected Adam direction plus decoupled decay,
scaled by |p| / |u| per layer; LARS: You, Gitman and Ginsburg, 2017, local rate
eta |p| / (|g| + wd |p|) inside the momentum).  Neither ships with torch, so the
pins are the closed forms of the first step from zero state, the exact
invariances of the definitions, and the identities with the other kinds.
"""
import numpy as np
import pytest

import oracle


def rnd(seed, n, scale):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def lamb32(p, g, m, v, step, **hp):
    oracle.optim32_step(oracle.LAMB, p, g, m, v, step=step, **hp)


def lars32(p, g, buf, step, **hp):
    oracle.optim32_step(oracle.LARS, p, g, buf, step=step, **hp)


LAMB_HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, wd=0.01)
LARS_HP = dict(lr=0.5, beta1=0.9, wd=5e-4, trust=0.001)


def test_lamb_first_step_closed_form():
    # from zero state the bias-corrected moments are g and g*g, so r = g / (|g| + eps)
    n = 6000
    p0, g = rnd(1, n, 0.02), rnd(2, n, 1e-2)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    lamb32(p, g, m, v, 1, **LAMB_HP)
    P, G = p0.astype(np.float64), g.astype(np.float64)
    u = G / (np.abs(G) + LAMB_HP["eps"]) + LAMB_HP["wd"] * P
    want = P - LAMB_HP["lr"] * np.linalg.norm(P) / np.linalg.norm(u) * u
    np.testing.assert_allclose(p, want, rtol=0, atol=1e-6 * 0.02)


def test_lamb_moves_each_layer_by_lr_times_its_norm():
    # the trust ratio makes |p' - p| = lr |p| at every step, for any layer scale
    for scale, seed in ((0.02, 3), (3.0, 4), (1e-4, 5)):
        n = 4097
        p = rnd(seed, n, scale)
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        for step in range(1, 6):
            p0 = p.copy()
            lamb32(p, rnd(100 * seed + step, n, 1e-3), m, v, step, **LAMB_HP)
            rel = np.linalg.norm((p - p0).astype(np.float64)) / np.linalg.norm(p0.astype(np.float64))
            assert abs(rel / LAMB_HP["lr"] - 1) < 1e-4, (scale, step, rel)


def test_lamb_states_are_adams_states():
    # the moments are Adam's: equal, bit for bit, to AdamW's after several steps
    n = 3000
    pl, pa = rnd(6, n, 0.02), rnd(6, n, 0.02)
    ml, vl, ma, va = (np.zeros(n, np.float32) for _ in range(4))
    for step in range(1, 5):
        g = rnd(60 + step, n, 1e-3)
        lamb32(pl, g, ml, vl, step, **LAMB_HP)
        oracle.optim32_step(oracle.ADAMW, pa, g, ma, va, step=step, **LAMB_HP)
    assert np.array_equal(ml, ma) and np.array_equal(vl, va)


def test_lamb_direction_is_adams_plus_decay():
    # p - p' is parallel to r + wd p, r the bias-corrected Adam direction
    # (AdamW with lr 1 and no decay moves p by exactly -r up to one rounding)
    n = 5000
    p0 = rnd(7, n, 0.02)
    m0, v0 = rnd(8, n, 1e-3), np.abs(rnd(9, n, 1e-6))
    g = rnd(10, n, 1e-3)
    p, m, v = p0.copy(), m0.copy(), v0.copy()
    lamb32(p, g, m, v, 4, **LAMB_HP)
    pa, ma, va = p0.copy(), m0.copy(), v0.copy()
    oracle.optim32_step(oracle.ADAMW, pa, g, ma, va, step=4, **dict(LAMB_HP, lr=1.0, wd=0.0))
    u = (p0.astype(np.float64) - pa) + LAMB_HP["wd"] * p0.astype(np.float64)
    d = p0.astype(np.float64) - p
    cos = np.dot(u, d) / (np.linalg.norm(u) * np.linalg.norm(d))
    assert cos > 1 - 1e-10
    assert abs(np.linalg.norm(d) / (LAMB_HP["lr"] * np.linalg.norm(p0.astype(np.float64))) - 1) < 1e-5


def test_lars_first_step_closed_form():
    n = 6000
    p0, g = rnd(11, n, 0.05), rnd(12, n, 1e-3)
    p, buf = p0.copy(), np.zeros(n, np.float32)
    lars32(p, g, buf, 1, **LARS_HP)
    P, G = p0.astype(np.float64), g.astype(np.float64)
    lam = LARS_HP["trust"] * np.linalg.norm(P) / (np.linalg.norm(G) + LARS_HP["wd"] * np.linalg.norm(P))
    want_buf = LARS_HP["lr"] * lam * (G + LARS_HP["wd"] * P)
    np.testing.assert_allclose(buf, want_buf, rtol=1e-6, atol=1e-6 * np.abs(want_buf).max())
    np.testing.assert_allclose(p, P - want_buf, rtol=0, atol=1e-6 * 0.05)


def test_lars_without_decay_moves_by_lr_eta_norm():
    # wd = 0, zero momentum state: |p' - p| = lr * eta * |p|, whatever |g|
    n = 4096
    for gs in (1e-6, 1e-3, 10.0):
        p0 = rnd(13, n, 0.02)
        p, buf = p0.copy(), np.zeros(n, np.float32)
        lars32(p, rnd(14, n, gs), buf, 1, **dict(LARS_HP, wd=0.0))
        rel = np.linalg.norm((p - p0).astype(np.float64)) / np.linalg.norm(p0.astype(np.float64))
        assert abs(rel / (LARS_HP["lr"] * LARS_HP["trust"]) - 1) < 1e-5


@pytest.mark.parametrize("kind", ["lamb", "lars"])
def test_gradient_scale_invariance_is_exact(kind):
    """Without decay both steps are invariant to scaling the gradients by 2^k
    (for LAMB with eps scaled alike): the trajectories agree bit for bit, 8-bit
    codes included (the blocks are normalized by their absmax)."""
    n, B = 2048 * 3 + 77, 2048
    two = kind == "lamb"
    k = oracle.LAMB if two else oracle.LARS
    base = dict(LAMB_HP, wd=0.0) if two else dict(LARS_HP, wd=0.0)
    runs = []
    for c in (1.0, 2.0 ** 7):
        hp = dict(base, eps=base["eps"] * c) if two else base
        p = rnd(15, n, 0.02)
        c1, a1 = np.full(n, 127, np.uint8), np.zeros(-(-n // B), np.float32)
        c2, a2 = np.full(n, 127, np.uint8), np.zeros(-(-n // B), np.float32)
        for step in range(1, 5):
            g = (rnd(150 + step, n, 1e-3) * np.float32(c)).astype(np.float32)
            oracle.optim8bit_step(k, p, g, c1, a1, c2 if two else None, a2 if two else None, B, step=step, **hp)
        runs.append((p, c1, c2))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1], runs[1][1])
    if two:
        assert np.array_equal(runs[0][2], runs[1][2])


def test_zero_norms_make_the_ratio_one():
    n = 1000
    g = rnd(16, n, 1e-3)
    # LAMB, p = 0: p' = -lr * u with u = r (the decay term is 0)
    p, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    lamb32(p, g, m, v, 1, **LAMB_HP)
    G = g.astype(np.float64)
    np.testing.assert_allclose(p, -LAMB_HP["lr"] * G / (np.abs(G) + LAMB_HP["eps"]), rtol=1e-6)
    # LARS, p = 0: buf' = lr * g exactly, p' = -buf'
    p, buf = np.zeros(n, np.float32), np.zeros(n, np.float32)
    lars32(p, g, buf, 1, **LARS_HP)
    assert np.array_equal(buf, (np.float32(LARS_HP["lr"]) * g).astype(np.float32)) and np.array_equal(p, -buf)
    # LARS, g = 0 and wd = 0: nothing moves
    p0 = rnd(17, n, 0.02)
    p, buf = p0.copy(), np.zeros(n, np.float32)
    lars32(p, np.zeros(n, np.float32), buf, 1, **dict(LARS_HP, wd=0.0))
    assert np.array_equal(p, p0) and np.all(buf == 0)


def test_norms_are_per_layer():
    # a layer's step depends on its own norms only: two layers stepped apart differ
    # from the same values stepped as one layer, and each moves by lr |p|
    n = 2000
    a, b = rnd(18, n, 0.02), rnd(19, n, 2.0)
    ga, gb = rnd(20, n, 1e-3), rnd(21, n, 1e-3)
    pa, pb, pab = a.copy(), b.copy(), np.concatenate([a, b])
    z = lambda k: np.zeros(k, np.float32)
    lamb32(pa, ga, z(n), z(n), 1, **LAMB_HP)
    lamb32(pb, gb, z(n), z(n), 1, **LAMB_HP)
    lamb32(pab, np.concatenate([ga, gb]), z(2 * n), z(2 * n), 1, **LAMB_HP)
    assert not np.array_equal(np.concatenate([pa, pb]), pab)
    for p1, p0 in ((pa, a), (pb, b)):
        assert abs(np.linalg.norm((p1 - p0).astype(np.float64)) / np.linalg.norm(p0) / LAMB_HP["lr"] - 1) < 1e-4


@pytest.mark.parametrize("kind,hp", [(oracle.LAMB, LAMB_HP), (oracle.LARS, LARS_HP)])
def test_8bit_state_is_the_quantized_binary32_update(kind, hp):
    n, B = 2048 * 4 + 333, 2048
    two = oracle.OPTIMIZER_STATES[kind] == 2
    p0, g = rnd(22, n, 0.02), rnd(23, n, 1e-3)
    c1, a1 = oracle.quantize_blockwise(rnd(24, n, 1e-3), oracle.DYN8, B)
    c2, a2 = oracle.quantize_blockwise(np.abs(rnd(25, n, 1e-6)), oracle.DYN8, B)
    x1 = oracle.dequantize_blockwise(c1, a1, oracle.DYN8, B, n)
    x2 = oracle.dequantize_blockwise(c2, a2, oracle.DYN8, B, n)
    p32 = p0.copy()
    oracle.optim32_step(kind, p32, g, x1, x2 if two else None, step=3, **hp)
    p8 = p0.copy()
    oracle.optim8bit_step(kind, p8, g, c1, a1, c2 if two else None, a2 if two else None, B, step=3, **hp)
    assert np.array_equal(p8, p32)
    q1, qa1 = oracle.quantize_blockwise(x1, oracle.DYN8, B)
    assert np.array_equal(c1, q1) and np.array_equal(a1, qa1)
    if two:
        q2, qa2 = oracle.quantize_blockwise(x2, oracle.DYN8, B)
        assert np.array_equal(c2, q2) and np.array_equal(a2, qa2)


def test_lars_needs_a_trust_coefficient():
    p = np.zeros(10, np.float32)
    with pytest.raises(RuntimeError):
        oracle.optim32_step(oracle.LARS, p, p.copy(), p.copy(), step=1, lr=0.1, beta1=0.9, trust=0.0)
