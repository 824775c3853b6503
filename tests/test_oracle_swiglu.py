"""Pins of the oracle's SwiGLU + 1x128 quantisation (oracle.swiglu,
oracle.swiglu_quantize_1x128) against facts fixed outside it: silu(0) = 0, the odd
identity silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1), scipy's logistic
function, gate on the first half, up = 1 with a large gate reducing to the pinned plain
quantiser, and padding rows quantising to zero codes with unit scales."""
import numpy as np
from scipy.special import expit

import oracle


def test_silu_zero_and_odd_identity():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(64, 128)).astype(np.float32) * 4
    ones = np.ones_like(x)
    pos = oracle.swiglu(np.concatenate([x, ones], axis=1))
    neg = oracle.swiglu(np.concatenate([-x, ones], axis=1))
    assert np.allclose(pos - neg, x.astype(np.float64), rtol=1e-14, atol=1e-14)
    z = oracle.swiglu(np.concatenate([np.zeros_like(x), ones], axis=1))
    assert np.all(z == 0.0)


def test_against_library_logistic():
    rng = np.random.default_rng(1)
    g = rng.normal(size=(32, 256)).astype(np.float32) * 3
    u = rng.normal(size=(32, 256)).astype(np.float32)
    want = g.astype(np.float64) * expit(g.astype(np.float64)) * u.astype(np.float64)
    got = oracle.swiglu(np.concatenate([g, u], axis=1))
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300)


def test_gate_is_the_first_half():
    g = np.full((1, 128), 2.0, np.float32)
    u = np.full((1, 128), 3.0, np.float32)
    a = oracle.swiglu(np.concatenate([g, u], axis=1))
    b = oracle.swiglu(np.concatenate([u, g], axis=1))
    assert np.allclose(a, 2.0 * expit(2.0) * 3.0) and np.allclose(b, 3.0 * expit(3.0) * 2.0)


def test_large_gate_with_unit_up_is_the_plain_quantiser():
    """For g >= 40, 1 + e^-g rounds to 1 in FP64, so silu(g) = g exactly."""
    rng = np.random.default_rng(2)
    g = (40.0 + rng.random(size=(8, 256)) * 400).astype(np.float32)
    q, s, y = oracle.swiglu_quantize_1x128(np.concatenate([g, np.ones_like(g)], axis=1))
    q0, s0 = oracle.quantize_1x128(g)
    assert np.array_equal(y, g) and np.array_equal(q, q0) and np.array_equal(s, s0)


def test_padding_rows_are_zero():
    rng = np.random.default_rng(3)
    h = rng.normal(size=(6, 512)).astype(np.float32)
    mi = np.array([0, -1, 2, -1, 1, 0], np.int32)
    q, s, y = oracle.swiglu_quantize_1x128(h, mi)
    assert np.all(q[mi < 0] == 0) and np.all(s[:, mi < 0] == 1.0) and np.all(y[mi < 0] == 0)
    q2, s2, _ = oracle.swiglu_quantize_1x128(h)
    assert np.array_equal(q[mi >= 0], q2[mi >= 0])
