"""Pins of the oracle's 1x128 activation quantisation (oracle.quantize_1x128 and its
FP32 -> e4m3 rounding) against facts fixed outside it: hand-derived rounding cases,
a brute-force nearest search in exact rationals, exact round trips, zero blocks and
the half-spacing error bound."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_rne_cases.txt")


def _e4m3_exact(code):
    """Exact value of a finite e4m3 code from the format definition (bias 7)."""
    s = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _brute_code(v):
    """Nearest e4m3 code to the float v by exhaustive search, ties to the even code."""
    f = Fraction(float(v))
    best = None
    for code in range(0x7F):  # non-negative finite codes
        d = abs(abs(f) - _e4m3_exact(code))
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    code = 0x7E if abs(f) >= 448 else best[1]
    return code | (0x80 if np.signbit(np.float32(v)) else 0)


def test_rounding_cases_from_golden_file():
    rows = [l.split("#")[0].split() for l in open(GOLDEN)]
    rows = [r for r in rows if r]
    assert len(rows) >= 20
    vals = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    got = oracle.e4m3_rne_codes(vals)
    assert np.array_equal(got, want), [(v, hex(g), hex(w)) for v, g, w in zip(vals, got, want) if g != w]


def test_rounding_matches_exhaustive_search_at_every_midpoint():
    # every midpoint between neighbouring e4m3 values, its float32 neighbours, the
    # values themselves, and random magnitudes over the whole range
    vals = [_e4m3_exact(c) for c in range(0x7F)]
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = np.float32(float((a + b) / 2))
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9)), np.float32(float(a))]
    rng = np.random.default_rng(7)
    pts += list((2.0 ** rng.uniform(-12, 9.2, 400)).astype(np.float32))
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts])
    got = oracle.e4m3_rne_codes(pts)
    want = np.array([_brute_code(v) for v in pts], dtype=np.uint8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("e", [-20, -7, 0, 3, 17])
def test_blocks_on_the_e4m3_grid_round_trip_exactly(e):
    # values c * 2^e with one +-448 * 2^e per block: amax / 448 = 2^e exactly, every
    # quotient is an e4m3 value, so the codes come back unchanged
    rng = np.random.default_rng(100 + e)
    R, K = 6, 384
    codes = rng.integers(0, 0x7F, size=(R, K)).astype(np.uint8) | (rng.integers(0, 2, size=(R, K)) * 0x80).astype(np.uint8)
    codes[:, ::128] = np.where(rng.integers(0, 2, size=(R, K // 128)) > 0, 0x7E, 0xFE)
    x = (oracle.decode_e4m3(codes) * 2.0 ** e).astype(np.float32)
    q, s = oracle.quantize_1x128(x)
    assert np.array_equal(q, codes)
    assert np.all(s == np.float32(2.0 ** e)) and s.shape == (K // 128, R)


def test_zero_blocks_take_unit_scale():
    x = np.zeros((3, 256), dtype=np.float32)
    x[1, :128] = -0.0
    x[2, 128:] = np.linspace(-1, 1, 128, dtype=np.float32)
    q, s = oracle.quantize_1x128(x)
    assert s[0, 0] == 1 and s[0, 1] == 1 and s[0, 2] == 1 and s[1, 0] == 1 and s[1, 1] == 1
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80)
    assert s[1, 2] == np.float32(1.0) / np.float32(448.0)


def test_error_within_half_spacing_of_the_grid():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 1024)) * 2.0 ** rng.integers(-10, 10, size=(16, 1))).astype(np.float32)
    q, s = oracle.quantize_1x128(x)
    y = x.astype(np.float64) / np.repeat(s.T.astype(np.float64), 128, axis=1)
    spacing = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 3), 2.0 ** -9)
    err = np.abs(oracle.decode_e4m3(q) - y)
    assert np.all(err <= spacing / 2 * (1 + 2.0 ** -20) + 2.0 ** -30)
    # every block reaches +-448 at its largest element
    assert np.all(np.max(np.abs(oracle.decode_e4m3(q)).reshape(16, 8, 128), axis=-1) == 448.0)
