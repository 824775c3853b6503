"""Pins of the oracle's packed UE8M0 handling (oracle.ue8m0_pack / ue8m0_unpack /
ue8m0_from_fp32 / transform_sf / gemm_nt_ue8m0_packed): hand-computed words and codes
(tests/golden/ue8m0_packed_words.txt, tests/golden/ue8m0_from_fp32.txt), round trips with
a partial last word along either axis, the rounding-up rule checked in exact rationals,
the transposed layout entry by entry, and the packed GEMM against the FP32-scale GEMM
with scales decoded by math.ldexp and against exact rationals."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    rows = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, name))]
    return [r for r in rows if r]


def test_golden_words_both_directions():
    rows = _rows("ue8m0_packed_words.txt")
    assert len(rows) >= 6
    codes = np.array([[int(x) for x in r[:4]] for r in rows], dtype=np.uint8)
    words = np.array([int(r[4], 16) for r in rows], dtype=np.uint32)
    packed = oracle.ue8m0_pack(codes, axis=1).view(np.uint32)[:, 0]
    assert np.array_equal(packed, words)
    assert np.array_equal(oracle.ue8m0_unpack(words.view(np.int32)[:, None], 4, axis=1), codes)
    # the same words along axis 0 (the activation-scale orientation)
    assert np.array_equal(oracle.ue8m0_unpack(words.view(np.int32)[None, :], 4, axis=0), codes.T)


@pytest.mark.parametrize("nkb", [1, 2, 3, 4, 5, 7, 8, 9, 56])
@pytest.mark.parametrize("axis", [0, 1])
def test_round_trip_with_partial_last_word(nkb, axis):
    rng = np.random.default_rng(nkb + 10 * axis)
    shape = (nkb, 6) if axis == 0 else (5, nkb)
    codes = rng.integers(0, 256, shape, dtype=np.uint8)
    words = oracle.ue8m0_pack(codes, axis=axis)
    assert words.dtype == np.int32 and words.shape[axis] == (nkb + 3) // 4
    assert np.array_equal(oracle.ue8m0_unpack(words, nkb, axis=axis), codes)
    # bytes past nkb in the last word are zero
    full = oracle.ue8m0_unpack(words, words.shape[axis] * 4, axis=axis)
    tail = np.take(full, range(nkb, words.shape[axis] * 4), axis=axis)
    assert np.all(tail == 0)


def test_golden_codes_from_fp32():
    rows = _rows("ue8m0_from_fp32.txt")
    vals = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1]) for r in rows], dtype=np.uint8)
    assert np.array_equal(oracle.ue8m0_from_fp32(vals), want)


def test_code_is_smallest_power_of_two_not_below_the_scale():
    rng = np.random.default_rng(3)
    x = np.concatenate([np.float32(2.0) ** rng.integers(-126, 128, 200).astype(np.float32),
                        (rng.random(400) * 1e3 + 1e-30).astype(np.float32),
                        np.exp(rng.uniform(-80, 80, 400)).astype(np.float32)])
    x = x[(x >= 2.0 ** -126) & (x <= 2.0 ** 127)]
    codes = oracle.ue8m0_from_fp32(x)
    for v, c in zip(x.tolist(), codes.tolist()):
        fv = Fraction(v)
        assert Fraction(2) ** (c - 127) >= fv and Fraction(2) ** (c - 128) < fv, (v, c)


def test_transform_layouts():
    rng = np.random.default_rng(5)
    rows, nkb = 37, 6
    sf = np.float32(2.0) ** rng.integers(-20, 20, (rows, nkb)).astype(np.float32)
    sf[3, 2] = np.float32(0.3)   # not a power of two: rounds up to 0.5
    t = oracle.transform_sf(sf, True, False, ld=40)
    assert t.shape == (nkb, 40) and t.dtype == np.float32
    assert np.array_equal(t[:, :rows], sf.T) and np.all(t[:, rows:] == 0)
    tp = oracle.transform_sf(sf, True, True, ld=40)
    assert tp.shape == (2, 40) and tp.dtype == np.int32 and np.all(tp[:, rows:] == 0)
    codes = oracle.ue8m0_unpack(tp[:, :rows], nkb, axis=0)
    for m in range(rows):
        for kb in range(nkb):
            f, e = math.frexp(float(sf[m, kb]))
            assert codes[kb, m] == (e - 1 if f == 0.5 else e) + 127
    assert codes[2, 3] == 126  # 0.3 -> 2^-1
    wb = oracle.transform_sf(sf[:5], False, True)
    assert wb.shape == (5, 2) and np.array_equal(oracle.ue8m0_unpack(wb, nkb, axis=1),
                                                oracle.ue8m0_from_fp32(sf[:5]))
    assert np.array_equal(oracle.transform_sf(sf[:5], False, False), sf[:5])


@pytest.mark.parametrize("K", [128, 512, 640, 1152])
def test_packed_gemm_equals_fp32_scale_gemm_and_exact_rationals(K):
    rng = np.random.default_rng(K)
    M, N, nkb = 5, 130, K // 128
    A = rng.integers(0, 256, (M, K), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K), dtype=np.uint8)
    for X in (A, B):
        X[(X & 0x7F) == 0x7F] = 0x38
    ca = rng.integers(115, 140, (nkb, M), dtype=np.uint8)
    cb = rng.integers(115, 140, (2, nkb), dtype=np.uint8)
    bits, S = oracle.gemm_nt_ue8m0_packed(A, oracle.ue8m0_pack(ca, axis=0), B, oracle.ue8m0_pack(cb, axis=1), K)
    dec = np.vectorize(lambda c: math.ldexp(1.0, int(c) - 127))
    ref_bits, ref_S = oracle.gemm_nt(A, dec(ca).astype(np.float32), B, dec(cb).astype(np.float32))
    assert np.array_equal(bits, ref_bits) and np.array_equal(S, ref_S)

    def val(c):
        s = -1 if c & 0x80 else 1
        e, m = (c >> 3) & 0xF, c & 7
        return s * (Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    for i in range(0, M, 2):
        for j in (0, 1, 127, 128, 129):
            tot, mag = Fraction(0), Fraction(0)
            for kb in range(nkb):
                p = sum(val(int(A[i, k])) * val(int(B[j, k])) for k in range(128 * kb, 128 * kb + 128))
                t = p * Fraction(2) ** (int(ca[kb, i]) - 127) * Fraction(2) ** (int(cb[j // 128, kb]) - 127)
                tot, mag = tot + t, mag + abs(t)
            # the block partials are exact; summing nkb of them in FP64 rounds nkb times at most
            assert abs(Fraction(float(S[i, j])) - tot) <= nkb * Fraction(2) ** -53 * mag
