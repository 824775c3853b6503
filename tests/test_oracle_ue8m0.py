"""Pins of the oracle's UE8M0 scale handling (oracle.ue8m0_decode, oracle.gemm_nt_ue8m0)
against facts fixed outside it: the format's anchor values (tests/golden/ue8m0_anchors.txt),
the IEEE-754 single-precision encoding of powers of two (the exponent field of 2^(e-127)
is e, which the GPU path reads), brute-force exact rationals on tiny GEMMs, and the
generator's power-of-two rounding of scales."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ue8m0_anchors.txt")


def test_anchor_values():
    rows = [l.split("#")[0].split() for l in open(GOLDEN)]
    rows = [r for r in rows if r]
    assert len(rows) >= 8
    for code, val in rows:
        got = oracle.ue8m0_decode(np.array([int(code)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)


def test_every_code_is_a_power_of_two_whose_fp32_exponent_field_is_the_code():
    codes = np.arange(255, dtype=np.uint8)
    v = oracle.ue8m0_decode(codes)
    assert np.all(v == np.array([math.ldexp(1.0, int(c) - 127) for c in codes]))
    f32 = v.astype(np.float32)
    assert np.all(f32.astype(np.float64) == v)                      # exact in FP32
    bits = f32.view(np.uint32)
    normal = codes >= 1
    assert np.all(((bits[normal] >> 23) & 0xFF) == codes[normal])    # exponent field = code
    assert np.all((bits[normal] & 0x7FFFFF) == 0)                    # no mantissa


@pytest.mark.parametrize("seed", range(4))
def test_gemm_with_ue8m0_codes_equals_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 4, 256
    A = rng.integers(0, 256, (M, K), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K), dtype=np.uint8)
    for X in (A, B):  # no NaN codes
        X[(X & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(110, 145, (K // 128, M), dtype=np.uint8)
    sb = rng.integers(110, 145, (1, K // 128), dtype=np.uint8)
    bits, S = oracle.gemm_nt_ue8m0(A, sa, B, sb)

    def dec(c):
        s = -1 if c & 0x80 else 1
        e, m = (c >> 3) & 0xF, c & 7
        return s * (Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    for i in range(M):
        for j in range(N):
            exact = Fraction(0)
            for kb in range(K // 128):
                p = sum(dec(int(A[i, k])) * dec(int(B[j, k])) for k in range(kb * 128, kb * 128 + 128))
                exact += p * Fraction(2) ** (int(sa[kb, i]) - 127) * Fraction(2) ** (int(sb[0, kb]) - 127)
            assert S[i, j] == float(exact)  # every term is dyadic and small: exact in FP64


def test_generator_pow2_scales():
    s = torch.tensor([1e-30, 3.0e-3, 0.25, 0.2500001, 1.0, 448.0, 1000.0], dtype=torch.float32)
    p = synth.pow2_ceil(s)
    m, _ = torch.frexp(p)
    assert bool((m == 0.5).all()), "powers of two"
    assert bool((p >= s).all() and (p < 2 * s).all()), "smallest power of two not below s"
    c = synth.dense_case(64, 256, 512, seed=5, kind="pow2")
    for key in ("sa", "sb"):
        v = c[key][c[key] != 0]
        assert bool((torch.frexp(v)[0] == 0.5).all())
    # every block fits the e4m3 range without clamping: codes never saturate more than the
    # block maximum would
    assert int((c["A"] & 0x7F).max()) <= 0x7E
