"""Pins of the oracle's D = C + A B^T (oracle.gemm_nt_c) against facts fixed outside it:
C = +0 reduces to the plain GEMM, brute-force exact rationals on tiny inputs (C + the
exact scaled sum, rounded once to BF16 with ties to even), C = -(exact product) gives
zero, and an E1-style case whose every sum is exact in FP32 has a closed-form result."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16_rne_of_fraction(x: Fraction) -> int:
    """Correctly rounded BF16 bits of a rational (normal range; ties to even)."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    q = a * 128  # 8 significant bits: [128, 256)
    n = int(q)
    frac = q - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 256:
        n = 128
        e += 1
    val = np.float32(n * 2.0 ** (e - 7))
    return sign | int(np.array([val], dtype=np.float32).view(np.uint32)[0] >> 16)


def _bf16_value(bits) -> Fraction:
    return Fraction(float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]))


def test_zero_c_is_the_plain_gemm():
    c = synth.dense_case(20, 40, 256, seed=3)
    args = [c[k].numpy() for k in ("A", "sa", "B", "sb")]
    plain, _ = oracle.gemm_nt(*args)
    with_c, _ = oracle.gemm_nt_c(*args, np.zeros((20, 40), dtype=np.uint16))
    assert np.array_equal(plain, with_c)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 3, 256
    c = synth.dense_case(M, N, K, seed=100 + seed)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    C = (rng.normal(size=(M, N)).astype(np.float32) * 4).astype(np.float32)
    C_bits = (torch.from_numpy(C).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    got, _ = oracle.gemm_nt_c(A, sa, B, sb, C_bits)
    dec = {i: Fraction(float(v)) for i, v in enumerate(oracle.decode_e4m3(np.arange(256, dtype=np.uint8)))
           if np.isfinite(v)}
    for i in range(M):
        for j in range(N):
            exact = _bf16_value(C_bits[i, j])
            for kb in range(K // 128):
                p = sum(dec[int(A[i, k])] * dec[int(B[j, k])] for k in range(kb * 128, kb * 128 + 128))
                exact += p * Fraction(float(sa[kb, i])) * Fraction(float(sb[j // 128, kb]))
            assert int(got[i, j]) == _bf16_rne_of_fraction(exact), (i, j)


def test_c_cancelling_an_exact_product_gives_zero():
    c = synth.dense_case(16, 24, 384, seed=7, kind="e1")
    args = [c[k].numpy() for k in ("A", "sa", "B", "sb")]
    d, S = oracle.gemm_nt(*args)
    neg = d ^ np.uint16(0x8000)  # -D, exact since the E1 sums are representable
    out, T = oracle.gemm_nt_c(*args, neg)
    assert np.all(T == 0.0) and np.all((out & 0x7FFF) == 0)


def test_exact_integer_case_closed_form():
    # E1 sums are multiples of 1/4 within +-64 and C multiples of 1/4 within +-64: C + S is
    # exact in FP32 and in FP64, so D is the one BF16 rounding of the exact integer sum
    rng = np.random.default_rng(11)
    c = synth.dense_case(32, 48, 512, seed=12, kind="e1")
    args = [c[k].numpy() for k in ("A", "sa", "B", "sb")]
    _, S = oracle.gemm_nt(*args)
    C = rng.integers(-256, 257, (32, 48)) / 4.0
    C_bits = torch.from_numpy(C.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.all(oracle.bf16_bits_to_f64(C_bits) == C)  # the C values are exact in BF16
    out, T = oracle.gemm_nt_c(*args, C_bits)
    assert np.all(T == S + C)
    expect = [_bf16_rne_of_fraction(Fraction(float(v))) for v in (S + C).ravel()]
    assert np.array_equal(out.ravel(), np.array(expect, dtype=np.uint16))
