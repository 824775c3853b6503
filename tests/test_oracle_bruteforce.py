"""Oracle vs exact rational brute force on tiny inputs.

The brute force decodes with torch's float8 cast, sums every product in exact
rationals (fractions.Fraction) per 128-wide K block, applies both scales exactly and
rounds the rational to BF16 with integer arithmetic. None of it reuses the oracle.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16_bits_of_fraction(q: Fraction) -> int:
    if q == 0:
        return 0
    neg = q < 0
    q = -q if neg else q
    # exponent e with 2^e <= q < 2^(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    assert Fraction(2) ** e <= q < Fraction(2) ** (e + 1)
    ulp = Fraction(2) ** (max(e, -126) - 7)
    n = q / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * ulp)
    bits = struct.unpack(">I", struct.pack(">f", v))[0] >> 16
    return bits | (0x8000 if neg else 0)


def _brute(A, sa, B, sb):
    M, K = A.shape
    N = B.shape[0]
    a = torch.from_numpy(A).view(torch.float8_e4m3fn).double().numpy()
    b = torch.from_numpy(B).view(torch.float8_e4m3fn).double().numpy()
    out = np.zeros((M, N), dtype=np.uint16)
    exact = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // 128):
                part = Fraction(0)
                for k in range(kb * 128, kb * 128 + 128):
                    part += Fraction(a[m, k]) * Fraction(b[n, k])
                tot += part * Fraction(float(sa[kb, m])) * Fraction(float(sb[n // 128, kb]))
            exact[m][n] = tot
            out[m, n] = _bf16_bits_of_fraction(tot)
    return out, exact


@pytest.mark.parametrize("M,N,K,seed", [(3, 4, 128, 1), (4, 3, 256, 2), (2, 2, 384, 3), (4, 4, 256, 4)])
def test_oracle_equals_exact_rational(M, N, K, seed):
    g = synth.make_generator(seed)
    A, sa = synth.make_act(M, K, "normal", g, "cpu")
    B, sb = synth.make_weight(N, K, "normal", g, "cpu")
    ref, exact = _brute(A.numpy(), sa.numpy(), B.numpy(), sb.numpy())
    bits, S = oracle.gemm_nt(A.numpy(), sa.numpy(), B.numpy(), sb.numpy())
    assert np.array_equal(bits, ref)
    # the float64 sum is within a few ulps of the exact rational
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(S[m, n]) - exact[m][n]) <= abs(exact[m][n]) * Fraction(1, 2 ** 49) + Fraction(1, 2 ** 200)


def test_oracle_equals_exact_rational_wide_scales():
    # scales spanning many binades and an N that straddles two 128-column scale blocks
    M, N, K = 2, 3, 256
    g = synth.make_generator(11)
    A, sa = synth.make_act(M, K, "normal", g, "cpu")
    B, sb = synth.make_weight(130, K, "normal", g, "cpu")
    cols = np.array([0, 127, 128, 129])
    sa = sa * torch.exp2(torch.randint(-30, 30, sa.shape, generator=g).float())
    sb = sb * torch.exp2(torch.randint(-30, 30, sb.shape, generator=g).float())
    Bn, sbn = B.numpy(), sb.numpy()
    ref, _ = _brute(A.numpy(), sa.numpy(), Bn, sbn)
    bits, _ = oracle.gemm_nt(A.numpy(), sa.numpy(), Bn, sbn)
    assert np.array_equal(bits[:, cols], ref[:, cols])
    del N
