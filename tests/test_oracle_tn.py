"""Pins of the oracle's dense TN, NN and TT GEMMs (oracle.gemm_tn, gemm_nn, gemm_tt): brute force in exact rationals on
tiny inputs (one BF16 rounding, ties to even), equality with the separately pinned NT
oracle on transposed copies of the operands, and the exact small-integer case."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from test_oracle_c import _bf16_rne_of_fraction


@pytest.mark.parametrize("seed", range(2))
def test_brute_force_exact_rationals(seed):
    M, N, K = 3, 130, 256     # N spans two 128-column scale blocks
    c = synth.dense_case(M, N, K, seed=300 + seed)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    got, _ = oracle.gemm_tn(A.T.copy(), sa, B.T.copy(), sb)
    dec = {i: Fraction(float(v)) for i, v in enumerate(oracle.decode_e4m3(np.arange(256, dtype=np.uint8)))
           if np.isfinite(v)}
    for i in range(M):
        for j in (0, 1, 127, 128, 129):
            exact = Fraction(0)
            for kb in range(K // 128):
                p = sum(dec[int(A[i, k])] * dec[int(B[j, k])] for k in range(kb * 128, kb * 128 + 128))
                exact += p * Fraction(float(sa[kb, i])) * Fraction(float(sb[j // 128, kb]))
            assert int(got[i, j]) == _bf16_rne_of_fraction(exact), (i, j)


@pytest.mark.parametrize("kind", ["normal", "e1", "e3"])
def test_equals_nt_of_transposed_operands(kind):
    c = synth.dense_case(70, 300, 384, seed=310, kind=kind)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    nt, S_nt = oracle.gemm_nt(A, sa, B, sb)
    tn, S_tn = oracle.gemm_tn(A.T.copy(), sa, B.T.copy(), sb)
    assert np.array_equal(nt, tn) and np.array_equal(S_nt, S_tn)


@pytest.mark.parametrize("kind", ["normal", "e1", "e3"])
def test_nn_and_tt_equal_nt_of_transposed_operands(kind):
    c = synth.dense_case(70, 300, 384, seed=320, kind=kind)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    nt, S_nt = oracle.gemm_nt(A, sa, B, sb)
    nn, S_nn = oracle.gemm_nn(A, sa, B.T.copy(), sb)
    tt, S_tt = oracle.gemm_tt(A.T.copy(), sa, B, sb)
    assert np.array_equal(nt, nn) and np.array_equal(S_nt, S_nn)
    assert np.array_equal(nt, tt) and np.array_equal(S_nt, S_tt)


def test_nn_tt_brute_force_exact_rationals():
    M, N, K = 2, 129, 256
    c = synth.dense_case(M, N, K, seed=330)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    nn, _ = oracle.gemm_nn(A, sa, B.T.copy(), sb)
    tt, _ = oracle.gemm_tt(A.T.copy(), sa, B, sb)
    dec = {i: Fraction(float(v)) for i, v in enumerate(oracle.decode_e4m3(np.arange(256, dtype=np.uint8)))
           if np.isfinite(v)}
    for i in range(M):
        for j in (0, 127, 128):
            exact = Fraction(0)
            for kb in range(K // 128):
                p = sum(dec[int(A[i, k])] * dec[int(B[j, k])] for k in range(kb * 128, kb * 128 + 128))
                exact += p * Fraction(float(sa[kb, i])) * Fraction(float(sb[j // 128, kb]))
            want = _bf16_rne_of_fraction(exact)
            assert int(nn[i, j]) == want and int(tt[i, j]) == want, (i, j)
