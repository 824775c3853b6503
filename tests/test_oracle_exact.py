"""Oracle pins by construction: integer-exact cases, a scale-indexing probe, textbook
special cases, metamorphic relations and global statistics.

Expected values here are computed with integer arithmetic or library routines on
values decoded by torch's float8 cast, never with the oracle's own helpers.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_bruteforce import _bf16_bits_of_fraction


def _dec(codes):
    return torch.as_tensor(codes).view(torch.float8_e4m3fn).double().numpy()


def _exp2_int(x):
    e = np.log2(np.asarray(x, dtype=np.float64))
    ei = np.round(e).astype(np.int64)
    assert np.all(np.exp2(ei) == x), "scale is not a power of two"
    return ei


def _bits_exact(v):
    """bf16 bits of a float64 value that must be exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def _canon_zero(bits):
    """Signed zeros compare equal: map -0 (0x8000) to +0."""
    b = np.asarray(bits, dtype=np.uint16).copy()
    b[b == 0x8000] = 0
    return b


def _integer_sum(A, sa, B, sb, M, N, K, shift):
    """T = sum_kb (a_kb . b_kb) * 2^(ea+eb+shift) with int64 arithmetic."""
    a = _dec(A).astype(np.int64)
    b = _dec(B).astype(np.int64)
    assert np.array_equal(a, _dec(A)) and np.array_equal(b, _dec(B))
    ea = _exp2_int(sa[:, :M])
    eb = _exp2_int(sb)
    T = np.zeros((M, N), dtype=np.int64)
    nb = np.arange(N) // 128
    for kb in range(K // 128):
        P = a[:, kb * 128:(kb + 1) * 128] @ b[:, kb * 128:(kb + 1) * 128].T
        e = ea[kb][:, None] + eb[nb, kb][None, :] + shift
        assert e.min() >= 0
        T += P * (1 << e)
    return T


@pytest.mark.parametrize("M,N,K,seed", [(128, 256, 512, 101), (77, 2112, 384, 102), (64, 300, 1024, 103)])
def test_e1_small_integer_case_is_bit_exact(M, N, K, seed):
    c = synth.dense_case(M, N, K, seed, kind="e1")
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    T = _integer_sum(A, sa, B, sb, M, N, K, shift=2)
    exact = T.astype(np.float64) / 4.0
    assert np.abs(exact).max() <= 64, "E1 generator must keep every output within +-64"
    assert np.count_nonzero(exact) > 0.5 * exact.size
    bits, S = oracle.gemm_nt(A, sa, B, sb)
    assert np.array_equal(S, exact)
    assert np.array_equal(bits, _bits_exact(exact))


@pytest.mark.parametrize("M,N,K,seed", [(128, 256, 512, 201), (64, 192, 1024, 202), (33, 130, 128, 203)])
def test_e2_ties_pin_round_to_nearest_even(M, N, K, seed):
    c = synth.dense_case(M, N, K, seed, kind="e2")
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    T = _integer_sum(A, sa, B, sb, M, N, K, shift=0)
    bits, S = oracle.gemm_nt(A, sa, B, sb)
    assert np.array_equal(S, T.astype(np.float64))
    ref = np.array([_bf16_bits_of_fraction(Fraction(int(t))) for t in T.reshape(-1)],
                   dtype=np.uint16).reshape(T.shape)
    assert np.array_equal(bits, ref)
    # the case must actually contain exact ties (odd multiples of half a bf16 ulp)
    t = np.abs(T)
    big = t >= 256
    ulp = np.exp2(np.floor(np.log2(np.maximum(t, 1))) - 7).astype(np.int64)
    ties = big & (t % ulp == ulp // 2)
    assert ties.sum() >= 20


@pytest.mark.parametrize("M,N,K,seed", [(96, 2112, 512, 301), (128, 256, 384, 302)])
def test_e3_one_hot_scale_indexing_probe(M, N, K, seed):
    c = synth.dense_case(M, N, K, seed, kind="e3")
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    a = _dec(A)
    k_of = np.argmax(a != 0, axis=1)
    assert np.all(a[np.arange(M), k_of] == 1.0) and np.all((a != 0).sum(1) == 1)
    kb = k_of // 128
    b = _dec(B)
    n = np.arange(N)
    expect = (sa[kb, np.arange(M)].astype(np.float64)[:, None]
              * sb[n // 128][:, kb].T.astype(np.float64)
              * b[:, k_of].T)
    bits, S = oracle.gemm_nt(A, sa, B, sb)
    assert np.array_equal(S, expect)
    assert np.array_equal(_canon_zero(bits), _canon_zero(_bits_exact(expect)))


def test_k128_unit_scales_equal_library_matmul():
    g = synth.make_generator(7)
    A, _ = synth.make_act(50, 128, "normal", g, "cpu")
    B, _ = synth.make_weight(70, 128, "normal", g, "cpu")
    sa = np.ones((1, 52), dtype=np.float32)
    sb = np.ones((1, 1), dtype=np.float32)
    ref = torch.matmul(torch.from_numpy(_dec(A.numpy())), torch.from_numpy(_dec(B.numpy())).T).numpy()
    _, S = oracle.gemm_nt(A.numpy(), sa, B.numpy(), sb)
    assert np.array_equal(S, ref)


def test_metamorphic_relations():
    c = synth.dense_case(64, 2112, 384, 9)
    A, sa, B, sb = (c[k].numpy() for k in ("A", "sa", "B", "sb"))
    bits, S = oracle.gemm_nt(A, sa, B, sb)
    # doubling every activation scale doubles every output exactly
    bits2, S2 = oracle.gemm_nt(A, sa * 2, B, sb)
    assert np.array_equal(S2, 2 * S)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits2), 2 * oracle.bf16_bits_to_f64(bits))
    # flipping the sign bit of every B code negates the output
    bitsn, Sn = oracle.gemm_nt(A, sa, B ^ 0x80, sb)
    assert np.array_equal(Sn, -S)
    # scaling only the partial last 128-column block (N=2112: columns 2048..2111)
    sb4 = sb.copy()
    sb4[16] *= 4
    _, S4 = oracle.gemm_nt(A, sa, B, sb4)
    assert np.array_equal(S4[:, :2048], S[:, :2048])
    assert np.array_equal(S4[:, 2048:], 4 * S[:, 2048:])
    # scaling one K block of one row touches only that block's contribution
    sa1 = sa.copy()
    sa1[1, 5] = 0.0
    _, S1 = oracle.gemm_nt(A, sa1, B, sb)
    assert np.array_equal(np.delete(S1, 5, 0), np.delete(S, 5, 0))
    blk = _dec(A[5:6, 128:256]) @ _dec(B[:, 128:256]).T * (np.float64(sa[1, 5]) * sb[np.arange(2112) // 128, 1].astype(np.float64))
    assert np.allclose(S[5] - S1[5], blk[0], rtol=1e-12, atol=1e-12 * np.abs(S[5]).max())
    # permuting rows of A (with their scales) permutes output rows
    p = np.random.default_rng(0).permutation(64)
    sap = sa.copy()
    sap[:, :64] = sa[:, p]
    bitsp, _ = oracle.gemm_nt(A[p], sap, B, sb)
    assert np.array_equal(bitsp, bits[p])
    # sampled outputs equal the same entries of the full result
    rows, cols = np.array([0, 17, 63]), np.array([0, 5, 2047, 2048, 2111])
    bs, Ss = oracle.gemm_nt_sampled(A, sa, B, sb, rows, cols)
    assert np.array_equal(Ss, S[np.ix_(rows, cols)]) and np.array_equal(bs, bits[np.ix_(rows, cols)])


def test_global_error_statistics_of_bf16_rounding():
    # relative squared error of a single BF16 rounding of N(0,1)-like data is
    # about E[(ulp/x)^2]/12 ~ 2.8e-6; the oracle's output must sit there
    c = synth.dense_case(128, 512, 512, 13)
    bits, S = oracle.gemm_nt(*(c[k].numpy() for k in ("A", "sa", "B", "sb")))
    v = oracle.bf16_bits_to_f64(bits)
    rel = ((v - S) ** 2).sum() / (S ** 2).sum()
    assert 1.5e-6 < rel < 4.5e-6, rel
    assert np.all(np.abs(v - S) <= 2.0 ** -8 * np.abs(S))  # half an ulp
