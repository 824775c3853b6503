"""Pins of the oracle's K-grouped TN GEMM (oracle.k_grouped_tn) against facts fixed
outside it: brute force in exact rationals on tiny inputs (one rounding to FP32, ties
to even), the reduction of a single group to the already pinned NT GEMM (A^T, B^T and
a per-column B scale that is constant over 128-column blocks), a closed form for
all-ones operands with power-of-two scales (any wrong K-block or scale index shows as
a wrong power of two), independence of a group from the K rows of the others, the
split of one segment into two groups, and accumulation into an old D."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

ONE = 0x38  # e4m3 code of 1.0


def _f32_rne_of_fraction(x: Fraction) -> np.float32:
    """The FP32 value nearest to a rational (ties to the even significand)."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        even = int(np.array([c], dtype=np.float32).view(np.uint32)[0]) % 2 == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _host(c):
    return [c[k].numpy() for k in ("A", "sa", "B", "sb")]


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_exact_rationals(seed):
    M, N = 3, 2
    c = synth.k_grouped_case([100, 0, 256], M, N, seed=200 + seed)
    A, sa, B, sb = _host(c)
    ks = c["ks"]
    rng = np.random.default_rng(seed)
    D_in = rng.normal(size=(len(ks), M, N)).astype(np.float32) if seed == 2 else None
    got, _ = oracle.k_grouped_tn(A, sa, B, sb, ks, D_in)
    dec = {i: Fraction(float(v)) for i, v in enumerate(oracle.decode_e4m3(np.arange(256, dtype=np.uint8)))
           if np.isfinite(v)}
    k0 = 0
    for g, kg in enumerate(ks):
        for m in range(M):
            for n in range(N):
                exact = Fraction(float(D_in[g, m, n])) if D_in is not None else Fraction(0)
                for kb in range(k0 // 128, (k0 + kg) // 128):
                    p = sum(dec[int(A[k, m])] * dec[int(B[k, n])] for k in range(kb * 128, kb * 128 + 128))
                    exact += p * Fraction(float(sa[kb, m])) * Fraction(float(sb[kb, n]))
                assert got[g, m, n] == _f32_rne_of_fraction(exact), (g, m, n)
        k0 += kg


def test_single_group_is_the_nt_gemm_transposed():
    """One group over all of K with sb[kb, n] = sb_nt[n // 128, kb] is the NT GEMM of
    A^T and B^T (whose oracle has its own pins), to the last bit of the FP64 sum."""
    M, N, K = 40, 300, 512
    d = synth.dense_case(M, N, K, seed=11)
    A, sa, B, sb_nt = (d[k].numpy() for k in ("A", "sa", "B", "sb"))
    sb_cols = sb_nt[np.arange(N) // 128, :].T.copy()          # [K/128, N]
    S_nt = oracle.scaled_block_sum(A, sa, B, sb_nt)
    S_tn = oracle.k_grouped_tn_sum(A.T.copy(), sa, B.T.copy(), sb_cols, 0, K)
    assert np.array_equal(S_nt, S_tn)


def test_closed_form_all_ones_with_power_of_two_scales():
    """A = B = 1: D[g, m, n] = 128 * sum_{kb in g} 2^(ea[kb, m] + eb[kb, n]), exactly."""
    rng = np.random.default_rng(5)
    ks = [256, 128, 0, 384]
    K, M, N = sum(ks), 7, 9
    A = np.full((K, M), ONE, np.uint8)
    B = np.full((K, N), ONE, np.uint8)
    ea = rng.integers(-10, 11, size=(K // 128, M))
    eb = rng.integers(-10, 11, size=(K // 128, N))
    sa = np.ldexp(np.float32(1), ea).astype(np.float32)
    sb = np.ldexp(np.float32(1), eb).astype(np.float32)
    got, _ = oracle.k_grouped_tn(A, sa, B, sb, ks)
    k0 = 0
    for g, kg in enumerate(ks):
        want = np.zeros((M, N))
        for kb in range(k0 // 128, (k0 + kg) // 128):
            want += 128.0 * np.ldexp(1.0, ea[kb][:, None] + eb[kb][None, :])
        assert np.array_equal(got[g], want.astype(np.float32)), g
        k0 += kg


def test_group_ignores_other_groups_rows_and_empty_group_is_zero():
    c = synth.k_grouped_case([130, 0, 200], 24, 20, seed=4)
    A, sa, B, sb = _host(c)
    ks = c["ks"]
    ref, _ = oracle.k_grouped_tn(A, sa, B, sb, ks)
    A2, B2 = A.copy(), B.copy()
    A2[:ks[0]] = np.random.default_rng(0).integers(0, 0x7E, size=A2[:ks[0]].shape)  # group 0's rows
    B2[:ks[0]] ^= 0x80
    got, _ = oracle.k_grouped_tn(A2, sa, B2, sb, ks)
    assert np.array_equal(got[1:], ref[1:])
    assert not np.array_equal(got[0], ref[0])
    assert np.all(ref[1] == 0.0)


def test_two_groups_sum_to_one_group_exactly():
    """With the small-integer kind every FP32 sum is exact, so splitting one segment
    into two groups and adding their results gives the one-group result bit for bit."""
    c = synth.k_grouped_case([384], 32, 48, seed=9, kind="e1")
    A, sa, B, sb = _host(c)
    one, _ = oracle.k_grouped_tn(A, sa, B, sb, [384])
    two, _ = oracle.k_grouped_tn(A, sa, B, sb, [128, 256])
    assert np.array_equal(two[0] + two[1], one[0])


def test_accumulate_into_old_d():
    c = synth.k_grouped_case([256, 128], 16, 16, seed=3, kind="e1")
    A, sa, B, sb = _host(c)
    ks = c["ks"]
    plain, _ = oracle.k_grouped_tn(A, sa, B, sb, ks)
    again, T = oracle.k_grouped_tn(A, sa, B, sb, ks, D_in=-plain)   # exact: cancels
    assert np.all(T == 0.0) and np.all(again == 0.0)
    twice, _ = oracle.k_grouped_tn(A, sa, B, sb, ks, D_in=plain)
    assert np.array_equal(twice, 2 * plain)


def test_row_and_column_subsets():
    c = synth.k_grouped_case([200, 60], 50, 70, seed=6)
    A, sa, B, sb = _host(c)
    full, _ = oracle.k_grouped_tn(A, sa, B, sb, c["ks"])
    rows, cols = np.array([0, 7, 49]), np.array([1, 64, 69])
    sub, _ = oracle.k_grouped_tn(A, sa, B, sb, c["ks"], rows=rows, cols=cols)
    assert np.array_equal(sub, full[:, rows][:, :, cols])


def test_generator_layout():
    c = synth.k_grouped_case([1, 129], 20, 8, seed=2, lda=32)
    assert c["ks"] == [128, 256] and c["K"] == 384
    assert c["A"].shape == (384, 32) and c["sa"].shape == (3, 20)
    A = c["A"].numpy()
    assert np.all(A[1:128, :20] == 0) and np.all(A[128 + 129:, :20] == 0)   # zero padding tokens
