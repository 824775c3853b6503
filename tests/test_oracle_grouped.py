"""Pins of the oracle's grouped variants against its dense form and the layout rules:
contiguous rows with m_indices = -1 and masked rows at or beyond masked_m[g] keep the
sentinel, and every live row equals a dense GEMM with its group's weights."""
import numpy as np
import torch

import oracle
import synth

SENT = synth.SENTINEL_BITS


def _np(c, *keys):
    return [c[k].numpy() if hasattr(c[k], "numpy") else c[k] for k in keys]


def _d_bits(c):
    return c["D"].view(torch.int16).numpy().view(np.uint16)


def test_contiguous_equals_per_group_dense_and_keeps_padding():
    c = synth.contiguous_case([5, 128, 0, 130, 1], 200, 256, seed=21)
    A, sa, B, sb, mi = _np(c, "A", "sa", "B", "sb", "m_indices")
    D0 = _d_bits(c)
    D, S = oracle.grouped_contiguous(A, sa, B, sb, mi, D0)
    assert D.shape == D0.shape
    pad = mi < 0
    assert pad.sum() > 0
    assert np.all(D[pad] == SENT) and np.all(np.isnan(S[pad]))
    for g, (start, rows) in enumerate(c["segments"]):
        if rows == 0:
            continue
        seg = slice(start, start + rows)
        assert np.all(mi[seg] == g)
        ref, _ = oracle.gemm_nt(A[seg], sa[:, seg], B[g], sb[g])
        assert np.array_equal(D[seg], ref)
    # the padding rows hold random bytes including NaN codes: they stay isolated
    assert np.any((A[pad] == 0x7F) | (A[pad] == 0xFF))
    assert not np.any(np.isnan(S[~pad]))


def test_contiguous_sampled_rows_match_full():
    c = synth.contiguous_case([40, 200], 96, 128, seed=22)
    A, sa, B, sb, mi = _np(c, "A", "sa", "B", "sb", "m_indices")
    D0 = _d_bits(c)
    D, _ = oracle.grouped_contiguous(A, sa, B, sb, mi, D0)
    rows, cols = np.array([0, 39, 40, 127, 128, 300, 383]), np.array([0, 95])
    Ds, _ = oracle.grouped_contiguous(A, sa, B, sb, mi, D0, rows, cols)
    assert np.array_equal(Ds, D[np.ix_(rows, cols)])


def test_masked_live_rows_equal_dense_dead_rows_untouched():
    c = synth.masked_case(4, 256, 160, 256, seed=23, masked_m=[256, 0, 1, 179])
    A, sa, B, sb = _np(c, "A", "sa", "B", "sb")
    mm = c["masked_m_list"]
    D0 = _d_bits(c)
    D, S = oracle.grouped_masked(A, sa, B, sb, mm, D0)
    for g in range(4):
        live = mm[g]
        assert np.all(D[g, live:] == SENT)
        assert np.all(np.isnan(S[g, live:]))
        if live:
            ref, _ = oracle.gemm_nt(A[g, :live], sa[g][:, :live], B[g], sb[g])
            assert np.array_equal(D[g, :live], ref)
    # group 0 is fully live: identical to the dense GEMM of the whole group
    ref0, _ = oracle.gemm_nt(A[0], sa[0], B[0], sb[0])
    assert np.array_equal(D[0], ref0)
    assert np.any((A[3, 179:] == 0x7F) | (A[3, 179:] == 0xFF))


def test_masked_sampled_rows_match_full():
    c = synth.masked_case(2, 128, 64, 128, seed=24, masked_m=[100, 7])
    A, sa, B, sb = _np(c, "A", "sa", "B", "sb")
    D0 = _d_bits(c)
    D, _ = oracle.grouped_masked(A, sa, B, sb, c["masked_m_list"], D0)
    rows, cols = np.array([0, 6, 7, 99, 100, 127]), np.array([1, 63])
    Ds, _ = oracle.grouped_masked(A, sa, B, sb, c["masked_m_list"], D0, rows, cols)
    assert np.array_equal(Ds, D[:, rows][:, :, cols])


def test_moe_routing_layout():
    expert_of, counts = synth.moe_routing(tokens=4096, experts=256, topk=8, zipf_s=1.1, seed=0)
    assert expert_of.shape == (4096, 8)
    srt = expert_of.sort(dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all()), "experts per token must be distinct"
    assert sum(counts) == 4096 * 8
    mi, tok = synth.moe_contiguous_rows(expert_of, 256)
    assert mi.numel() % 128 == 0 and mi.numel() >= 32768
    assert int((mi >= 0).sum()) == 32768
    # Zipf skew: the most popular expert gets far more than the mean of 128 rows
    assert max(counts) > 1000 and min(counts) < 128
    # every 128-row block holds one expert plus -1 tail padding
    blocks = mi.view(-1, 128)
    for b in blocks:
        live = b[b >= 0]
        assert live.numel() > 0 and bool((live == live[0]).all())
        assert bool((b[:live.numel()] >= 0).all())
