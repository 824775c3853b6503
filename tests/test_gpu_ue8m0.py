"""GPU parity of the UE8M0 dense GEMM (fp8_gemm_nt_ue8m0: power-of-two scales through
gfx950's block-scaled MFMA) against the CPU oracle: every tile shape and split-K factor
on small and ragged shapes with exact integer cases bit for bit, power-of-two-quantised
N(0,1) / N(0,0.02) operands within tolerance, and full DeepSeek-V3-like shapes on
sampled outputs."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import SENT, assert_bit_exact, bits_of, compare, forced_workspace_bytes, host, sample_rows

pytestmark = pytest.mark.gpu

TILES = [None, (64, 64, 1), (128, 64, 1), (64, 128, 1), (128, 128, 1), (256, 128, 1), (128, 256, 1), (64, 96, 1),
         (64, 64, 3), (128, 128, 2), (256, 128, 2), (128, 256, 3), (128, 96, 2)]


def run(c, tile=None):
    D = c["D"].clone()
    M, N, K = c["M"], c["N"], c["K"]
    nbytes = fg.workspace_size(fg.KIND_DENSE, M, N, K)
    if tile is not None and tile[2] > 1:
        nbytes = forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, tile)
    work = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=D.device)
    if tile is None:
        fg.fp8_gemm_nt_ue8m0(c["A"], c["sa"], c["B"], c["sb"], D, work)
    else:
        with fg.force_config(*tile):
            fg.fp8_gemm_nt_ue8m0(c["A"], c["sa"], c["B"], c["sb"], D, work)
    torch.cuda.synchronize()
    return bits_of(D)


@pytest.mark.parametrize("kind", ["pow2", "e1", "e2", "e3"])
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 64, 128), (65, 200, 384), (300, 1000, 1280)])
def test_every_tile_against_the_oracle(cuda_device, kind, M, N, K):
    c = synth.dense_case(M, N, K, seed=9000 + M + N + K, device=cuda_device, kind=kind)
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    cmp_kind = "normal" if kind == "pow2" else kind
    for tile in TILES:
        got = run(c, tile)
        compare(cmp_kind, got, ref, f"ue8m0 {kind} {M}x{N}x{K} {tile}")


def test_agrees_with_the_fp32_scale_path(cuda_device):
    # the same power-of-two scales given to fp8_gemm_nt (promotion by FP32 FMAs) and to
    # the block-scaled MFMA: both within the bar of the oracle, and close to each other
    M, N, K = 512, 768, 2048
    c = synth.dense_case(M, N, K, seed=9100, device=cuda_device, kind="pow2")
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    e8 = run(c)
    D = c["D"].clone()
    fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, fg.make_workspace(fg.KIND_DENSE, M, N, K, device=cuda_device))
    torch.cuda.synchronize()
    f32 = bits_of(D)
    compare("normal", e8, ref, "ue8m0")
    compare("normal", f32, ref, "fp32 scales")
    g = oracle.bf16_bits_to_f64(e8)
    h = oracle.bf16_bits_to_f64(f32)
    assert np.all(np.abs(g - h) <= 2.0 ** -7 * np.abs(h) + 1e-12), "paths differ by more than one BF16 ulp"


@pytest.mark.parametrize("M,N,K", [(4096, 7168, 16384), (64, 2112, 7168), (4096, 32768, 512)])
def test_full_size_sampled(cuda_device, M, N, K):
    c = synth.dense_case(M, N, K, seed=9200 + M + N, device=cuda_device, kind="pow2", a_std=1.0, b_std=0.02)
    got = run(c)
    assert not np.any(got == SENT), "every output must be written"
    rows = sample_rows(M, 10, K)
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))
    compare("normal", got[rows], ref, f"ue8m0 full {M}x{N}x{K}")


def test_exact_case_full_size_sampled(cuda_device):
    M, N, K = 4096, 4096, 7168
    c = synth.dense_case(M, N, K, seed=9300, device=cuda_device, kind="e1")
    got = run(c)
    rows = sample_rows(M, 8, K)
    cols = np.unique(np.concatenate([np.arange(0, N, 7), [N - 1]]))
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, cols)
    assert_bit_exact(got[np.ix_(rows, cols)], ref, "ue8m0 e1 4096x4096x7168")


def _contig(c, tile, ue8m0=True):
    D = c["D"].clone()
    M, N, K, G = c["M"], c["N"], c["K"], c["G"]
    nbytes = fg.workspace_size(fg.KIND_CONTIGUOUS, M, N, K, G)
    if tile is not None and tile[2] > 1:
        nbytes = forced_workspace_bytes(fg.KIND_CONTIGUOUS, M, N, K, G, tile)
    work = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=D.device)
    args = (c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"], work)
    if tile is None:
        fg.fp8_grouped_gemm_nt_contiguous(*args, ue8m0=ue8m0)
    else:
        with fg.force_config(*tile):
            fg.fp8_grouped_gemm_nt_contiguous(*args, ue8m0=ue8m0)
    torch.cuda.synchronize()
    return bits_of(D)


def _masked(c, tile, ue8m0=True):
    D = c["D"].clone()
    args = (c["A"], c["sa"], c["B"], c["sb"], D, c["masked_m"], c["expected_m"])
    if tile is None:
        fg.fp8_grouped_gemm_nt_masked(*args, ue8m0=ue8m0)
    else:
        with fg.force_config(*tile):
            fg.fp8_grouped_gemm_nt_masked(*args, ue8m0=ue8m0)
    torch.cuda.synchronize()
    return bits_of(D)


@pytest.mark.parametrize("kind", ["pow2", "e1", "e3"])
def test_contiguous_every_tile(cuda_device, kind):
    c = synth.contiguous_case([5, 128, 0, 130, 1, 300], 200, 384, seed=43, device=cuda_device, kind=kind)
    ref, _ = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), bits_of(c["D"]))
    pad = c["m_indices"].cpu().numpy() < 0
    for tile in (None, (64, 64, 1), (128, 128, 1), (64, 128, 1), (128, 256, 1), (64, 64, 2), (128, 256, 2)):
        got = _contig(c, tile)
        assert np.all(got[pad] == SENT), f"padding rows written {tile}"
        compare("normal" if kind == "pow2" else kind, got[~pad], ref[~pad], f"contiguous ue8m0 {kind} {tile}")


@pytest.mark.parametrize("kind", ["pow2", "e1", "e2"])
def test_masked_every_tile(cuda_device, kind):
    c = synth.masked_case(5, 256, 160, 384, seed=53, device=cuda_device, masked_m=[256, 0, 1, 179, 64],
                          kind=kind, expected_m=128)
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), c["masked_m_list"], bits_of(c["D"]))
    for tile in (None, (64, 64, 1), (64, 128, 1), (128, 128, 1), (256, 128, 1), (128, 256, 1)):
        got = _masked(c, tile)
        for g, live in enumerate(c["masked_m_list"]):
            assert np.all(got[g, live:] == SENT), f"dead rows of group {g} written {tile}"
            compare("normal" if kind == "pow2" else kind, got[g, :live], ref[g, :live],
                    f"masked ue8m0 {kind} {tile} group {g}")


def test_grouped_full_size_sampled(cuda_device):
    # the second contiguous configuration and a masked decode case at full size
    c = synth.contiguous_case([4096] * 8, 7168, 2048, seed=9400, device=cuda_device, kind="pow2")
    got = _contig(c, None)
    assert not np.any(got == SENT)
    rs = np.unique(np.concatenate([g * 4096 + sample_rows(4096, 2, g) for g in range(8)]))
    ref, _ = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), bits_of(c["D"]), rs,
                                       np.arange(7168))
    compare("normal", got[rs], ref, "contiguous ue8m0 8x4096 N=7168 K=2048")
    del c, got
    m = synth.masked_case(4, 4096, 4096, 7168, seed=9401, device=cuda_device, kind="pow2", expected_m=256)
    got = _masked(m, None)
    mm = m["masked_m_list"]
    rows = [0, 1, 100, 178]
    ref, _ = oracle.grouped_masked(*host(m, "A", "sa", "B", "sb"), mm, bits_of(m["D"]), rows, np.arange(4096))
    compare("normal", got[:, rows], ref, "masked ue8m0 G=4 N=4096 K=7168")
    for g, live in enumerate(mm):
        assert np.all(got[g, live:] == SENT)
