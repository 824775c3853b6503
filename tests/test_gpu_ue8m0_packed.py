"""GPU parity of the packed-UE8M0 calls (fp8_gemm_nt_ue8m0_packed and the grouped forms)
and of the scale-layout transform (fp8_transform_sf_into_required_layout) against the CPU
oracle: bit-exact on the integer cases (e1, e3: power-of-two scales, exact sums), within
the bar on N(0,1) data with power-of-two scales, bitwise equal to the FP32-power-of-two
UE8M0 calls, with K block counts that leave a partial last word and K slices that start
inside a word."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import SENT, assert_bit_exact, bits_of, compare, forced_workspace_bytes, host, sample_rows

pytestmark = pytest.mark.gpu


def packed(c):
    return synth.pack_ue8m0(c["sa"], axis=0), synth.pack_ue8m0(c["sb"], axis=c["sb"].dim() - 1)


def run_dense(c, tile=None):
    M, N, K = c["M"], c["N"], c["K"]
    sa_w, sb_w = packed(c)
    D = c["D"].clone()
    if tile is None:
        fg.fp8_gemm_nt_ue8m0_packed(c["A"], sa_w, c["B"], sb_w, D, fg.make_workspace(fg.KIND_DENSE, M, N, K,
                                                                                      device=D.device))
    else:
        ws = torch.zeros(forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, tile), dtype=torch.uint8, device=D.device)
        with fg.force_config(*tile):
            fg.fp8_gemm_nt_ue8m0_packed(c["A"], sa_w, c["B"], sb_w, D, ws)
    torch.cuda.synchronize()
    return D, sa_w, sb_w


TILES = [None, (64, 64, 1), (64, 64, 3), (128, 128, 2), (128, 64, 5), (256, 128, 1), (128, 256, 3), (64, 96, 2)]


@pytest.mark.parametrize("kind", ["e1", "e3", "pow2"])
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (96, 384, 640), (200, 300, 1152), (64, 130, 384)])
@pytest.mark.parametrize("tile", TILES, ids=lambda t: "auto" if t is None else "%dx%d_s%d" % t)
def test_dense_packed_against_oracle(cuda_device, kind, M, N, K, tile):
    c = synth.dense_case(M, N, K, seed=8000 + M + N + K, device=cuda_device, kind=kind)
    D, sa_w, sb_w = run_dense(c, tile)
    ref, _ = oracle.gemm_nt_ue8m0_packed(c["A"].cpu().numpy(), sa_w.cpu().numpy(), c["B"].cpu().numpy(),
                                         sb_w.cpu().numpy(), K)
    compare("e1" if kind != "pow2" else "normal", bits_of(D), ref, f"packed {kind} {M}x{N}x{K} {tile}")
    # the same codes as FP32 powers of two through fp8_gemm_nt_ue8m0: the same bits
    D2 = c["D"].clone()
    if tile is None:
        fg.fp8_gemm_nt_ue8m0(c["A"], c["sa"], c["B"], c["sb"], D2, fg.make_workspace(fg.KIND_DENSE, M, N, K,
                                                                                      device=cuda_device))
    else:
        ws = torch.zeros(forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, tile), dtype=torch.uint8, device=cuda_device)
        with fg.force_config(*tile):
            fg.fp8_gemm_nt_ue8m0(c["A"], c["sa"], c["B"], c["sb"], D2, ws)
    torch.cuda.synchronize()
    assert_bit_exact(bits_of(D), bits_of(D2), "packed vs FP32 power-of-two scales")


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (4096, 4096, 7168), (128, 7168, 2048)])
def test_dense_packed_full_size_sampled(cuda_device, M, N, K):
    c = synth.dense_case(M, N, K, seed=8100 + M, device=cuda_device, kind="pow2", a_std=1.0, b_std=0.02)
    D, sa_w, sb_w = run_dense(c)
    bits = bits_of(D)
    assert not np.any(bits == SENT)
    rows = sample_rows(M, 10, N)
    # the oracle on the sampled rows: unpack with the oracle's own code, then its dense GEMM
    nkb = K // 128
    ca = oracle.ue8m0_unpack(sa_w.cpu().numpy(), nkb, axis=0)
    cb = oracle.ue8m0_unpack(sb_w.cpu().numpy(), nkb, axis=1)
    ref, _ = oracle.gemm_nt_sampled(c["A"].cpu().numpy(), oracle.ue8m0_decode(ca), c["B"].cpu().numpy(),
                                    oracle.ue8m0_decode(cb), rows, np.arange(N))
    compare("normal", bits[rows], ref, f"packed full size {M}x{N}x{K}")


@pytest.mark.parametrize("kind", ["e1", "pow2"])
def test_contiguous_packed(cuda_device, kind):
    c = synth.contiguous_case([100, 0, 256, 37], 256, 640, seed=8200, device=cuda_device, kind=kind)
    sa_w = synth.pack_ue8m0(c["sa"], axis=0)
    sb_w = synth.pack_ue8m0(c["sb"], axis=2)
    D = c["D"].clone()
    fg.fp8_grouped_gemm_nt_contiguous_ue8m0_packed(c["A"], sa_w, c["B"], sb_w, D, c["m_indices"])
    torch.cuda.synchronize()
    mi = c["m_indices"].cpu().numpy()
    nkb = c["K"] // 128
    ca = oracle.ue8m0_decode(oracle.ue8m0_unpack(sa_w.cpu().numpy(), nkb, axis=0))
    cb = oracle.ue8m0_decode(oracle.ue8m0_unpack(sb_w.cpu().numpy(), nkb, axis=2))
    ref, _ = oracle.grouped_contiguous(c["A"].cpu().numpy(), ca, c["B"].cpu().numpy(), cb, mi, bits_of(c["D"]))
    got = bits_of(D)
    assert np.all(got[mi < 0] == SENT), "padding rows written"
    compare("e1" if kind == "e1" else "normal", got[mi >= 0], ref[mi >= 0], f"contiguous packed {kind}")


@pytest.mark.parametrize("kind", ["e1", "pow2"])
def test_masked_packed(cuda_device, kind):
    mm = [70, 0, 130, 256]
    c = synth.masked_case(4, 256, 384, 1152, seed=8300, device=cuda_device, masked_m=mm, expected_m=128, kind=kind)
    sa_w = synth.pack_ue8m0(c["sa"], axis=1)
    sb_w = synth.pack_ue8m0(c["sb"], axis=2)
    D = c["D"].clone()
    fg.fp8_grouped_gemm_nt_masked_ue8m0_packed(c["A"], sa_w, c["B"], sb_w, D, c["masked_m"], 128)
    torch.cuda.synchronize()
    nkb = c["K"] // 128
    ca = oracle.ue8m0_decode(oracle.ue8m0_unpack(sa_w.cpu().numpy(), nkb, axis=1))
    cb = oracle.ue8m0_decode(oracle.ue8m0_unpack(sb_w.cpu().numpy(), nkb, axis=2))
    ref, _ = oracle.grouped_masked(c["A"].cpu().numpy(), ca, c["B"].cpu().numpy(), cb, mm, bits_of(c["D"]))
    got = bits_of(D)
    for g, live in enumerate(mm):
        assert np.all(got[g, live:] == SENT), f"dead rows of group {g} written"
        compare("e1" if kind == "e1" else "normal", got[g, :live], ref[g, :live], f"masked packed {kind} group {g}")


@pytest.mark.parametrize("is_activation", [True, False])
@pytest.mark.parametrize("pack", [True, False])
@pytest.mark.parametrize("rows,nkb", [(300, 9), (17, 56), (1, 1), (64, 4)])
def test_transform_matches_oracle(cuda_device, is_activation, pack, rows, nkb):
    gen = synth.make_generator(8400 + rows + nkb, cuda_device)
    e = torch.randint(-60, 60, (rows, nkb), generator=gen, device=cuda_device).float()
    frac = torch.where(torch.rand(rows, nkb, generator=gen, device=cuda_device) < 0.3,
                       1.0 + torch.rand(rows, nkb, generator=gen, device=cuda_device), torch.ones(rows, nkb,
                                                                                                  device=cuda_device))
    sf = (frac * torch.exp2(e)).float()       # powers of two and values between them
    ld = rows + 12 if is_activation else None
    if is_activation:
        ld = (ld + 3) // 4 * 4
    cols = (nkb + 3) // 4 if pack else nkb
    dt = torch.int32 if pack else torch.float32
    shape = (cols, ld) if is_activation else (rows, cols + 5)
    out = torch.full(shape, -7, dtype=torch.int32, device=cuda_device).view(dt)
    fg.transform_sf_into_required_layout(sf, is_activation, pack, out=out)
    torch.cuda.synchronize()
    want = oracle.transform_sf(sf.cpu().numpy(), is_activation, pack)
    got = out.cpu().numpy()
    gi = got.view(np.int32)
    if is_activation:
        assert np.array_equal(gi[:, :rows], want.view(np.int32))
        assert np.all(gi[:, rows:] == -7), "entries past the rows must be untouched"
    else:
        assert np.array_equal(gi[:, :cols], want.view(np.int32))
        assert np.all(gi[:, cols:] == -7)
