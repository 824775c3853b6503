"""GPU parity of the dense FP8 NT GEMM (fp8_gemm_nt through the C ABI) against the
CPU oracle: every compiled tile shape and split-K factor on small shapes, ragged
edges, bit-exact integer cases, and the full-size DeepSeek-V3-like shape list on
sampled outputs."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import SENT, assert_bit_exact, bits_of, compare, forced_workspace_bytes, host, sample_rows

pytestmark = pytest.mark.gpu

TILES = [(64, 64, 1), (128, 64, 1), (64, 128, 1), (128, 128, 1), (256, 128, 1), (128, 256, 1), (64, 96, 1),
         (128, 96, 1), (64, 64, 2), (128, 64, 3), (128, 128, 4), (256, 128, 2), (128, 256, 3), (64, 96, 2),
         (128, 96, 3)]
CONFIG2_NK = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048)]
COUNTER_BYTES = 16384  # the workspace's leading block of split-K arrival counters


def run_dense(c, forced=None, ws=True):
    D = c["D"].clone()
    M, N, K = c["M"], c["N"], c["K"]
    work = None
    if ws:
        nbytes = fg.workspace_size(fg.KIND_DENSE, M, N, K)
        if forced is not None and forced[2] > 1:
            nbytes = forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, forced)
        work = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=D.device)
    if forced is None:
        fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
    else:
        with fg.force_config(*forced):
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
    torch.cuda.synchronize()
    return D, work


@pytest.mark.parametrize("kind", ["normal", "e1", "e2", "e3"])
@pytest.mark.parametrize("tile", TILES, ids=lambda t: "%dx%d_s%d" % t)
def test_config1_every_tile(cuda_device, kind, tile):
    c = synth.dense_case(128, 256, 512, seed=1000 + 1, device=cuda_device, kind=kind)
    D, _ = run_dense(c, forced=tile)
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    compare(kind, bits_of(D), ref, f"config1 {kind} {tile}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (63, 130, 256), (65, 200, 384), (200, 2112, 512),
                                   (129, 96, 1024), (257, 320, 640), (17, 16, 128), (300, 1000, 1280)])
@pytest.mark.parametrize("kind", ["normal", "e1"])
def test_ragged_shapes_auto_and_forced(cuda_device, M, N, K, kind):
    c = synth.dense_case(M, N, K, seed=7 * M + N + K, device=cuda_device, kind=kind)
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    D, _ = run_dense(c)
    compare(kind, bits_of(D), ref, f"auto {M}x{N}x{K}")
    for tile in [(64, 64, 1), (128, 128, 2), (64, 128, 3), (256, 128, 1), (128, 256, 2), (64, 96, 1), (128, 96, 2)]:
        D, _ = run_dense(c, forced=tile)
        compare(kind, bits_of(D), ref, f"{tile} {M}x{N}x{K}")


def test_split_k_is_deterministic_and_workspace_self_resets(cuda_device):
    c = synth.dense_case(64, 2112, 7168, seed=31, device=cuda_device)
    ws_n = fg.workspace_size(fg.KIND_DENSE, 64, 2112, 7168)
    assert ws_n > 0
    work = torch.zeros(ws_n, dtype=torch.uint8, device=cuda_device)
    outs = []
    for _ in range(3):
        D = c["D"].clone()
        fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
        torch.cuda.synchronize()
        outs.append(bits_of(D))
        assert int(work[:COUNTER_BYTES].count_nonzero()) == 0, "split-K counters must be left at zero"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # without a workspace the call runs unsplit and agrees within tolerance
    D = c["D"].clone()
    fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, None)
    torch.cuda.synchronize()
    rows = sample_rows(64, 16, 3)
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(2112))
    compare("normal", bits_of(D)[rows], ref, "unsplit")
    compare("normal", outs[0][rows], ref, "split")


@pytest.mark.parametrize("order", [0, 1])
def test_one_workspace_shared_by_different_split_plans(cuda_device, order):
    """Shapes whose plans differ (tile, split count and number of split tiles) run one
    after the other through one workspace, in both orders, twice, with a TN-layout call
    (its own tiles and split) among them: the counters sit at a fixed place, so no call
    sees another's partials as counters."""
    shapes = [(64, 2112, 7168), (64, 4096, 7168), (128, 2112, 7168), (64, 7168, 2048)]
    kinds = [fg.KIND_DENSE, fg.KIND_DENSE, fg.KIND_DENSE, fg.KIND_LAYOUT]
    if order:
        shapes, kinds = shapes[::-1], kinds[::-1]
    plans = [fg.query_config(k, *s) for k, s in zip(kinds, shapes)]
    assert all(p["split_k"] > 1 for p in plans), plans
    assert len({(p["block_m"], p["block_n"], p["split_k"], p["num_units"]) for p in plans}) == len(plans)
    nbytes = max(fg.workspace_size(k, *s) for k, s in zip(kinds, shapes))
    work = torch.zeros(nbytes, dtype=torch.uint8, device=cuda_device)
    cases = [synth.dense_case(M, N, K, seed=4100 + i, device=cuda_device, a_std=1.0, b_std=0.02)
             for i, (M, N, K) in enumerate(shapes)]
    refs = []
    for (M, N, K), c in zip(shapes, cases):
        rows = sample_rows(M, 10, N + K)
        refs.append((rows, oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))[0]))
    for rep in range(2):
        for (M, N, K), kind, c, (rows, ref) in zip(shapes, kinds, cases, refs):
            D = c["D"].clone()
            if kind == fg.KIND_LAYOUT:   # the same product with both operands stored K-major
                At = c["A"].t().contiguous()
                Bt = torch.zeros(K, (N + 15) // 16 * 16, dtype=torch.uint8, device=cuda_device)
                Bt[:, :N] = c["B"].t()
                fg.fp8_gemm_tn(At, c["sa"], Bt, c["sb"], D, workspace=work)
            else:
                fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
            torch.cuda.synchronize()
            bits = bits_of(D)
            assert not np.any(bits == SENT), f"{M}x{N}x{K} pass {rep}: an output tile was not written"
            compare("normal", bits[rows], ref, f"shared workspace {M}x{N}x{K} pass {rep}")
            assert int(work[:COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("M", [64, 128, 4096])
@pytest.mark.parametrize("N,K", CONFIG2_NK)
def test_config2_full_size_sampled(cuda_device, M, N, K):
    c = synth.dense_case(M, N, K, seed=2000 + M + N + K, device=cuda_device, a_std=1.0, b_std=0.02)
    D, _ = run_dense(c)
    bits = bits_of(D)
    assert not np.any(bits == SENT), "every output must be written"
    rows = sample_rows(M, 12, M + N)
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))
    compare("normal", bits[rows], ref, f"config2 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (128, 7168, 2048), (4096, 4096, 7168), (4096, 32768, 512)])
def test_config2_exact_case_full_size_sampled(cuda_device, M, N, K):
    c = synth.dense_case(M, N, K, seed=3000 + M + N, device=cuda_device, kind="e1")
    D, _ = run_dense(c)
    rows = sample_rows(M, 8, K)
    cols = np.unique(np.concatenate([np.arange(0, N, 7), [N - 1]]))
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, cols)
    assert_bit_exact(bits_of(D)[np.ix_(rows, cols)], ref, f"e1 M={M} N={N} K={K}")


def test_strided_operands(cuda_device):
    # leading dimensions larger than the logical sizes
    M, N, K = 96, 192, 384
    c = synth.dense_case(M, N, K, seed=77, device=cuda_device)
    A = torch.zeros(M, K + 128, dtype=torch.uint8, device=cuda_device)
    A[:, :K] = c["A"]
    B = torch.zeros(N, K + 256, dtype=torch.uint8, device=cuda_device)
    B[:, :K] = c["B"]
    sa = torch.zeros(K // 128, 128, dtype=torch.float32, device=cuda_device)
    sa[:, :c["sa"].shape[1]] = c["sa"]
    Dbig = synth.sentinel_output((M, N + 64), cuda_device)
    fg.fp8_gemm_nt(A[:, :K], sa, B[:, :K], c["sb"], Dbig[:, :N])
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    compare("normal", bits_of(Dbig)[:, :N], ref, "strided")
    assert np.all(bits_of(Dbig)[:, N:] == SENT), "columns beyond N must not be written"


@pytest.mark.parametrize("col0,pitch_mod8", [(0, 4), (4, 0), (1, 0), (2, 3), (0, 0)],
                         ids=["ldd%8=4", "D+8B", "D+2B", "odd_ldd", "aligned"])
@pytest.mark.parametrize("N", [192, 252])
def test_output_alignment_and_pitch(cuda_device, col0, pitch_mod8, N):
    # D rows of every alignment the store widths distinguish (16-, 8- and 2-byte), with
    # column edges inside a tile (N=252); cells around the output keep the sentinel
    M, K = 80, 384
    c = synth.dense_case(M, N, K, seed=91 + col0 + N, device=cuda_device)
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    pitch = (N + col0 + 15) // 8 * 8 + pitch_mod8
    for tile in (None, (64, 64, 1), (128, 128, 1), (256, 128, 1), (128, 256, 1)):
        big = synth.sentinel_output((M + 1, pitch), cuda_device)
        D = big[:M, col0:col0 + N]
        if tile is None:
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D)
        else:
            with fg.force_config(*tile):
                fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D)
        torch.cuda.synchronize()
        out = bits_of(big)
        compare("normal", out[:M, col0:col0 + N], ref, f"pitch {pitch} col0 {col0} N {N} {tile}")
        keep = np.ones(out.shape, dtype=bool)
        keep[:M, col0:col0 + N] = False
        assert np.all(out[keep] == SENT), f"cells outside D written: {tile}"


@pytest.mark.parametrize("tile,full", [((64, 64, 3), 50), ((128, 128, 2), 5), ((256, 128, 4), 3), ((128, 256, 2), 1),
                                       ((64, 128, 8), 31), ((128, 64, 5), 0)])
def test_whole_tiles_then_split_tiles(cuda_device, tile, full):
    # the first `full` tiles of the work order computed whole, the others as split-K
    # units: every element equals the unsplit or the all-split result of the same
    # tile shape, and matches the oracle; two calls share one workspace (the arrival
    # counters reset themselves)
    M, N, K = 300, 1000, 1280
    c = synth.dense_case(M, N, K, seed=5150 + full, device=cuda_device)
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    whole, _ = run_dense(c, forced=(tile[0], tile[1], 1))
    split_all, _ = run_dense(c, forced=tile)
    tiles = fg.num_tiles(M, N, tile[0], tile[1])
    ws = torch.zeros(forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, tile, full), dtype=torch.uint8,
                     device=cuda_device)
    for rep in range(2):
        D = synth.sentinel_output((M, N), cuda_device)
        with fg.force_config(*tile, full_tiles=full):
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, ws)
        torch.cuda.synchronize()
        got = bits_of(D)
        compare("normal", got, ref, f"{tile} full {full} call {rep}")
        assert np.all((got == bits_of(whole)) | (got == bits_of(split_all))), f"{tile} full {full}"
        if 0 < full < tiles:
            assert np.any(got != bits_of(split_all)) and np.any(got != bits_of(whole)), "both kinds of unit ran"
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0 if full < tiles else True


@pytest.mark.parametrize("M,N,K,tile", [(64, 2112, 7168, None), (128, 4096, 7168, None), (100, 384, 2048, (64, 64, 8)),
                                        (256, 640, 4096, (128, 128, 5))])
def test_split_k_workspace_reuse_with_new_inputs(cuda_device, M, N, K, tile):
    # a reduction that read a partial left from the previous call would pass a
    # same-input determinism test; here every call has different operands
    nbytes = fg.workspace_size(fg.KIND_DENSE, M, N, K)
    if tile is not None:
        nbytes = forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, tile)
    work = torch.zeros(nbytes, dtype=torch.uint8, device=cuda_device)
    rows = sample_rows(M, 10, K)
    for call in range(3):
        c = synth.dense_case(M, N, K, seed=600 + call, device=cuda_device, kind="e1" if call == 1 else "normal")
        D = c["D"].clone()
        if tile is None:
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
        else:
            with fg.force_config(*tile):
                fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, work)
        torch.cuda.synchronize()
        ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))
        compare("e1" if call == 1 else "normal", bits_of(D)[rows], ref, f"call {call} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 384), (1000, 1000, 640), (512, 768, 128), (768, 512, 256),
                                   (4096, 2048, 1536)])
@pytest.mark.parametrize("kind", ["normal", "e1"])
def test_many_tiles_per_workgroup(cuda_device, M, N, K, kind):
    # a small grid (8 CUs) makes every workgroup run many whole tiles in a row, so each
    # tile's first stages are loaded before the previous tile's epilogue; full and
    # ragged (edge) tiles alternate, and K covers one to twelve 128-wide blocks
    c = synth.dense_case(M, N, K, seed=8100 + M + N + K, device=cuda_device, kind=kind)
    rows = sample_rows(M, 48, K) if M * N > 2_000_000 else np.arange(M)
    ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))
    fg.set_num_cus(8)
    try:
        for tile in [(256, 128, 1), (128, 256, 1), None]:
            D, _ = run_dense(c, forced=tile)
            got = bits_of(D)
            assert not np.any(got == SENT), f"every output written {tile}"
            compare(kind, got[rows], ref, f"8 CUs {tile} {M}x{N}x{K} {kind}")
    finally:
        fg.set_num_cus(0)
