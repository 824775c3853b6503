"""GPU parity of the dense TN, NN and TT layouts (fp8_gemm_tn: D = A^T B, A [K, M], B [K, N];
fp8_gemm_nn: A [M, K], B [K, N]; fp8_gemm_tt: A [K, M], B [N, K]) against the CPU oracle
(oracle.gemm_tn / gemm_nn / gemm_tt): every tile instance, ragged M / N tails with padded
leading dimensions, exact integer cases bit for bit (the library's bar otherwise), a
strided and 2-byte-aligned D, and the dominant dense shape on sampled rows."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import bits_of, compare, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["128x128", "128x128-2stage", "256x256", "64x128", "128x64"])
def tile(request):
    """The instances: 128x128 tiles with the 4-stage ring (a plan whose units all fit one
    round), 128x128 with the 2-stage ring (more units than CUs), 256x256, and the 6-stage
    64x128 and 128x64 tiles (64-wide panels of A, of B)."""
    if request.param == "128x128":
        fg.set_num_cus(1 << 20)
        yield request.param
    else:
        fg.set_num_cus(1)
        if request.param == "256x256":
            yield request.param
        else:
            bm, bn = (128, 128) if request.param == "128x128-2stage" else (int(x) for x in request.param.split("x"))
            with fg.force_config(bm, bn, 1):
                yield request.param
    fg.set_num_cus(0)


def tn_case(M, N, K, seed, device, kind, lda=None, ldb=None):
    """The NT case's operands stored K-major (A^T [K, lda], B^T [K, ldb])."""
    c = synth.dense_case(M, N, K, seed=seed, device=device, kind=kind)
    lda, ldb = (M + 15) // 16 * 16 if lda is None else lda, (N + 15) // 16 * 16 if ldb is None else ldb
    At = torch.zeros(K, lda, dtype=torch.uint8, device=device)
    Bt = torch.zeros(K, ldb, dtype=torch.uint8, device=device)
    At[:, :M] = c["A"].t()
    Bt[:, :N] = c["B"].t()
    return c, At, Bt


def run(c, At, Bt, D=None):
    D = c["D"].clone() if D is None else D
    fg.fp8_gemm_tn(At, c["sa"], Bt, c["sb"], D)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("kind", ["normal", "e1", "e2", "e3"])
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (65, 200, 384), (300, 520, 1280), (1, 8, 128)])
def test_parity(cuda_device, tile, kind, M, N, K):
    c, At, Bt = tn_case(M, N, K, 4000 + M + N + K, cuda_device, kind)
    ref, _ = oracle.gemm_tn(At[:, :M].cpu().numpy(), c["sa"].cpu().numpy(), Bt[:, :N].cpu().numpy(),
                            c["sb"].cpu().numpy())
    compare(kind, bits_of(run(c, At, Bt)), ref, f"tn {tile} {kind} {M}x{N}x{K}")


def test_strided_d(cuda_device, tile):
    M, N, K = 136, 130, 256
    c, At, Bt = tn_case(M, N, K, 4100, cuda_device, "e1", lda=160, ldb=144)
    big = torch.full((M * 135 + 1,), float("nan"), dtype=torch.bfloat16, device=cuda_device)
    D = big[1:].view(M, 135)[:, :N]                        # ldd 135, 2-byte aligned only
    got = run(c, At, Bt, D)
    ref, _ = oracle.gemm_tn(At[:, :M].cpu().numpy(), c["sa"].cpu().numpy(), Bt[:, :N].cpu().numpy(),
                            c["sb"].cpu().numpy())
    compare("e1", bits_of(got.contiguous()), ref, "tn strided D")
    assert torch.all(torch.isnan(big[1:].view(M, 135)[:, N:]))


def test_dominant_shape_sampled(cuda_device):
    M, N, K = 4096, 7168, 16384
    c, At, Bt = tn_case(M, N, K, 4200, cuda_device, "normal")
    got = bits_of(run(c, At, Bt))
    rows = sample_rows(M, 24, 4201)
    A = At[:, :M].cpu().numpy()[:, rows]
    ref, _ = oracle.gemm_tn(A, c["sa"].cpu().numpy()[:, rows], Bt[:, :N].cpu().numpy(), c["sb"].cpu().numpy())
    compare("normal", got[rows], ref, "tn 4096x7168x16384 sampled rows")


def layout_operands(c, At, Bt, layout):
    """(A, B) for the call and the oracle function of a layout."""
    if layout == "nn":
        return c["A"], Bt, fg.fp8_gemm_nn
    return At, c["B"], fg.fp8_gemm_tt


@pytest.mark.parametrize("layout", ["nn", "tt"])
@pytest.mark.parametrize("kind", ["normal", "e1", "e2"])
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (65, 200, 384), (300, 520, 1280)])
def test_nn_tt_parity(cuda_device, tile, layout, kind, M, N, K):
    c, At, Bt = tn_case(M, N, K, 4300 + M + N + K, cuda_device, kind)
    A, B, fn = layout_operands(c, At, Bt, layout)
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    if layout == "nn":
        ref2, _ = oracle.gemm_nn(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), Bt[:, :N].cpu().numpy(),
                                 c["sb"].cpu().numpy())
    else:
        ref2, _ = oracle.gemm_tt(At[:, :M].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(),
                                 c["sb"].cpu().numpy())
    assert np.array_equal(ref, ref2)
    compare(kind, bits_of(D), ref2, f"{layout} {tile} {kind} {M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["nn", "tt"])
def test_nn_tt_dominant_shape_sampled(cuda_device, layout):
    M, N, K = 4096, 7168, 16384
    c, At, Bt = tn_case(M, N, K, 4400, cuda_device, "normal")
    A, B, fn = layout_operands(c, At, Bt, layout)
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D)
    torch.cuda.synchronize()
    rows = sample_rows(M, 24, 4401)
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy()[rows], c["sa"].cpu().numpy()[:, rows], c["B"].cpu().numpy(),
                            c["sb"].cpu().numpy())
    compare("normal", bits_of(D)[rows], ref, f"{layout} 4096x7168x16384 sampled rows")


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
def test_degenerate_shapes(cuda_device, layout):
    """M = 0 launches nothing; one K block and a single output row or column still match."""
    fns = {"tn": fg.fp8_gemm_tn, "nn": fg.fp8_gemm_nn, "tt": fg.fp8_gemm_tt}
    for M, N, K in [(1, 8, 128), (200, 1, 256)]:
        c, At, Bt = tn_case(M, N, K, 4500 + M + N, cuda_device, "e1")
        A = c["A"] if layout == "nn" else At
        B = c["B"] if layout == "tt" else Bt
        D = c["D"].clone()
        fns[layout](A, c["sa"], B, c["sb"], D)
        torch.cuda.synchronize()
        ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(),
                                c["sb"].cpu().numpy())
        compare("e1", bits_of(D), ref, f"{layout} {M}x{N}x{K}")
    # M = 0 through the C ABI (torch gives zero-element tensors a null pointer): a no-op
    import ctypes
    c, At, Bt = tn_case(16, 16, 128, 4600, cuda_device, "e1")
    A = c["A"] if layout == "nn" else At
    B = c["B"] if layout == "tt" else Bt
    D = c["D"].clone()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = getattr(fg.lib(), "fp8_gemm_" + layout)(P(A), A.stride(0), P(c["sa"]), c["sa"].stride(0), P(B), B.stride(0),
                                                 P(c["sb"]), P(D), D.stride(0), 0, 16, 128, None, 0,
                                                 ctypes.c_void_p(torch.cuda.current_stream(cuda_device).cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(D.view(torch.int16), c["D"].view(torch.int16))


# ---- UE8M0 (power-of-two) scales through fp8_gemm_{tn,nn,tt}_ue8m0: the oracle is the
# same layout definition on the same power-of-two FP32 scale values
@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("kind", ["pow2", "e1"])
@pytest.mark.parametrize("M,N,K", [(65, 200, 384), (300, 520, 1280)])
def test_ue8m0_parity(cuda_device, tile, layout, kind, M, N, K):
    c, At, Bt = tn_case(M, N, K, 4700 + M + N + K, cuda_device, kind)
    A = c["A"] if layout == "nn" else At
    B = c["B"] if layout == "tt" else Bt
    fn = {"tn": fg.fp8_gemm_tn, "nn": fg.fp8_gemm_nn, "tt": fg.fp8_gemm_tt}[layout]
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D, ue8m0=True)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    compare("e1" if kind == "e1" else "normal", bits_of(D), ref, f"{layout} ue8m0 {tile} {kind} {M}x{N}x{K}")


# ---- D = C + A B in the three layouts (fp8_gemm_{tn,nn,tt}_c): the oracle is the NT
# accumulate form on the same operands (the layout oracles equal the NT one, pinned)
@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("kind", ["normal", "e1"])
def test_c_parity_and_in_place(cuda_device, tile, layout, kind):
    M, N, K = 300, 520, 1280
    c, At, Bt = tn_case(M, N, K, 4800 + len(layout) + len(kind), cuda_device, kind)
    A = c["A"] if layout == "nn" else At
    B = c["B"] if layout == "tt" else Bt
    fn = {"tn": fg.fp8_gemm_tn, "nn": fg.fp8_gemm_nn, "tt": fg.fp8_gemm_tt}[layout]
    g = synth.make_generator(4900, cuda_device)
    if kind == "e1":  # multiples of 1/4 within +-64: C + (an E1 sum) is exact in FP32
        C = (torch.randint(-256, 257, (M, N), generator=g, device=cuda_device).float() / 4).to(torch.bfloat16)
    else:
        C = (torch.randn(M, N, generator=g, device=cuda_device) * 0.5).to(torch.bfloat16)
    ref, _ = oracle.gemm_nt_c(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(),
                              c["sb"].cpu().numpy(), bits_of(C))
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D, C=C)
    torch.cuda.synchronize()
    compare(kind, bits_of(D), ref, f"{layout} C {tile} {kind}")
    fn(A, c["sa"], B, c["sb"], C, C=C)                      # in place: C is D
    torch.cuda.synchronize()
    compare(kind, bits_of(C), ref, f"{layout} C in place {tile} {kind}")


# ---- split-K of the layout calls: forced splits over ragged K ranges (K = 1280: ten K
# blocks in splits of 4, 4, 2 or 2, 2, 2, 2, 2 ...), M with a partly live 64-row half
# (the fragments past M are not published), the UE8M0 and C forms, and the planner's own
# split on the few-row shapes at full size
def _layout_call(layout, c, At, Bt):
    A = c["A"] if layout == "nn" else At
    B = c["B"] if layout == "tt" else Bt
    return A, B, {"tn": fg.fp8_gemm_tn, "nn": fg.fp8_gemm_nn, "tt": fg.fp8_gemm_tt}[layout]


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("split", [2, 3, 10])
@pytest.mark.parametrize("kind", ["normal", "e1"])
@pytest.mark.parametrize("M,N,K", [(65, 200, 1280), (300, 520, 1280)])
@pytest.mark.parametrize("ring", ["4-stage", "2-stage"])
def test_split_k_parity(cuda_device, layout, split, kind, M, N, K, ring):
    """ring: with 8 CUs assumed the units outnumber the CUs and the 2-stage instance runs."""
    from parity_util import forced_workspace_bytes
    c, At, Bt = tn_case(M, N, K, 5000 + split + M, cuda_device, kind)
    A, B, fn = _layout_call(layout, c, At, Bt)
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    fg.set_num_cus(8 if ring == "2-stage" else 0)
    try:
        ws = torch.zeros(forced_workspace_bytes(fg.KIND_LAYOUT, M, N, K, 1, (128, 128, split)), dtype=torch.uint8,
                         device=cuda_device)
        for rep in range(2):   # the counters the first call leaves serve the second
            D = c["D"].clone()
            with fg.force_config(128, 128, split):
                fn(A, c["sa"], B, c["sb"], D, workspace=ws)
            torch.cuda.synchronize()
            compare(kind, bits_of(D), ref, f"{layout} split {split} {ring} {kind} {M}x{N}x{K} call {rep}")
    finally:
        fg.set_num_cus(0)
    assert int(ws[:16384].view(torch.int32).abs().sum()) == 0   # every arrival counter reset


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("split", [2, 3, 10])
@pytest.mark.parametrize("kind", ["normal", "e1"])
@pytest.mark.parametrize("M,N,K", [(65, 200, 1280), (300, 520, 1280)])
@pytest.mark.parametrize("bm,bn", [(64, 128), (128, 64)])
def test_split_k_parity_narrow_tiles(cuda_device, layout, split, kind, M, N, K, bm, bn):
    """Split K on the 64x128 and 128x64 tiles (64-wide panels, 6-stage ring), twice through
    one workspace."""
    from parity_util import forced_workspace_bytes
    c, At, Bt = tn_case(M, N, K, 5050 + split + M + bm, cuda_device, kind)
    A, B, fn = _layout_call(layout, c, At, Bt)
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    ws = torch.zeros(forced_workspace_bytes(fg.KIND_LAYOUT, M, N, K, 1, (bm, bn, split)), dtype=torch.uint8,
                     device=cuda_device)
    for rep in range(2):
        D = c["D"].clone()
        with fg.force_config(bm, bn, split):
            fn(A, c["sa"], B, c["sb"], D, workspace=ws)
        torch.cuda.synchronize()
        compare(kind, bits_of(D), ref, f"{layout} {bm}x{bn} split {split} {kind} {M}x{N}x{K} call {rep}")
    assert int(ws[:16384].view(torch.int32).abs().sum()) == 0   # every arrival counter reset


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("bm,bn", [(128, 128), (64, 128), (128, 64)])
def test_split_k_ue8m0_and_c(cuda_device, layout, bm, bn):
    from parity_util import forced_workspace_bytes
    M, N, K = 130, 260, 1536
    ws = torch.zeros(forced_workspace_bytes(fg.KIND_LAYOUT, M, N, K, 1, (bm, bn, 4)), dtype=torch.uint8,
                     device=cuda_device)
    c, At, Bt = tn_case(M, N, K, 5100, cuda_device, "pow2")
    A, B, fn = _layout_call(layout, c, At, Bt)
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    D = c["D"].clone()
    with fg.force_config(bm, bn, 4):
        fn(A, c["sa"], B, c["sb"], D, ue8m0=True, workspace=ws)
    torch.cuda.synchronize()
    compare("normal", bits_of(D), ref, f"{layout} {bm}x{bn} ue8m0 split 4")
    c, At, Bt = tn_case(M, N, K, 5101, cuda_device, "normal")
    A, B, fn = _layout_call(layout, c, At, Bt)
    C = (torch.randn(M, N, generator=synth.make_generator(5102, cuda_device), device=cuda_device) * 0.5).to(
        torch.bfloat16)
    ref, _ = oracle.gemm_nt_c(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(),
                              c["sb"].cpu().numpy(), bits_of(C))
    with fg.force_config(bm, bn, 4):
        fn(A, c["sa"], B, c["sb"], C, C=C, workspace=ws)      # in place: C is D
    torch.cuda.synchronize()
    compare("normal", bits_of(C), ref, f"{layout} {bm}x{bn} C in place split 4")


def test_split_k_of_256_tiles_is_rejected(cuda_device):
    """K is not split with 256x256 tiles (their reduce would spill)."""
    M, N, K = 64, 256, 1024
    c, At, Bt = tn_case(M, N, K, 5250, cuda_device, "e1")
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=cuda_device)
    with fg.force_config(256, 256, 2):
        with pytest.raises(fg.Fp8GemmError, match="configuration"):
            fg.fp8_gemm_tn(At, c["sa"], Bt, c["sb"], c["D"].clone(), workspace=ws)


def test_split_k_workspace_too_small_is_an_error(cuda_device):
    M, N, K = 64, 256, 1024
    c, At, Bt = tn_case(M, N, K, 5200, cuda_device, "e1")
    ws = torch.zeros(1024, dtype=torch.uint8, device=cuda_device)
    with fg.force_config(128, 128, 4):
        with pytest.raises(fg.Fp8GemmError, match="workspace"):
            fg.fp8_gemm_tn(At, c["sa"], Bt, c["sb"], c["D"].clone(), workspace=ws)


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (128, 7168, 2048)])
def test_planner_split_few_row_full_size(cuda_device, layout, M, N, K):
    """The few-row shapes at full size with the planner's own split (auto plan, library
    workspace), against the oracle on every output."""
    cfg = fg.query_config(fg.KIND_LAYOUT, M, N, K)
    assert cfg["split_k"] > 1
    c, At, Bt = tn_case(M, N, K, 5300 + M + N, cuda_device, "normal")
    A, B, fn = _layout_call(layout, c, At, Bt)
    ws = fg.make_workspace(fg.KIND_LAYOUT, M, N, K, device=cuda_device)
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(), c["sb"].cpu().numpy())
    compare("normal", bits_of(D), ref, f"{layout} {M}x{N}x{K} auto split {cfg['split_k']}")


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
def test_planner_256_tiles_ragged_n_full_size(cuda_device, layout):
    """4096x2112x7168 with the planner's own plan on the full chip: 144 tiles of 256x256
    (N = 8 tiles + 64 columns), checked on sampled rows, every column, against the oracle."""
    M, N, K = 4096, 2112, 7168
    cfg = fg.query_config(fg.KIND_LAYOUT, M, N, K)
    assert (cfg["block_m"], cfg["block_n"], cfg["split_k"]) == (256, 256, 1)
    c, At, Bt = tn_case(M, N, K, 5400, cuda_device, "normal")
    A, B, fn = _layout_call(layout, c, At, Bt)
    D = c["D"].clone()
    fn(A, c["sa"], B, c["sb"], D)
    torch.cuda.synchronize()
    rows = sample_rows(M, 24, 5401)
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy()[rows], c["sa"].cpu().numpy()[:, rows], c["B"].cpu().numpy(),
                            c["sb"].cpu().numpy())
    compare("normal", bits_of(D)[rows], ref, f"{layout} {M}x{N}x{K} auto 256x256 sampled rows")
