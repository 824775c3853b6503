"""GPU parity of the K-grouped TN GEMM (fp8_k_grouped_gemm_tn_contiguous) against the CPU
oracle (oracle.k_grouped_tn): several tiles per group with ragged M / N tails and padded
leading dimensions, empty groups, exact integer cases bit for bit, accumulation into an
old D, strided and misaligned D (the scalar store path), 256 groups, and the MoE
weight-gradient shapes at full size on sampled rows and columns.

Tolerance: the exact integer cases must match bit for bit; every other case must meet
the library's floating-point bar, per element |gpu - oracle| <= 2^-7 |oracle| + 1e-3
rms(oracle) and globally sum (gpu - oracle)^2 / sum oracle^2 <= 1e-5. (An FP32-rounding
bound does not apply: the matrix unit's own sum of a 128-K block is less precise than
FP32, the imprecision that the per-block promotion exists to contain.)"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["128x128", "256x256"])
def tile(request):
    """Select the tile instance through the CU count the planner sees: the 256x256 tiles
    are taken once they alone give every CU a tile."""
    fg.set_num_cus(1 if request.param == "256x256" else 1 << 20)
    yield request.param
    fg.set_num_cus(0)


def _host(c):
    """The oracle's operands: A [K, M] and B [K, N] without the padding columns."""
    return [c["A"][:, :c["M"]].cpu().numpy(), c["sa"].cpu().numpy(),
            c["B"][:, :c["N"]].cpu().numpy(), c["sb"].cpu().numpy()]


def run(c, D=None, accumulate=False):
    D = c["D"].clone() if D is None else D
    fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["ks"], accumulate=accumulate)
    torch.cuda.synchronize()
    return D


def check(c, got, D_in=None, exact=False, rows=None, cols=None, what=""):
    A, sa, B, sb = _host(c)
    ref, T = oracle.k_grouped_tn(A, sa, B, sb, c["ks"], D_in, rows, cols)
    g = got.cpu().numpy()
    if rows is not None:
        g = g[:, rows][:, :, cols]
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if exact:
        bad = np.argwhere(g != ref)
        assert not len(bad), f"{what}: {len(bad)} of {g.size} differ; first {tuple(bad[0])}: {g[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
        return
    o = ref.astype(np.float64)
    gg = g.astype(np.float64)
    if o.size == 0:
        return
    rms = float(np.sqrt(np.mean(o * o)))
    bound = 2.0 ** -7 * np.abs(o) + 1e-3 * rms
    bad = np.argwhere(np.abs(gg - o) > bound)
    assert not len(bad), (f"{what}: {len(bad)} outputs exceed the per-element bound; first {tuple(bad[0])}: "
                          f"gpu {gg[tuple(bad[0])]!r} oracle {o[tuple(bad[0])]!r}")
    den = float(np.sum(o * o))
    if den > 0:
        rel = float(np.sum((gg - o) ** 2)) / den
        assert rel <= 1e-5, f"{what}: global relative squared error {rel:.3e} > 1e-5"
    return rel if den > 0 else 0.0


CASES = [
    # tokens per group, M, N, lda, ldb
    ([256, 384], 256, 256, None, None),
    ([100, 0, 300, 128], 384, 256, None, None),
    ([200, 57], 200, 136, 208, 144),          # ragged M / N tails, padded rows
    ([129], 40, 24, 48, 32),                  # one partial tile
    ([1000, 640, 0, 30], 128, 640, None, None),
    ([300, 500], 520, 600, 528, 608),          # three 256-row tile rows, ragged last ones
]


@pytest.mark.parametrize("kind", ["normal", "e1"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_parity(cuda_device, tile, kind, case):
    tokens, M, N, lda, ldb = CASES[case]
    c = synth.k_grouped_case(tokens, M, N, seed=9100 + case, device=cuda_device, kind=kind, lda=lda, ldb=ldb)
    got = run(c)
    check(c, got, exact=kind == "e1", what=f"{tile} {kind} case {case}")


@pytest.mark.parametrize("kind", ["normal", "e1"])
def test_accumulate(cuda_device, tile, kind):
    c = synth.k_grouped_case([256, 0, 128], 192, 160, seed=9200, device=cuda_device, kind=kind)
    gen = synth.make_generator(9201, cuda_device)
    D0 = torch.randint(-64, 65, (3, 192, 160), generator=gen, device=cuda_device).float() / 4
    if kind == "normal":
        D0 = torch.randn(3, 192, 160, generator=gen, device=cuda_device)
    got = run(c, D=D0.clone(), accumulate=True)
    check(c, got, D_in=D0.cpu().numpy(), exact=kind == "e1", what=f"accumulate {kind}")
    # an empty group leaves its old values untouched when accumulating, and is +0 otherwise
    assert torch.equal(got[1], D0[1])
    assert torch.all(run(c)[1] == 0)


def test_strided_and_misaligned_d(cuda_device, tile):
    c = synth.k_grouped_case([384, 128], 136, 100, seed=9300, device=cuda_device, kind="e1", lda=144, ldb=112)
    big = torch.full((2 * 150 * 103 + 1,), float("nan"), device=cuda_device)
    D = big[1:].view(2, 150, 103)[:, :136, :100]          # ldd 103 (odd), 4-byte aligned only
    got = run(c, D=D)
    check(c, got, exact=True, what="strided D")
    # the padding between rows and groups is not written
    full = big[1:].view(2, 150, 103)
    assert torch.all(torch.isnan(full[:, :, 100:])) and torch.all(torch.isnan(full[:, 136:, :]))


def test_many_groups(cuda_device):
    rng = np.random.default_rng(4)
    tokens = [int(t) for t in rng.choice([0, 1, 128, 200], size=fg.MAX_K_GROUPS)]
    c = synth.k_grouped_case(tokens, 64, 48, seed=9400, device=cuda_device, kind="e1")
    got = run(c)
    check(c, got, exact=True, what="256 groups")


def test_rejects_bad_arguments(cuda_device):
    c = synth.k_grouped_case([256], 64, 64, seed=9500, device=cuda_device)
    with pytest.raises(fg.Fp8GemmError):
        fg.k_grouped_fp8_gemm_tn_contiguous(c["A"][:200], c["sa"][:1], c["B"][:200], c["sb"][:1],
                                            c["D"], [200])                     # K not a multiple of 128
    A = torch.zeros(256, 72, dtype=torch.uint8, device=cuda_device)[:, :64]  # lda 72: not a multiple of 16
    with pytest.raises(fg.Fp8GemmError):
        fg.k_grouped_fp8_gemm_tn_contiguous(A, c["sa"], c["B"], c["sb"], c["D"], [256])


# the MoE weight-gradient shapes of the benchmark (gate+up and down projections), on
# sampled rows and columns
@pytest.mark.parametrize("M,N", [(4096, 7168), (7168, 2048)])
def test_full_size_sampled(cuda_device, M, N):
    tokens = synth.k_grouped_tokens(8, seed=9600)
    c = synth.k_grouped_case(tokens, M, N, seed=9601, device=cuda_device)
    got = run(c)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 12, replace=False)]))
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 12, replace=False)]))
    check(c, got, rows=rows, cols=cols, what=f"full {M}x{N}")


# ---- UE8M0 (power-of-two) scales through fp8_k_grouped_gemm_tn_contiguous_ue8m0: the
# oracle is the same K-grouped definition on the same power-of-two FP32 scale values
@pytest.mark.parametrize("kind", ["pow2", "e1"])
@pytest.mark.parametrize("case", [1, 2, 4, 5])
def test_ue8m0_parity(cuda_device, tile, kind, case):
    tokens, M, N, lda, ldb = CASES[case]
    c = synth.k_grouped_case(tokens, M, N, seed=9800 + case, device=cuda_device, kind=kind, lda=lda, ldb=ldb)
    D = c["D"].clone()
    fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["ks"], ue8m0=True)
    torch.cuda.synchronize()
    check(c, D, exact=kind == "e1", what=f"ue8m0 {tile} {kind} case {case}")


def test_ue8m0_accumulate_matches_fp32_scale_path(cuda_device):
    c = synth.k_grouped_case([300, 0, 500], 256, 384, seed=9900, device=cuda_device, kind="pow2")
    gen = synth.make_generator(9901, cuda_device)
    D0 = torch.randn(3, 256, 384, generator=gen, device=cuda_device)
    a, b = D0.clone(), D0.clone()
    fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], a, c["ks"], accumulate=True, ue8m0=True)
    fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], b, c["ks"], accumulate=True)
    torch.cuda.synchronize()
    check(c, a, D_in=D0.cpu().numpy(), what="ue8m0 accumulate")
    assert torch.equal(a[1], D0[1])
    rel = float(((a - b) ** 2).sum() / (b ** 2).sum())
    assert rel < 1e-9, f"UE8M0 and FP32-scale paths differ: {rel:.3e}"


@pytest.mark.parametrize("M,N", [(4096, 7168)])
def test_ue8m0_full_size_sampled(cuda_device, M, N):
    tokens = synth.k_grouped_tokens(8, seed=9600)
    c = synth.k_grouped_case(tokens, M, N, seed=9602, device=cuda_device, kind="pow2")
    D = c["D"].clone()
    fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["ks"], ue8m0=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + 1)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 12, replace=False)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.choice(N, 12, replace=False)]))
    check(c, D, rows=rows, cols=cols, what=f"ue8m0 full {M}x{N}")


def test_all_groups_empty(cuda_device, tile):
    """Every group of length 0 (called through the C ABI with valid buffers, none of them
    read): D is zero-filled, or left as it was when accumulating."""
    import ctypes
    c = synth.k_grouped_case([128], 96, 80, seed=9950, device=cuda_device)
    D = torch.full((3, 96, 80), 7.0, device=cuda_device)
    ks = (ctypes.c_int32 * 3)(0, 0, 0)
    stream = ctypes.c_void_p(torch.cuda.current_stream(cuda_device).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for accumulate, want in ((1, 7.0), (0, 0.0)):
        st = fg.lib().fp8_k_grouped_gemm_tn_contiguous(
            P(c["A"]), c["A"].stride(0), P(c["sa"]), c["sa"].stride(0), P(c["B"]), c["B"].stride(0), P(c["sb"]),
            c["sb"].stride(0), P(D), D.stride(1), D.stride(0), ctypes.cast(ks, ctypes.c_void_p), 3, 96, 80,
            accumulate, stream)
        assert st == 0, fg.status_string(st)
        torch.cuda.synchronize()
        assert torch.all(D == want)
