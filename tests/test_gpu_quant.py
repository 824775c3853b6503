"""GPU parity of the 1x128 activation quantisation (fp8_quantize_1x128 through the C
ABI) against the CPU oracle: e4m3 codes and FP32 scales bit for bit, over value
distributions that reach every rounding case (exact ties included), ragged shapes,
padded strides and the full-size activation of the dominant GEMM shape."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle

pytestmark = pytest.mark.gpu


def _rows(M, K, kind, seed):
    g = np.random.default_rng(seed)
    if kind == "normal":
        x = g.standard_normal((M, K))
    elif kind == "wide":  # every block its own magnitude, 2^-60 .. 2^60
        x = g.standard_normal((M, K)) * np.repeat(2.0 ** g.integers(-60, 60, size=(M, K // 128)), 128, axis=1)
    elif kind == "sparse":  # zero blocks, negative zeros, single non-zeros, bf16 subnormals
        x = np.zeros((M, K))
        x[:, 1::7] = -0.0
        x[::3, 5] = g.standard_normal(len(x[::3, 5]))
        x[1::4, 20:30] = 2.0 ** -130 * g.integers(1, 100, size=(len(x[1::4]), 10))
    elif kind == "ties":  # amax = 448 * 2^e, the rest exactly on e4m3 midpoints * 2^e
        vals = oracle.E4M3_TABLE[:0x7F]
        mids = (vals[:-1] + vals[1:]) / 2
        e = np.repeat(2.0 ** g.integers(-8, 8, size=(M, K // 128)), 128, axis=1)
        x = g.choice(np.concatenate([mids, vals]), size=(M, K)) * np.where(g.random((M, K)) < 0.5, -1, 1)
        x[:, ::128] = 448.0
        x = x * e
    else:
        raise ValueError(kind)
    return torch.tensor(x, dtype=torch.float32)


def _check(X, M, K, ldx_pad=0, ldq_pad=0, ldsa_pad=0, dtype=torch.bfloat16, what=""):
    dev = torch.device("cuda:0")
    big = torch.zeros(M, K + ldx_pad, dtype=dtype, device=dev)
    big[:, :K] = X.to(dtype).to(dev)
    x_host = big[:, :K].float().cpu().numpy()  # the values the kernel reads
    Qb = torch.full((M, K + ldq_pad), 0x5A, dtype=torch.uint8, device=dev)
    ld_sa = fg.scale_ld(M) + ldsa_pad
    sab = torch.full((K // 128, ld_sa), -7.0, dtype=torch.float32, device=dev)
    fg.quantize_1x128(big[:, :K], Qb[:, :K], sab)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_1x128(x_host)
    q = Qb.cpu().numpy()
    s = sab.cpu().numpy()
    bad = np.argwhere(q[:, :K] != q_ref)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:3].tolist()} " \
        f"x={x_host[tuple(bad[0])]!r} got {q[tuple(bad[0])]:#x} want {q_ref[tuple(bad[0])]:#x}"
    assert np.array_equal(s[:, :M].view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    assert np.all(q[:, K:] == 0x5A) and np.all(s[:, M:] == -7.0), f"{what}: wrote outside Q / sa"


@pytest.mark.parametrize("kind", ["normal", "wide", "sparse", "ties"])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (67, 1024), (300, 2048)])
def test_quantize_matches_oracle(cuda_device, kind, M, K):
    X = _rows(M, K, kind, seed=M * 7 + K + len(kind))
    _check(X, M, K, what=f"{kind} {M}x{K}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_padded_strides_and_fp32_input(cuda_device, dtype):
    X = _rows(70, 640, "wide", seed=5)
    _check(X, 70, 640, ldx_pad=8 if dtype == torch.bfloat16 else 4, ldq_pad=24, ldsa_pad=8, dtype=dtype,
           what=f"padded {dtype}")


def test_quantize_full_size_activation(cuda_device):
    # the A operand of the 4096 x 7168 x 16384 GEMM shape's K = 7168 sibling
    X = _rows(4096, 7168, "normal", seed=11)
    _check(X, 4096, 7168, what="4096x7168")


def test_quantized_output_feeds_the_gemm(cuda_device):
    # quantise A on the GPU, run the GEMM on it, compare with the oracle GEMM on the
    # oracle's own quantisation of the same values (identical bytes, so identical D)
    import synth
    from parity_util import bits_of, compare, host
    c = synth.dense_case(96, 256, 512, seed=3, device=cuda_device)
    X = torch.randn(96, 512, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    Q, sa = fg.quantize_1x128(X.to(cuda_device))
    q_ref, s_ref = oracle.quantize_1x128(X.float().numpy())
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    D = c["D"].clone()
    fg.fp8_gemm_nt(Q, sa, c["B"], c["sb"], D)
    torch.cuda.synchronize()
    sa_ref = np.zeros(sa.shape, dtype=np.float32)
    sa_ref[:, :96] = s_ref
    ref, _ = oracle.gemm_nt(q_ref, sa_ref, *host(c, "B", "sb"))
    compare("normal", bits_of(D), ref, "quantised A")
