"""GPU parity of the SwiGLU-fused 1x128 quantisation (fp8_swiglu_quantize_1x128 through
the C ABI) against the CPU oracle (oracle.swiglu_quantize_1x128).

The kernel evaluates silu(g) * u in FP64 and rounds it once to FP32, as the oracle
does (the two FP64 values can differ by an FP64 ulp or so through the exponential, which
changes the FP32 rounding only within ~2^-28 of an FP32 ulp of a midpoint); both then take
every quantisation decision in FP32. The bar: codes and scales bit for bit, as for the
plain quantiser; and, for every element, the dequantised value within half an e4m3 step
(times the scale, plus 2^-18 relative) of the exact SwiGLU value -- the quantiser's own
error bound. Padding rows (m_indices = -1) must be zero codes with unit scales."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth

pytestmark = pytest.mark.gpu

POS = oracle.E4M3_TABLE[:0x7F]                      # increasing values of codes 0x00..0x7E


def _step(a):
    """e4m3 spacing at magnitude a (the gap to the next code above)."""
    hi = np.clip(np.searchsorted(POS, a, side="right"), 1, 0x7E)
    return POS[hi] - POS[hi - 1]


def _check(H, mi, what):
    dev = H.device
    Q, sa = fg.swiglu_quantize_1x128(H, mi)
    torch.cuda.synchronize()
    h = H.float().cpu().numpy()
    m = None if mi is None else mi.cpu().numpy()
    q_ref, s_ref, y_ref = oracle.swiglu_quantize_1x128(h, m)
    M, F = y_ref.shape
    q, s = Q.cpu().numpy(), sa.cpu().numpy()[:, :M]
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ bitwise"
    bad = np.argwhere(q != q_ref)
    assert not len(bad), f"{what}: {len(bad)} codes differ; first at {tuple(bad[0])}: gpu {q[tuple(bad[0])]:#04x} " \
                         f"oracle {q_ref[tuple(bad[0])]:#04x}"
    # the quantiser's error bound against the exact SwiGLU value
    exact = oracle.swiglu(h)
    if m is not None:
        exact[m[:M] < 0] = 0.0
    sg = np.repeat(s.T.astype(np.float64), 128, axis=1)
    deq = oracle.decode_e4m3(q) * sg
    bound = 0.5 * _step(np.minimum(np.abs(exact) / sg, 448.0)) * sg * (1 + 2.0 ** -18) + 2.0 ** -18 * np.abs(exact)
    assert np.all(np.abs(deq - exact) <= bound), f"{what}: dequantised values exceed the quantiser's bound"
    if m is not None:
        pad = m[:M] < 0
        assert np.all(q[pad] == 0) and np.all(s[:, pad] == 1.0), f"{what}: padding rows"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,F", [(1, 128), (37, 256), (300, 2048)])
def test_parity(cuda_device, dtype, M, F):
    g = synth.make_generator(1200 + M + F, cuda_device)
    H = (torch.randn(M, 2 * F, generator=g, device=cuda_device) * 2).to(dtype)
    _check(H, None, f"{dtype} {M}x{F}")


def test_extreme_gates_and_near_ties(cuda_device):
    """Gates where the FP32 exponential overflows (g < -88) with large ups, so the exact
    value is normal while a plain FP32 evaluation gives 0; blocks whose maximum is tiny;
    gates whose SwiGLU values sit on e4m3 rounding midpoints; and a block where two
    elements tie for the maximum: codes and scales bit for bit."""
    g = synth.make_generator(1600, cuda_device)
    M, F = 8, 512
    gate = torch.randn(M, F, generator=g, device=cuda_device) * 3
    upv = torch.randn(M, F, generator=g, device=cuda_device)
    gate[0, :128] = -torch.linspace(85, 100, 128, device=cuda_device)      # exp(-g) past FP32
    upv[0, :128] = 1e30
    gate[1, 128:256] = -95.0                                                # a whole block of tiny values
    upv[1, 128:256] = torch.linspace(1, 2, 128, device=cuda_device)
    gate[2, :128] = 40.0                                                    # silu(g) = g: y = 40 u
    upv[2, :128] = (torch.arange(128, device=cuda_device) + 0.5) / 40.0   # y on odd multiples of 0.5
    gate[3, 256:384] = 5.0
    upv[3, 256:384] = 1.0                                                   # every element ties for the max
    H = torch.cat([gate, upv], dim=1)
    _check(H, None, "extreme gates")


def test_contiguous_padding_rows(cuda_device):
    mi, _ = synth.contiguous_layout([100, 0, 57, 128])
    M = mi.numel()
    g = synth.make_generator(1300, cuda_device)
    H = torch.randn(M, 2 * 512, generator=g, device=cuda_device).to(torch.bfloat16)
    _check(H, mi.to(cuda_device), "contiguous padding")


def test_strided_input_and_wide_range(cuda_device):
    g = synth.make_generator(1400, cuda_device)
    big = torch.randn(64, 2 * 384 + 16, generator=g, device=cuda_device)
    big[:, :384] *= torch.exp2(torch.randint(-20, 20, (64, 1), generator=g, device=cuda_device).float())
    H = big[:, :2 * 384]                                   # row stride 784 elements
    _check(H, None, "strided fp32")


def test_moe_down_projection_input(cuda_device):
    """The MoE FFN's down-projection input: the gate+up GEMM output of the routed rows."""
    c = synth.moe_case(seed=5, device=cuda_device, tokens=256, experts=16, N=2 * 256, K=512)
    D = c["D"].clone()
    fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"])
    torch.cuda.synchronize()
    live = c["m_indices"] >= 0
    H = torch.where(live[:, None], D, torch.zeros_like(D))   # padding rows of D were never written
    _check(H, c["m_indices"], "moe down input")


def test_rejects_bad_arguments(cuda_device):
    H = torch.zeros(4, 200, dtype=torch.bfloat16, device=cuda_device)
    with pytest.raises(ValueError):
        fg.swiglu_quantize_1x128(H)                          # F = 100 is not a multiple of 128


def test_empty_and_single_row(cuda_device):
    # M = 0 through the C ABI (torch gives zero-element tensors a null pointer): a no-op
    import ctypes
    big = torch.zeros(4, 256, dtype=torch.bfloat16, device=cuda_device)
    Qb = torch.zeros(4, 128, dtype=torch.uint8, device=cuda_device)
    sab = torch.ones(1, 4, dtype=torch.float32, device=cuda_device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = fg.lib().fp8_swiglu_quantize_1x128(P(big), 256, fg.QUANT_BF16, None, P(Qb), 128, P(sab), 4, 0, 128,
                                            ctypes.c_void_p(torch.cuda.current_stream(cuda_device).cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and torch.all(Qb == 0) and torch.all(sab == 1)
    g = synth.make_generator(1500, cuda_device)
    _check(torch.randn(1, 256, generator=g, device=cuda_device).to(torch.bfloat16), None, "one row")
