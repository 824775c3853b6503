"""Randomised parity sweep of the TN, NN and TT calls: seeded random shapes (ragged M and
N, K of 1-10 blocks) in every layout, each under a randomly forced plan (128x128, 64x128,
128x64 or 256x256 tiles; K split 1-6 except on 256x256) or the automatic one, with FP32
or UE8M0 scales. The inputs are the exact cases E1 (small integers) and E3 (one-hot A,
power-of-two scales): every partial and final sum is exact in FP32 and representable in
BF16, so every output must equal the oracle's bit for bit whatever the plan."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import assert_bit_exact, bits_of, forced_workspace_bytes

pytestmark = pytest.mark.gpu

TILES = [(128, 128), (64, 128), (128, 64), (256, 256)]
LAYOUTS = ["tn", "nn", "tt"]


def cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N, K = int(rng.integers(1, 420)), int(rng.integers(1, 700)), 128 * int(rng.integers(1, 11))
        layout = LAYOUTS[int(rng.integers(len(LAYOUTS)))]
        ue8m0 = bool(rng.random() < 0.3)
        kind = "e3" if rng.random() < 0.3 else "e1"   # both exact, both with power-of-two scales
        plan = None
        if rng.random() >= 0.2:
            tile = TILES[int(rng.integers(len(TILES)))]
            split = 1 if tile == (256, 256) else int(rng.integers(1, min(K // 128, 6) + 1))
            plan = tile + (split,)
        out.append((i, M, N, K, layout, ue8m0, kind, plan))
    return out


def case_id(v):
    if isinstance(v, tuple):
        return "%dx%d_s%d" % v
    if v is None:
        return "auto"
    return str(v)


@pytest.mark.parametrize("i,M,N,K,layout,ue8m0,kind,plan", cases(48, 20251206), ids=case_id)
def test_random_layout_plans_bit_exact(cuda_device, i, M, N, K, layout, ue8m0, kind, plan):
    c = synth.dense_case(M, N, K, seed=9900 + i, device=cuda_device, kind=kind)
    # the operands the layout stores K-major, as [K, rows] with rows padded to 16 bytes
    At = torch.zeros(K, (M + 15) // 16 * 16, dtype=torch.uint8, device=cuda_device)
    Bt = torch.zeros(K, (N + 15) // 16 * 16, dtype=torch.uint8, device=cuda_device)
    At[:, :M] = c["A"].t()
    Bt[:, :N] = c["B"].t()
    A = c["A"] if layout == "nn" else At
    B = c["B"] if layout == "tt" else Bt
    fn = {"tn": fg.fp8_gemm_tn, "nn": fg.fp8_gemm_nn, "tt": fg.fp8_gemm_tt}[layout]
    if plan is None:
        ws = fg.make_workspace(fg.KIND_LAYOUT, M, N, K, device=cuda_device)
    else:
        ws = torch.zeros(forced_workspace_bytes(fg.KIND_LAYOUT, M, N, K, 1, plan), dtype=torch.uint8,
                         device=cuda_device)
    D = c["D"].clone()
    if plan is None:
        fn(A, c["sa"], B, c["sb"], D, ue8m0=ue8m0, workspace=ws)
    else:
        with fg.force_config(*plan):
            fn(A, c["sa"], B, c["sb"], D, ue8m0=ue8m0, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(c["A"].cpu().numpy(), c["sa"].cpu().numpy(), c["B"].cpu().numpy(),
                            c["sb"].cpu().numpy())
    what = f"{layout} {kind} case {i}: {M}x{N}x{K} plan {case_id(plan)}{' ue8m0' if ue8m0 else ''}"
    assert_bit_exact(bits_of(D), ref, what)
    if plan is not None and plan[2] > 1:
        assert int(ws[:16384].view(torch.int32).abs().sum()) == 0, what + ": an arrival counter was left set"
