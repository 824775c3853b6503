"""Randomised parity sweep of the K-grouped TN GEMM (fp8_k_grouped_gemm_tn_contiguous and
its UE8M0 form): seeded random group counts and token counts (empty groups and groups of
one token included), ragged M and N, both tile instances, and accumulation into an old D
of small integers. The inputs are the exact integer case E1 (every partial and final sum
is exact in FP32), so every output must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth

pytestmark = pytest.mark.gpu


def cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 11))
        tokens = [int(t) if rng.random() > 0.15 else 0 for t in rng.integers(1, 700, size=G)]
        M, N = int(rng.integers(1, 330)), int(rng.integers(1, 330))
        out.append((i, tokens, M, N, bool(rng.random() < 0.5), bool(rng.random() < 0.3),
                    "256x256" if rng.random() < 0.5 else "128x128"))
    return out


@pytest.mark.parametrize("i,tokens,M,N,accumulate,ue8m0,tile", cases(32, 20251207),
                         ids=lambda v: "-".join(map(str, v)) if isinstance(v, list) else str(v))
def test_random_k_grouped_bit_exact(cuda_device, i, tokens, M, N, accumulate, ue8m0, tile):
    # rows of the K-major operands padded to the 16-byte multiple the call requires
    c = synth.k_grouped_case(tokens, M, N, seed=9600 + i, device=cuda_device, kind="e1",
                             lda=(M + 15) // 16 * 16, ldb=(N + 15) // 16 * 16)
    G = c["G"]
    gen = synth.make_generator(9650 + i, cuda_device)
    D0 = torch.randint(-64, 65, (G, M, N), generator=gen, device=cuda_device).float() / 4
    D = D0.clone() if accumulate else c["D"].clone()
    fg.set_num_cus(1 if tile == "256x256" else 1 << 20)   # the planner's tile choice follows the CU count
    try:
        fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["ks"], accumulate=accumulate,
                                            ue8m0=ue8m0)
        torch.cuda.synchronize()
    finally:
        fg.set_num_cus(0)
    ref, _ = oracle.k_grouped_tn(c["A"][:, :M].cpu().numpy(), c["sa"].cpu().numpy(), c["B"][:, :N].cpu().numpy(),
                                 c["sb"].cpu().numpy(), c["ks"], D0.cpu().numpy() if accumulate else None)
    got = D.cpu().numpy()
    bad = np.argwhere(got != ref)
    what = f"case {i}: tokens {tokens} {M}x{N} {tile}{' accumulate' if accumulate else ''}{' ue8m0' if ue8m0 else ''}"
    assert not len(bad), f"{what}: {len(bad)} of {got.size} differ; first {tuple(bad[0])}: " \
                         f"{got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
