"""Randomised parity sweep: seeded random shapes (ragged M and N, K of 1-8 blocks) for the
dense, contiguous and masked calls, each under a randomly forced plan (every tile shape,
split K, whole-tile rounds) or the automatic one. The inputs are the bit-exact integer
case (E1: every partial and final sum is exact in FP32 and representable in BF16), so
every live output must equal the oracle's bit for bit whatever the plan, and every other
output cell must keep its sentinel."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import SENT, assert_bit_exact, bits_of, forced_workspace_bytes, host

pytestmark = pytest.mark.gpu

TILES = [(64, 64), (128, 64), (64, 128), (128, 128), (256, 128), (128, 256), (64, 96), (128, 96)]
GROUPED_TILES = [t for t in TILES if 128 % t[0] == 0]  # a contiguous tile holds one expert


def draw_plan(rng, K, tiles):
    if rng.random() < 0.2:
        return None
    tile = tiles[int(rng.integers(len(tiles)))]
    split = int(rng.integers(1, min(K // 128, 6) + 1))
    full = int(rng.integers(0, 4)) if split > 1 else 0
    return tile + (split, full)


def dense_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N, K = int(rng.integers(1, 400)), int(rng.integers(1, 800)), 128 * int(rng.integers(1, 9))
        out.append((i, M, N, K, draw_plan(rng, K, TILES)))
    return out


def plan_id(p):
    return "auto" if p is None else "%dx%d_s%d_f%d" % p


@pytest.mark.parametrize("i,M,N,K,plan", dense_cases(40, 20251203),
                         ids=lambda v: plan_id(v) if isinstance(v, tuple) or v is None else str(v))
def test_random_dense_plans_bit_exact(cuda_device, i, M, N, K, plan):
    c = synth.dense_case(M, N, K, seed=9000 + i, device=cuda_device, kind="e1")
    ref, _ = oracle.gemm_nt(*host(c, "A", "sa", "B", "sb"))
    D = c["D"].clone()
    if plan is None:
        ws = fg.make_workspace(fg.KIND_DENSE, M, N, K, device=cuda_device)
        fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, ws)
    else:
        nbytes = forced_workspace_bytes(fg.KIND_DENSE, M, N, K, 1, plan[:3], plan[3])
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=cuda_device)
        with fg.force_config(*plan[:3], full_tiles=plan[3]):
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D, ws)
    torch.cuda.synchronize()
    assert_bit_exact(bits_of(D), ref, f"dense case {i}: {M}x{N}x{K} plan {plan_id(plan)}")


def grouped_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 7))
        N, K = int(rng.integers(1, 600)), 128 * int(rng.integers(1, 7))
        out.append((i, G, N, K, draw_plan(rng, K, GROUPED_TILES)))
    return out


@pytest.mark.parametrize("i,G,N,K,plan", grouped_cases(16, 20251204),
                         ids=lambda v: plan_id(v) if isinstance(v, tuple) or v is None else str(v))
def test_random_contiguous_plans_bit_exact(cuda_device, i, G, N, K, plan):
    rng = np.random.default_rng(500 + i)
    rows = [int(v) for v in rng.choice([0, 1, 5, 63, 64, 127, 128, 129, 200, 300], size=G)]
    if sum(rows) == 0:
        rows[0] = 64  # at least one live row
    c = synth.contiguous_case(rows, N, K, seed=9500 + i, device=cuda_device, kind="e1")
    M = c["M"]
    D = c["D"].clone()
    if plan is None:
        nbytes = fg.workspace_size(fg.KIND_CONTIGUOUS, M, N, K, c["G"])
    else:
        nbytes = forced_workspace_bytes(fg.KIND_CONTIGUOUS, M, N, K, c["G"], plan[:3], plan[3])
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=cuda_device)
    if plan is None:
        fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"], ws)
    else:
        with fg.force_config(*plan[:3], full_tiles=plan[3]):
            fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["m_indices"], ws)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_contiguous(*host(c, "A", "sa", "B", "sb", "m_indices"), bits_of(c["D"]))
    got = bits_of(D)
    pad = c["m_indices"].cpu().numpy() < 0
    what = f"contiguous case {i}: rows {rows} N={N} K={K} plan {plan_id(plan)}"
    assert np.all(got[pad] == SENT), what + ": a padding row was written"
    assert_bit_exact(got[~pad], ref[~pad], what)


@pytest.mark.parametrize("i,G,N,K,plan", grouped_cases(16, 20251205),
                         ids=lambda v: plan_id(v) if isinstance(v, tuple) or v is None else str(v))
def test_random_masked_plans_bit_exact(cuda_device, i, G, N, K, plan):
    rng = np.random.default_rng(700 + i)
    M_max = int(rng.choice([64, 130, 256, 300]))
    mm = [int(v) for v in rng.integers(0, M_max + 1, size=G)]
    c = synth.masked_case(G, M_max, N, K, seed=9700 + i, device=cuda_device, masked_m=mm, kind="e1",
                          expected_m=max(1, M_max // 2))
    D = c["D"].clone()
    args = (c["A"], c["sa"], c["B"], c["sb"], D, c["masked_m"], c["expected_m"])
    if plan is None:
        fg.fp8_grouped_gemm_nt_masked(*args)
    else:
        # masked calls split every live tile (no whole-tile rounds)
        nbytes = forced_workspace_bytes(fg.KIND_MASKED, M_max, N, K, G, plan[:3])
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=cuda_device)
        with fg.force_config(*plan[:3]):
            fg.fp8_grouped_gemm_nt_masked(*args, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_masked(*host(c, "A", "sa", "B", "sb"), mm, bits_of(c["D"]))
    got = bits_of(D)
    what = f"masked case {i}: masked_m {mm} M_max={M_max} N={N} K={K} plan {plan_id(plan)}"
    for g, live in enumerate(mm):
        assert np.all(got[g, live:] == SENT), what + f": a dead row of group {g} was written"
        assert_bit_exact(got[g, :live], ref[g, :live], what + f" group {g}")
