"""fp8_gemm_nt_noalloc (dense NT GEMM whose split-K scratch is the library's own per-device
array) called through the C ABI, against fp8_gemm_nt with a caller workspace: two calls
in a row that both split K, the second with a smaller input, then a call that does not
split; and a forced plan larger than the scratch is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp32_amd as fg
import oracle
import synth
from parity_util import assert_bit_exact, bits_of, compare, host, sample_rows

pytestmark = pytest.mark.gpu


def _noalloc(c, D):
    st = fg.lib().fp8_gemm_nt_noalloc(
        ctypes.c_void_p(c["A"].data_ptr()), c["A"].stride(0), ctypes.c_void_p(c["sa"].data_ptr()), c["sa"].stride(0),
        ctypes.c_void_p(c["B"].data_ptr()), c["B"].stride(0), ctypes.c_void_p(c["sb"].data_ptr()),
        ctypes.c_void_p(D.data_ptr()), D.stride(0), c["M"], c["N"], c["K"],
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_call(cuda_device):
    scratch = fg.noalloc_scratch_bytes()
    assert scratch == (32 << 20) + 16384
    # both K-split; the second call's input is smaller; then one without split-K
    shapes = [(128, 2112, 7168), (64, 2112, 7168), (100, 384, 512)]
    for i, (M, N, K) in enumerate(shapes):
        plan = fg.query_config(fg.KIND_DENSE, M, N, K)
        assert plan == fg.query_config(fg.KIND_DENSE, M, N, K, workspace_bytes=scratch)
        assert (plan["split_k"] > 1) == (i < 2), plan
        c = synth.dense_case(M, N, K, seed=7700 + i, device=cuda_device, a_std=1.0, b_std=0.02)
        D_ws = c["D"].clone()
        fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], D_ws, fg.make_workspace(fg.KIND_DENSE, M, N, K,
                                                                                  device=cuda_device))
        D_na = c["D"].clone()
        assert _noalloc(c, D_na) == 0
        torch.cuda.synchronize()
        # same plan, same kernels: the results agree bit for bit (and so within the bar)
        assert_bit_exact(bits_of(D_na), bits_of(D_ws), f"noalloc vs workspace call {M}x{N}x{K}")
        rows = sample_rows(M, 8, N)
        ref, _ = oracle.gemm_nt_sampled(*host(c, "A", "sa", "B", "sb"), rows, np.arange(N))
        compare("normal", bits_of(D_na)[rows], ref, f"noalloc vs oracle {M}x{N}x{K}")


def test_noalloc_rejects_plan_larger_than_scratch(cuda_device):
    M, N, K = 512, 8192, 1024   # 256 tiles of 128x128, split 8: 128 MiB of partials
    c = synth.dense_case(M, N, K, seed=7710, device=cuda_device)
    D = c["D"].clone()
    with fg.force_config(128, 128, 8):
        assert _noalloc(c, D) == -4  # FP8GEMM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((D.view(torch.int16) == c["D"].view(torch.int16)).all()), "nothing may be written"
