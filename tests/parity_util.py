"""Comparison helpers for GPU-vs-oracle parity (numpy only)."""
import numpy as np
import torch

import oracle

SENT = 0xFFFF


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def canon_zero(bits: np.ndarray) -> np.ndarray:
    b = np.array(bits, dtype=np.uint16, copy=True)
    b[b == 0x8000] = 0
    return b


def assert_bit_exact(gpu_bits, ref_bits, what=""):
    g, r = canon_zero(gpu_bits), canon_zero(ref_bits)
    bad = np.argwhere(g != r)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {g.size} outputs differ bitwise; first at {i}: "
                             f"gpu {g[i]:#06x} oracle {r[i]:#06x}")


def assert_within_tolerance(gpu_bits, ref_bits, what=""):
    """Per element |g - o| <= 2^-7 |o| + 1e-3 rms(o); globally sum (g-o)^2 / sum o^2 <= 1e-5.

    o is the oracle's BF16 output; rms and sums run over the compared (live) outputs.
    """
    g = oracle.bf16_bits_to_f64(gpu_bits)
    o = oracle.bf16_bits_to_f64(ref_bits)
    assert np.all(np.isfinite(o)), f"{what}: oracle produced non-finite values"
    if not np.all(np.isfinite(g)):
        i = tuple(np.argwhere(~np.isfinite(g))[0])
        raise AssertionError(f"{what}: non-finite GPU output at {i} (bits {np.asarray(gpu_bits)[i]:#06x})")
    if o.size == 0:
        return
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    bound = 2.0 ** -7 * np.abs(o) + 1e-3 * rms
    bad = np.argwhere(err > bound)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} outputs exceed the per-element bound; first at {i}: "
                             f"gpu {g[i]!r} oracle {o[i]!r} bound {bound[i]!r}")
    den = float(np.sum(o * o))
    if den > 0:
        rel = float(np.sum((g - o) ** 2)) / den
        assert rel <= 1e-5, f"{what}: global relative squared error {rel:.3e} > 1e-5"


def compare(kind, gpu_bits, ref_bits, what=""):
    if kind in ("e1", "e2", "e3"):
        assert_bit_exact(gpu_bits, ref_bits, what)
    else:
        assert_within_tolerance(gpu_bits, ref_bits, what)


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """Deterministic row sample: both ends, the middle, and random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, 63, 64, M // 2, M - 2, M - 1]
    extra = rng.choice(M, size=min(M, n), replace=False) if M > 0 else []
    return np.unique(np.clip(np.array(fixed + list(extra)), 0, max(M - 1, 0)))


def forced_workspace_bytes(kind, M, N, K, G, tile, full_tiles=0):
    """Workspace bytes of a call under a forced (block_m, block_n, split_k) plan, as the
    library computes it (at least 16 bytes, so a buffer can always be allocated)."""
    import moe_grouped_gemm_fp32_amd as fg
    with fg.force_config(*tile, full_tiles=full_tiles):
        return max(16, fg.workspace_size(kind, M, N, K, G))


def host(c, *keys):
    return [c[k].cpu().numpy() if isinstance(c[k], torch.Tensor) else c[k] for k in keys]
