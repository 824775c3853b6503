"""Seeded synthetic inputs for the FP8 block-scaled NT GEMM and its M-grouped variants.

Shared by the GPU tests, the benchmark and the CPU oracle's tests. It holds none of
the GEMM's arithmetic: it draws FP32 tensors from a seeded torch generator, turns
them into e4m3 bytes plus FP32 block scales (the caller-side preparation that the
DeepGEMM pages leave to the user: "Interfaz GEMM y restricciones de layout",
es.news.hada.io/topic?id=19459), and builds the integer routing tensors of the
grouped variants (``m_indices`` with -1 padding rows, ``masked_m``).

Layouts produced (the library's documented layouts):
  A   uint8 (e4m3 bytes) [rows, K], row-major
  sa  float32 [K/128, ld_sa]: one scale per row per 128-wide K block, rows
      contiguous (the transposed scale layout the pages ask for), ld_sa = rows
      rounded up to a multiple of 4; grouped-masked adds a leading G
  B   uint8 [N, K] (grouped: [G, N, K])
  sb  float32 [ceil(N/128), K/128] (grouped: [G, ceil(N/128), K/128]): one scale
      per 128x128 block
  D   bfloat16 [rows, N], pre-filled with the sentinel bit pattern 0xFFFF

Kinds of operand content:
  "normal": A ~ N(0, a_std), B ~ N(0, b_std), quantised with scale = amax/448
            per block (scale 1 for an all-zero block).
  "pow2":   as "normal" with every scale rounded up to a power of two (UE8M0
            scale factors); the e1/e2/e3 kinds below also use power-of-two scales.
  "e1":     small-integer codes {0, +-1, +-2} (A) and {0, +-1} (B), scales drawn
            from {1/2, 1, 2}; sparse enough that every output is a multiple of
            1/4 of small magnitude, so any FP32 summation order is exact and the
            BF16 result is the exact sum.
  "e2":     scales 1, positive-biased integer codes so outputs are integers in
            the hundreds to thousands: exact in FP32 but often exact BF16 ties,
            which pins round-to-nearest-even.
  "e3":     one-hot A (a single 1.0 per row), power-of-two scales with random
            exponents: every output is one scaled B element, so a transposed
            or shifted scale index shows up as a wrong power of two.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import torch

BLOCK_K = 128          # K extent of one scale block (both operands)
BLOCK_N_SCALE = 128    # N extent of one B scale block
E4M3_MAX = 448.0
CONTIG_ALIGN = 128     # row alignment of each expert segment in the contiguous layout
SENTINEL_BITS = 0xFFFF  # bf16 NaN pattern no finite output can take

KINDS = ("normal", "e1", "e2", "e3")


def scale_ld(rows: int) -> int:
    """Leading dimension of the transposed activation-scale array: rows rounded up to 4."""
    return (int(rows) + 3) // 4 * 4


def make_generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _to_e4m3_bytes(x: torch.Tensor) -> torch.Tensor:
    """Cast FP32 values (already within +-448) to e4m3 bytes with torch's float8 cast."""
    return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def pow2_ceil(s: torch.Tensor) -> torch.Tensor:
    """Smallest power of two >= s (s > 0, FP32): the UE8M0 rounding of a scale, which
    keeps every |x / scale| within 448."""
    m, e = torch.frexp(s)  # s = m * 2^e, 0.5 <= m < 1
    return torch.where(m == 0.5, s, torch.ldexp(torch.ones_like(s), e))


def _block_scale(amax: torch.Tensor, pow2: bool) -> torch.Tensor:
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    return pow2_ceil(scale) if pow2 else scale


def quantize_act(x: torch.Tensor, ld: Optional[int] = None, pow2: bool = False):
    """1x128 quantisation of activations x [R, K] -> (codes [R, K], sa [K/128, ld]);
    pow2: scales rounded up to powers of two (UE8M0 scale factors)."""
    R, K = x.shape
    assert K % BLOCK_K == 0
    kb = K // BLOCK_K
    ld = scale_ld(R) if ld is None else ld
    xb = x.float().reshape(R, kb, BLOCK_K)
    amax = xb.abs().amax(dim=-1)
    scale = _block_scale(amax, pow2)
    q = _to_e4m3_bytes(xb / scale.unsqueeze(-1)).reshape(R, K)
    sa = torch.zeros(kb, ld, dtype=torch.float32, device=x.device)
    sa[:, :R] = scale.t()
    return q.contiguous(), sa


def quantize_weight(w: torch.Tensor, pow2: bool = False):
    """128x128 quantisation of weights w [N, K] -> (codes [N, K], sb [ceil(N/128), K/128]);
    pow2: scales rounded up to powers of two (UE8M0 scale factors)."""
    N, K = w.shape
    assert K % BLOCK_K == 0
    kb = K // BLOCK_K
    nb = (N + BLOCK_N_SCALE - 1) // BLOCK_N_SCALE
    pad = nb * BLOCK_N_SCALE - N
    wp = torch.nn.functional.pad(w.float(), (0, 0, 0, pad))
    blocks = wp.reshape(nb, BLOCK_N_SCALE, kb, BLOCK_K)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = _block_scale(amax, pow2)
    q = _to_e4m3_bytes(blocks / scale[:, None, :, None]).reshape(nb * BLOCK_N_SCALE, K)[:N]
    return q.contiguous(), scale.contiguous()


def pack_ue8m0(scales: torch.Tensor, axis: int) -> torch.Tensor:
    """Power-of-two FP32 scales -> int32 words of packed E8M0 codes (a power of two's code
    is its FP32 exponent field): entries 4w..4w+3 along `axis` in bytes 0..3 of word w,
    the last word zero-padded. The packed-UE8M0 inputs of the *_ue8m0_packed calls."""
    codes = ((scales.contiguous().view(torch.int32) >> 23) & 0xFF).to(torch.int64).movedim(axis, -1)
    n = codes.shape[-1]
    nw = (n + 3) // 4
    pad = torch.zeros(codes.shape[:-1] + (nw * 4,), dtype=torch.int64, device=codes.device)
    pad[..., :n] = codes
    pad = pad.reshape(codes.shape[:-1] + (nw, 4))
    w = pad[..., 0] | (pad[..., 1] << 8) | (pad[..., 2] << 16) | (pad[..., 3] << 24)
    w = torch.where(w >= 2 ** 31, w - 2 ** 32, w).to(torch.int32).movedim(-1, axis)
    out = torch.empty(w.shape, dtype=torch.int32, device=w.device)  # row-major strides
    out.copy_(w)
    return out


def random_bytes(shape, gen: torch.Generator, device) -> torch.Tensor:
    """Uniform random bytes (NaN codes 0x7F/0xFF included): content of dead rows."""
    return torch.randint(0, 256, tuple(shape), generator=gen, device=device, dtype=torch.uint8)


def _small_int_codes(shape, values: Sequence[int], probs: Sequence[float], gen, device):
    """e4m3 codes of integers drawn from ``values`` with probabilities ``probs``."""
    edges = torch.tensor(list(probs), dtype=torch.float64).cumsum(0)[:-1]
    edges = (edges / sum(probs)).to(torch.float32).to(device)
    u = torch.rand(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    idx = torch.bucketize(u, edges, right=True)
    v = torch.tensor(list(values), dtype=torch.float32, device=device)[idx]
    return _to_e4m3_bytes(v)


def _pow2(exps: torch.Tensor) -> torch.Tensor:
    return torch.exp2(exps.float())


# --------------------------------------------------------------------------- operands
def make_act(R: int, K: int, kind: str, gen, device, std: float = 1.0, ld: Optional[int] = None):
    """Activation operand (codes [R, K], sa [K/128, ld]) of the given kind."""
    kb = K // BLOCK_K
    ld = scale_ld(R) if ld is None else ld
    if kind in ("normal", "pow2"):
        x = torch.randn(R, K, generator=gen, device=device, dtype=torch.float32) * std
        return quantize_act(x, ld, pow2=kind == "pow2")
    sa = torch.zeros(kb, ld, dtype=torch.float32, device=device)
    if kind == "e1":
        # density chosen so the expected |sum| over all K blocks stays near 16
        pa = min(0.5, math.sqrt(16.0 / (1.5 * 5.44 * K)))
        q = _small_int_codes((R, K), [0, 1, -1, 2, -2], [1 - pa, pa / 4, pa / 4, pa / 4, pa / 4], gen, device)
        e = torch.randint(-1, 2, (kb, R), generator=gen, device=device)
        sa[:, :R] = _pow2(e)
    elif kind == "e2":
        q = _small_int_codes((R, K), [0, 1, 2, 3, 4, -1], [0.3, 0.25, 0.2, 0.1, 0.1, 0.05], gen, device)
        sa[:, :R] = 1.0
    elif kind == "e3":
        q = torch.zeros(R, K, dtype=torch.uint8, device=device)
        col = torch.randint(0, K, (R,), generator=gen, device=device)
        q[torch.arange(R, device=device), col] = _to_e4m3_bytes(torch.ones(R, device=device))
        e = torch.randint(-20, 21, (kb, R), generator=gen, device=device)
        sa[:, :R] = _pow2(e)
    else:
        raise ValueError(kind)
    return q.contiguous(), sa


def make_weight(N: int, K: int, kind: str, gen, device, std: float = 0.02):
    """Weight operand (codes [N, K], sb [ceil(N/128), K/128]) of the given kind."""
    kb = K // BLOCK_K
    nb = (N + BLOCK_N_SCALE - 1) // BLOCK_N_SCALE
    if kind in ("normal", "pow2"):
        w = torch.randn(N, K, generator=gen, device=device, dtype=torch.float32) * std
        return quantize_weight(w, pow2=kind == "pow2")
    if kind == "e1":
        pb = min(0.5, math.sqrt(16.0 / (1.5 * 5.44 * K)))
        q = _small_int_codes((N, K), [0, 1, -1], [1 - pb, pb / 2, pb / 2], gen, device)
        sb = _pow2(torch.randint(-1, 2, (nb, kb), generator=gen, device=device))
    elif kind == "e2":
        # scale so that typical row sums land in [256, 4096): many exact BF16 ties
        dens = min(1.0, 1200.0 / (K * 2.0))
        q = _small_int_codes((N, K), [0, 1, 2], [1 - dens, dens * 0.7, dens * 0.3], gen, device)
        sb = torch.ones(nb, kb, dtype=torch.float32, device=device)
    elif kind == "e3":
        x = torch.randn(N, K, generator=gen, device=device, dtype=torch.float32) * 64.0
        q = _to_e4m3_bytes(x)
        q = torch.where((q == 0x7F) | (q == 0xFF), torch.zeros_like(q), q)
        sb = _pow2(torch.randint(-20, 21, (nb, kb), generator=gen, device=device))
    else:
        raise ValueError(kind)
    return q.contiguous(), sb.contiguous()


def sentinel_output(shape, device) -> torch.Tensor:
    """BF16 output buffer whose every element holds the sentinel bits 0xFFFF."""
    return torch.full(tuple(shape), -1, dtype=torch.int16, device=device).view(torch.bfloat16)


# --------------------------------------------------------------------------- cases
def dense_case(M: int, N: int, K: int, seed: int, device="cpu", kind: str = "normal",
               a_std: float = 1.0, b_std: float = 0.02) -> Dict[str, object]:
    """Dense D[M,N] = A[M,K] B[N,K]^T inputs, A drawn first, then B."""
    gen = make_generator(seed, device)
    A, sa = make_act(M, K, kind, gen, device, std=a_std)
    B, sb = make_weight(N, K, kind, gen, device, std=b_std)
    return dict(kind="dense", M=M, N=N, K=K, A=A, sa=sa, B=B, sb=sb,
                D=sentinel_output((M, N), device))


def contiguous_layout(group_rows: Sequence[int], align: int = CONTIG_ALIGN):
    """Per-row expert ids for expert segments concatenated along M.

    Each segment of group_rows[g] live rows is followed by -1 padding rows up to a
    multiple of ``align`` (a segment with 0 rows takes no rows at all).
    Returns (m_indices int32 [M_total] on CPU, list of (start, live_rows) per group).
    """
    ids: List[int] = []
    segs = []
    for g, r in enumerate(group_rows):
        start = len(ids)
        padded = (r + align - 1) // align * align
        ids += [g] * r + [-1] * (padded - r)
        segs.append((start, r))
    return torch.tensor(ids, dtype=torch.int32), segs


def contiguous_case(group_rows: Sequence[int], N: int, K: int, seed: int, device="cpu",
                    kind: str = "normal", a_std: float = 1.0, b_std: float = 0.02,
                    garbage_padding: bool = True) -> Dict[str, object]:
    """M-grouped contiguous inputs: A [M_total, K] shared, B [G, N, K], m_indices [M_total]."""
    gen = make_generator(seed, device)
    G = len(group_rows)
    m_idx, segs = contiguous_layout(group_rows)
    Mt = int(m_idx.numel())
    A, sa = make_act(Mt, K, kind, gen, device, std=a_std)
    live = (m_idx >= 0).to(device)
    if garbage_padding and Mt > 0:
        junk = random_bytes((Mt, K), gen, device)
        A = torch.where(live[:, None], A, junk).contiguous()
    Bs, sbs = [], []
    for _ in range(G):
        b, s = make_weight(N, K, kind, gen, device, std=b_std)
        Bs.append(b)
        sbs.append(s)
    return dict(kind="contiguous", M=Mt, N=N, K=K, G=G, A=A, sa=sa,
                B=torch.stack(Bs).contiguous(), sb=torch.stack(sbs).contiguous(),
                m_indices=m_idx.to(device), segments=segs,
                D=sentinel_output((Mt, N), device))


def draw_masked_m(G: int, seed: int, lo: int = 179, hi: int = 333) -> List[int]:
    """Live rows per group, uniform integers in [lo, hi] inclusive (mean (lo+hi)/2)."""
    gen = make_generator(seed, "cpu")
    return torch.randint(lo, hi + 1, (G,), generator=gen).tolist()


def masked_case(G: int, M_max: int, N: int, K: int, seed: int, device="cpu",
                masked_m: Optional[Sequence[int]] = None, kind: str = "normal",
                a_std: float = 1.0, b_std: float = 0.02, expected_m: int = 256,
                garbage_dead: bool = True) -> Dict[str, object]:
    """M-grouped masked inputs: A [G, M_max, K], sa [G, K/128, ld], B [G, N, K], masked_m [G]."""
    gen = make_generator(seed, device)
    if masked_m is None:
        masked_m = draw_masked_m(G, seed + 7)
    masked_m = [int(v) for v in masked_m]
    assert len(masked_m) == G and all(0 <= v <= M_max for v in masked_m)
    ld = scale_ld(M_max)
    As, sas, Bs, sbs = [], [], [], []
    for g in range(G):
        live = masked_m[g]
        a_live, sa_live = make_act(max(live, 0), K, kind, gen, device, std=a_std, ld=ld) if live else (
            torch.zeros(0, K, dtype=torch.uint8, device=device),
            torch.zeros(K // BLOCK_K, ld, dtype=torch.float32, device=device))
        dead = M_max - live
        if garbage_dead:
            a_dead = random_bytes((dead, K), gen, device)
        else:
            a_dead = torch.zeros(dead, K, dtype=torch.uint8, device=device)
        As.append(torch.cat([a_live, a_dead], 0))
        sa_g = sa_live.clone()
        if dead:
            # dead rows get finite junk scales: they must not leak into live rows either
            sa_g[:, live:M_max] = torch.rand(K // BLOCK_K, dead, generator=gen, device=device) * 1e3
        sas.append(sa_g)
        b, s = make_weight(N, K, kind, gen, device, std=b_std)
        Bs.append(b)
        sbs.append(s)
    return dict(kind="masked", G=G, M_max=M_max, N=N, K=K, expected_m=expected_m,
                A=torch.stack(As).contiguous(), sa=torch.stack(sas).contiguous(),
                B=torch.stack(Bs).contiguous(), sb=torch.stack(sbs).contiguous(),
                masked_m=torch.tensor(masked_m, dtype=torch.int32, device=device),
                masked_m_list=masked_m,
                D=sentinel_output((G, M_max, N), device))


# --------------------------------------------------------------------------- MoE routing
def moe_routing(tokens: int = 4096, experts: int = 256, topk: int = 8, zipf_s: float = 1.1,
                seed: int = 0):
    """Top-k expert choice per token with Zipf(s) expert popularity.

    Expert popularity w_e is proportional to rank^-s under a seeded random
    permutation of the experts; each token draws ``topk`` distinct experts by
    weighted sampling without replacement (Gumbel-top-k on log w).
    Returns (expert_of int64 [tokens, topk], counts list[int] per expert).
    """
    gen = make_generator(seed, "cpu")
    perm = torch.randperm(experts, generator=gen)
    rank = torch.empty(experts, dtype=torch.float64)
    rank[perm] = torch.arange(1, experts + 1, dtype=torch.float64)
    logw = -zipf_s * torch.log(rank)
    u = torch.rand(tokens, experts, generator=gen, dtype=torch.float64).clamp_(1e-300, 1.0)
    keys = logw[None, :] - torch.log(-torch.log(u))
    expert_of = torch.topk(keys, topk, dim=1).indices
    counts = torch.bincount(expert_of.reshape(-1), minlength=experts).tolist()
    return expert_of, counts


def moe_contiguous_rows(expert_of: torch.Tensor, experts: int, align: int = CONTIG_ALIGN):
    """Row plan of the contiguous layout for a routing: (m_indices, token_of_row).

    Rows of expert e hold the tokens routed to e in token order, then -1 padding;
    token_of_row is -1 on padding rows.
    """
    tok = torch.arange(expert_of.shape[0]).repeat_interleave(expert_of.shape[1])
    exp_flat = expert_of.reshape(-1)
    ids: List[int] = []
    tokens: List[int] = []
    for e in range(experts):
        t = tok[exp_flat == e].tolist()
        padded = (len(t) + align - 1) // align * align
        ids += [e] * len(t) + [-1] * (padded - len(t))
        tokens += t + [-1] * (padded - len(t))
    return torch.tensor(ids, dtype=torch.int32), torch.tensor(tokens, dtype=torch.int64)


def moe_case(seed: int, device="cpu", tokens: int = 4096, experts: int = 256, topk: int = 8,
             zipf_s: float = 1.1, N: int = 4096, K: int = 7168, kind: str = "normal",
             b_std: float = 0.02, x: Optional[torch.Tensor] = None,
             garbage_padding: bool = True) -> Dict[str, object]:
    """Contiguous-layout inputs of one MoE FFN GEMM.

    ``x`` [tokens, K] FP32 token activations (drawn from N(0,1) when None) are
    gathered to their expert rows and quantised 1x128; padding rows get random
    bytes. B holds one [N, K] weight per expert.
    """
    gen = make_generator(seed, device)
    expert_of, counts = moe_routing(tokens, experts, topk, zipf_s, seed)
    m_idx, tok_of_row = moe_contiguous_rows(expert_of, experts)
    Mt = int(m_idx.numel())
    if x is None:
        x = torch.randn(tokens, K, generator=gen, device=device, dtype=torch.float32)
    rows = x[tok_of_row.clamp(min=0).to(device)]
    A, sa = quantize_act(rows, pow2=kind == "pow2")
    live = (m_idx >= 0).to(device)
    if garbage_padding:
        A = torch.where(live[:, None], A, random_bytes((Mt, K), gen, device)).contiguous()
    Bq = torch.empty(experts, N, K, dtype=torch.uint8, device=device)
    sb = torch.empty(experts, (N + 127) // 128, K // BLOCK_K, dtype=torch.float32, device=device)
    for e in range(experts):
        b, s = make_weight(N, K, kind, gen, device, std=b_std)
        Bq[e] = b
        sb[e] = s
    return dict(kind="contiguous", M=Mt, N=N, K=K, G=experts, A=A, sa=sa, B=Bq, sb=sb,
                m_indices=m_idx.to(device), token_of_row=tok_of_row, counts=counts,
                expert_of=expert_of, D=sentinel_output((Mt, N), device))


def swiglu_requant(h: torch.Tensor, m_indices: torch.Tensor, pow2: bool = False):
    """Down-projection input of the MoE FFN: SwiGLU(gate, up) of the BF16 gate+up output.

    h [rows, 2F] holds gate in the first F columns and up in the last F; padding
    rows (m_indices == -1) are zeroed before the 1x128 quantisation. This is the
    test harness's glue between the two GEMMs, not part of the measured path.
    """
    F = h.shape[1] // 2
    hf = h.float()
    live = (m_indices >= 0).to(h.device)
    hf = torch.where(live[:, None], hf, torch.zeros_like(hf))
    act = torch.nn.functional.silu(hf[:, :F]) * hf[:, F:]
    return quantize_act(act, pow2=pow2)


# --------------------------------------------------------------- K-grouped (TN) inputs
def k_grouped_case(tokens: Sequence[int], M: int, N: int, seed: int, device="cpu",
                   kind: str = "normal", a_std: float = 1.0, b_std: float = 1.0,
                   lda: Optional[int] = None, ldb: Optional[int] = None) -> Dict[str, object]:
    """Inputs of the K-grouped TN GEMM (MoE weight gradient): group g's segment holds
    tokens[g] token rows padded with zero rows to a multiple of 128 (ks[g]); the
    segments are laid end to end along K. Both operands are token-major activations,
    quantised per column per 128-row block: A codes [K, lda] with scales sa [K/128,
    scale_ld(M)], B codes [K, ldb] with sb [K/128, scale_ld(N)] (columns past M / N of
    the code arrays hold random bytes). D is FP32 [G, M, N] filled with NaN."""
    gen = make_generator(seed, device)
    ks = [(int(t) + BLOCK_K - 1) // BLOCK_K * BLOCK_K for t in tokens]
    K = sum(ks)
    lda = M if lda is None else lda
    ldb = N if ldb is None else ldb
    live = torch.zeros(K, dtype=torch.bool, device=device)
    k0 = 0
    for t, k in zip(tokens, ks):
        live[k0:k0 + int(t)] = True
        k0 += k

    def operand(C, ld, std):
        q, s = make_act(C, K, kind, gen, device, std=std)      # [C, K], [K/128, scale_ld(C)]
        q = torch.where(live[None, :], q, torch.zeros_like(q))
        full = random_bytes((K, ld), gen, device)
        full[:, :C] = q.t()
        return full.contiguous(), s

    A, sa = operand(M, lda, a_std)
    B, sb = operand(N, ldb, b_std)
    D = torch.full((len(ks), M, N), float("nan"), dtype=torch.float32, device=device)
    return dict(kind="k_grouped", M=M, N=N, K=K, G=len(ks), ks=ks, tokens=list(tokens),
                A=A, sa=sa, B=B, sb=sb, lda=lda, ldb=ldb, D=D)


def k_grouped_tokens(G: int = 8, seed: int = 0, mean: int = 2048, spread: float = 0.5) -> List[int]:
    """Tokens routed to each of G local experts: uniform integers in
    [mean (1 - spread), mean (1 + spread)] (the weight-gradient workload's segment mix)."""
    gen = make_generator(seed, "cpu")
    lo, hi = int(mean * (1 - spread)), int(mean * (1 + spread))
    return torch.randint(lo, hi + 1, (G,), generator=gen).tolist()
