"""CPU oracle for the FP8 block-scaled NT GEMM and its two M-grouped MoE variants.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import or run this module; the library never does.
It shares no code, table or helper with the HIP path.

What it computes (DeepGEMM pages: FP8 GEMM with DeepSeek-V3 fine-grained scaling and
two-level "promotion" accumulation -- es.news.hada.io/topic?id=19444 intro bullets;
bquan.live post 9429818, "Comprender profundamente DeepGEMM"; NT layout with BF16
output -- same post, "¿Cómo usarlo?"; es.news.hada.io/topic?id=19459 "Interfaz GEMM y
restricciones de layout"):

    D[m, n] = bf16_rne( sum_kb  P_kb[m, n] * sa[kb, m] * sb[n // 128, kb] )
    P_kb[m, n] = sum_{k in block kb} e4m3(A[m, k]) * e4m3(B[n, k])

with one FP32 scale per row per 128-wide K block for A (sa, stored K-block-major
[K/128, ld_sa]) and one FP32 scale per 128x128 block for B (sb [ceil(N/128), K/128]).
The pages name the scheme but not the block sizes; 1x128 / 128x128 is the DeepSeek-V3
granularity they refer to.

Precision: every block partial P_kb is computed in FP64 and is EXACT in any summation
order -- a decoded e4m3 value times 2^9 is an integer below 2^18, so a product times
2^18 is an integer below 2^36 and a 128-term sum stays below 2^43 < 2^53. The scaled
sum over blocks is FP64 (one rounding per operation), then a single round-to-nearest-
even to BF16.

Grouped variants ("Dense y Grouped GEMM", es.news.hada.io/topic?id=19459):
  contiguous -- rows of all experts concatenated along M; row r uses expert
                m_indices[r]; rows with -1 are padding and keep their old output.
  masked     -- A is [G, M_max, K]; only the first masked_m[g] rows of group g are
                computed, the rest keep their old output.
  K-grouped  -- the weight-gradient form D[g] = C[g] + A_g^T B_g, A [K, M] and B [K, N]
                split along K into per-expert segments, FP32 output (k_grouped_tn;
                its readings are stated beside it).

Every function below is pinned by tests/test_oracle_*.py (brute force in exact
rationals, bit-exact integer cases, a closed-form scale-indexing probe, library
cross-checks and invariants).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


# ------------------------------------------------------------------ e4m3 decode
def _e4m3_value(code: int) -> float:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; exponent field 0 is subnormal (2^-6 * m/8); max 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3 codes -> exact float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ------------------------------------------------------------------ bf16 rounding
def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even) -> uint16 bits.

    A single rounding straight from float64. bfloat16 keeps 8 significant bits and
    the float32 exponent range: for |x| in [2^(e-1), 2^e) the spacing is 2^(e-8),
    and below 2^-126 (subnormal) the spacing is fixed at 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    _, e = np.frexp(x)
    spacing_exp = np.maximum(e, -125) - 8
    q = np.rint(np.ldexp(x, -spacing_exp))          # np.rint: round half to even
    v = np.ldexp(q, spacing_exp)
    with np.errstate(over="ignore"):
        f32 = v.astype(np.float32)                  # exact: <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    # values that rounded past the largest finite bfloat16 become infinity
    big = np.abs(v) >= 2.0 ** 128
    bits = np.where(big, np.where(x < 0, 0xFF80, 0x7F80), bits).astype(np.uint16)
    out[...] = bits
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ core sum
def scaled_block_sum(A: np.ndarray, sa: np.ndarray, B: np.ndarray, sb: np.ndarray,
                     rows=None, cols=None) -> np.ndarray:
    """S[m, n] = sum_kb P_kb[m, n] * sa[kb, m] * sb[n // 128, kb] in float64.

    A uint8 [M, K], sa float32 [K/128, >=M], B uint8 [N, K], sb float32
    [ceil(N/128), K/128]. ``rows`` / ``cols`` select a subset of outputs (index
    arrays into M and N); the result is [len(rows), len(cols)].
    """
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2 and K % BLOCK == 0
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    Ar = A[rows]
    Bc = B[cols]
    S = np.zeros((len(rows), len(cols)), dtype=np.float64)   # starts at +0.0
    for kb in range(K // BLOCK):
        a = decode_e4m3(Ar[:, kb * BLOCK:(kb + 1) * BLOCK])
        b = decode_e4m3(Bc[:, kb * BLOCK:(kb + 1) * BLOCK])
        P = a @ b.T                                   # exact block partial
        s = sa[kb, rows].astype(np.float64)[:, None] * sb[cols // BLOCK, kb].astype(np.float64)[None, :]
        S += P * s                                    # promotion with both scales
    return S


# ------------------------------------------------------------------ the three calls
def gemm_nt(A, sa, B, sb):
    """Dense D = A B^T. Returns (bf16 bits uint16 [M, N], float64 S [M, N])."""
    S = scaled_block_sum(A, sa, B, sb)
    return bf16_bits_rne(S), S


def gemm_nt_sampled(A, sa, B, sb, rows, cols):
    """Dense D restricted to the outputs rows x cols: (bits, S) of shape [len(rows), len(cols)]."""
    S = scaled_block_sum(A, sa, B, sb, rows, cols)
    return bf16_bits_rne(S), S


def grouped_contiguous(A, sa, B, sb, m_indices, D_in, rows=None, cols=None):
    """M-grouped contiguous GEMM.

    A uint8 [M_total, K]; sa [K/128, >=M_total]; B uint8 [G, N, K];
    sb [G, ceil(N/128), K/128]; m_indices int32 [M_total] (-1 = padding row);
    D_in uint16 bits [M_total, N] (the output buffer before the call).
    Returns (D_out bits [len(rows), len(cols)], S float64 with NaN on padding rows).
    ``rows`` / ``cols`` restrict the computation to a sample.
    """
    m_indices = np.asarray(m_indices, dtype=np.int64)
    Mt = A.shape[0]
    N = B.shape[1]
    rows = np.arange(Mt) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    D = np.array(np.asarray(D_in, dtype=np.uint16)[np.ix_(rows, cols)], copy=True)
    S = np.full((len(rows), len(cols)), np.nan)
    for g in np.unique(m_indices[rows]):
        if g < 0:
            continue
        sel = np.nonzero(m_indices[rows] == g)[0]
        Sg = scaled_block_sum(A, sa, B[g], sb[g], rows[sel], cols)
        S[sel] = Sg
        D[sel] = bf16_bits_rne(Sg)
    return D, S


def grouped_masked(A, sa, B, sb, masked_m, D_in, rows=None, cols=None):
    """M-grouped masked GEMM.

    A uint8 [G, M_max, K]; sa [G, K/128, >=M_max]; B uint8 [G, N, K];
    sb [G, ceil(N/128), K/128]; masked_m int [G]; D_in bits [G, M_max, N].
    Rows m >= masked_m[g] keep D_in. Returns (D_out bits, S with NaN on dead rows),
    optionally restricted to rows/cols within each group.
    """
    G, M_max, _ = A.shape
    N = B.shape[1]
    rows = np.arange(M_max) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    D = np.array(np.asarray(D_in, dtype=np.uint16)[:, rows][:, :, cols], copy=True)
    S = np.full((G, len(rows), len(cols)), np.nan)
    for g in range(G):
        live = int(masked_m[g])
        sel = np.nonzero(rows < live)[0]
        if len(sel) == 0:
            continue
        Sg = scaled_block_sum(A[g], sa[g], B[g], sb[g], rows[sel], cols)
        S[g, sel] = Sg
        D[g, sel] = bf16_bits_rne(Sg)
    return D, S


# ------------------------------------------------------------------ 1x128 quantisation
# Upstream of every call: activations in FP32 or BF16 -> e4m3 codes plus one FP32
# scale per row per 128-wide K block, stored K-block-major [K/128, ld_sa] (the layout
# the GEMM reads). The pages leave the conversion to the user and give no formula
# (es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout": the
# library only offers simple PyTorch helpers). Reading used here, all in FP32 with
# IEEE round-to-nearest-even operations:
#     s = amax(|x| over the block) / 448      (s = 1 when that is 0)
#     q = e4m3_rne(x / s)                     (ties to the even code; a quotient past
#                                              448, reachable only by rounding, is 448)
_E4M3_POS = E4M3_TABLE[:0x7F]            # codes 0x00..0x7E, increasing values 0..448


def e4m3_rne_codes(y: np.ndarray) -> np.ndarray:
    """float32 values -> nearest e4m3 codes (ties to even code, saturating at 448).

    Positive codes 0x00..0x7E are increasing in value, so the code of the nearest
    value is its index in that list; the sign bit is copied (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, 0x7E)  # _E4M3_POS[hi-1] < a <= ...
    lo = hi - 1
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= _E4M3_POS[0x7E], 0x7E, code)          # at or past 448
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_1x128(x: np.ndarray):
    """x [R, K] (float32; BF16 inputs as their float32 values) -> (codes uint8 [R, K],
    scales float32 [K/128, R])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    assert K % BLOCK == 0
    xb = x.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=-1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (xb / s[..., None]).astype(np.float32)
    return e4m3_rne_codes(y).reshape(R, K), np.ascontiguousarray(s.T)


# ---------------------------------------------------------------- UE8M0 scale factors
# An E8M0 scale code e is the power of two 2^(e - 127) (8 exponent bits, bias 127, no
# sign and no mantissa); 255 is NaN. The pages list UE8M0 among DeepGEMM's scale
# formats (es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout");
# a GEMM with UE8M0 scales is the GEMM above with these values as sa and sb.
def ue8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 codes (uint8) -> FP64 scale values 2^(e - 127), NaN for 255."""
    e = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def gemm_nt_ue8m0(A, sa_codes, B, sb_codes):
    """Dense NT GEMM with UE8M0 scale codes sa_codes [K/128, >=M], sb_codes
    [ceil(N/128), K/128]: the definition of gemm_nt with the decoded scales."""
    return gemm_nt(A, ue8m0_decode(sa_codes), B, ue8m0_decode(sb_codes))


# ------------------------------------------------------------------ packed UE8M0 scale factors
# The newer API takes UE8M0 scale factors packed four to a 32-bit integer and offers a
# utility that converts FP32 scale factors into the layout a kernel requires (es.news.hada.io/
# topic?id=19459, "Interfaz GEMM y restricciones de layout": packed UE8M0, four per
# torch.int, LHS scales aligned and transposed; "Utilidades y variables de entorno":
# transform_sf_into_required_layout). The pages do not say along which axis or in which
# byte order the four codes are packed. The reading implemented: the four codes of one
# word belong to four consecutive 128-wide K blocks of the same row (activation scales)
# or 128x128 block row (weight scales), the code of K block 4w + j in byte j (bits
# 8j..8j+7) of word w; the words keep the FP32 layouts' orientation: activation scales
# [ceil(nkb / 4)][ld] (rows contiguous), weight scales [ceil(N/128)][ceil(nkb / 4)].
# Codes past nkb in the last word are 0.
def ue8m0_unpack(words, nkb: int, axis: int) -> np.ndarray:
    """Packed words (any integer dtype, 32-bit patterns) -> uint8 codes with nkb entries
    along `axis` (the packed axis holds ceil(nkb / 4) words)."""
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    w = np.moveaxis(w, axis, -1)
    codes = np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], axis=-1)   # [..., words, 4]
    codes = codes.reshape(codes.shape[:-2] + (codes.shape[-2] * 4,))[..., :nkb]
    return np.moveaxis(codes.astype(np.uint8), -1, axis)


def ue8m0_pack(codes, axis: int) -> np.ndarray:
    """uint8 codes -> int32 words packing four consecutive entries along `axis`."""
    c = np.moveaxis(np.asarray(codes, dtype=np.int64), axis, -1)
    nkb = c.shape[-1]
    nw = (nkb + 3) // 4
    pad = np.zeros(c.shape[:-1] + (nw * 4,), dtype=np.int64)
    pad[..., :nkb] = c
    pad = pad.reshape(c.shape[:-1] + (nw, 4))
    w = pad[..., 0] | (pad[..., 1] << 8) | (pad[..., 2] << 16) | (pad[..., 3] << 24)
    return np.moveaxis(w.astype(np.uint32).view(np.int32), -1, axis)


def ue8m0_from_fp32(sf) -> np.ndarray:
    """UE8M0 code of each positive, finite FP32 scale: the smallest power of two not
    below it, 2^(code - 127) >= sf (exact for a power of two; a scale between powers
    of two rounds up, so that no quantised value grows past the format's range)."""
    x = np.asarray(sf, dtype=np.float32).astype(np.float64)
    assert np.all(np.isfinite(x)) and np.all(x >= 2.0 ** -126) and np.all(x <= 2.0 ** 127), \
        "scales must be positive normal FP32 values no larger than 2^127"
    f, e = np.frexp(x)                   # x = f * 2^e, f in [0.5, 1)
    k = np.where(f == 0.5, e - 1, e)     # smallest k with 2^k >= x
    return (k + 127).astype(np.uint8)


def transform_sf(sf, is_activation: bool, pack: bool, ld: int = None) -> np.ndarray:
    """The scale layout the GEMMs require, from FP32 scales given per row:
    activation scales sf [rows][nkb] -> FP32 [nkb][ld] (transposed) or, packed,
    int32 [ceil(nkb/4)][ld]; weight scales sf [nb][nkb] -> FP32 [nb][nkb] (unchanged) or
    int32 [nb][ceil(nkb/4)]. ld >= rows (default rows); entries past `rows` are 0."""
    sf = np.asarray(sf, dtype=np.float32)
    rows, nkb = sf.shape
    if is_activation:
        ld = rows if ld is None else ld
        out_t = ue8m0_pack(ue8m0_from_fp32(sf), axis=1).T if pack else sf.T
        out = np.zeros((out_t.shape[0], ld), dtype=out_t.dtype)
        out[:, :rows] = out_t
        return out
    return ue8m0_pack(ue8m0_from_fp32(sf), axis=1) if pack else sf.copy()


def gemm_nt_ue8m0_packed(A, sa_words, B, sb_words, K: int):
    """Dense NT GEMM with packed UE8M0 scales: sa_words [ceil(nkb/4)][>=M] and sb_words
    [ceil(N/128)][ceil(nkb/4)] (nkb = K / 128), the definition of gemm_nt_ue8m0 on the
    unpacked codes."""
    nkb = K // BLOCK
    return gemm_nt_ue8m0(A, ue8m0_unpack(sa_words, nkb, axis=0), B, ue8m0_unpack(sb_words, nkb, axis=1))


# ------------------------------------------------------------------ D = C + A B^T
# The pages name the GEMMs D = C + A @ B (fp8_gemm_nt computes D = C + A @ B.T; es.news.
# hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout"). With a BF16 D the
# plainest reading is a BF16 C of D's shape added to the scaled sum before the one
# rounding: D = bf16_RNE(C + S).
def gemm_nt_c(A, sa, B, sb, C_bits, rows=None, cols=None):
    """D = C + A B^T. C_bits: BF16 bits [M, N] (or the rows x cols subset when those are
    given). Returns (bf16 bits, float64 C + S)."""
    S = scaled_block_sum(A, sa, B, sb, rows, cols)
    C = np.asarray(C_bits, dtype=np.uint16)
    if rows is not None or cols is not None:
        r = np.arange(C.shape[0]) if rows is None else np.asarray(rows)
        c = np.arange(C.shape[1]) if cols is None else np.asarray(cols)
        C = C[np.ix_(r, c)]
    T = bf16_bits_to_f64(C) + S
    return bf16_bits_rne(T), T


# ------------------------------------------------------ K-grouped TN (weight gradient)
# The pages name a K-grouped contiguous GEMM for the MoE weight-gradient backward:
# M and N fixed, the reduction axis K split into per-expert segments laid end to end
# (k_grouped_fp8_gemm_tn_contiguous; es.news.hada.io/topic?id=19459, "Dense y Grouped
# GEMM"). "TN" is the layout pair of D = A^T B: A stored [K, M] and B stored [K, N],
# K the outer (strided) axis of both ("Interfaz GEMM y restricciones de layout").
# Readings (the pages give no more): each segment's length is a multiple of 128 (the
# alignment of the contiguous layouts); both operands are token-axis activations, so
# each carries one FP32 scale per column per 128-long K block (sa [K/128, M],
# sb [K/128, N]); the output is one FP32 matrix per group, D[g] = C[g] + sum, rounded
# once to FP32, where C[g] is the old D[g] when accumulating and +0 otherwise.
def k_grouped_tn_sum(A, sa, B, sb, k_start, k_len, rows=None, cols=None):
    """S[m, n] = sum over the 128-blocks kb of [k_start, k_start + k_len) of
    P_kb[m, n] * sa[kb, m] * sb[kb, n], P_kb[m, n] = sum_{k in kb} A[k, m] B[k, n] (FP64;
    every P_kb exact). A uint8 [K, M], sa [K/128, >=M], B uint8 [K, N], sb [K/128, >=N]."""
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    assert k_start % BLOCK == 0 and k_len % BLOCK == 0
    rows = np.arange(A.shape[1]) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(B.shape[1]) if cols is None else np.asarray(cols, dtype=np.int64)
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    S = np.zeros((len(rows), len(cols)), dtype=np.float64)
    for k0 in range(k_start, k_start + k_len, BLOCK):
        kb = k0 // BLOCK
        a = decode_e4m3(A[k0:k0 + BLOCK][:, rows])        # [128, m]
        b = decode_e4m3(B[k0:k0 + BLOCK][:, cols])        # [128, n]
        P = a.T @ b                                       # exact block partial
        s = sa[kb, rows].astype(np.float64)[:, None] * sb[kb, cols].astype(np.float64)[None, :]
        S += P * s
    return S


def k_grouped_tn(A, sa, B, sb, ks, D_in=None, rows=None, cols=None):
    """K-grouped TN GEMM: group g covers K rows [sum(ks[:g]), sum(ks[:g+1])).
    D_in: FP32 [G, M, N] (or [G, rows, cols] with a subset) added when accumulating.
    Returns (FP32 [G, ., .], FP64 C + S [G, ., .])."""
    starts = np.concatenate([[0], np.cumsum(np.asarray(ks, dtype=np.int64))])
    T = []
    for g, k_len in enumerate(ks):
        S = k_grouped_tn_sum(A, sa, B, sb, int(starts[g]), int(k_len), rows, cols)
        if D_in is not None:
            S = np.asarray(D_in[g], dtype=np.float32).astype(np.float64) + S
        T.append(S)
    T = np.stack(T) if T else np.zeros((0, 0, 0))
    return T.astype(np.float32), T           # float64 -> float32 rounds to nearest even


# ------------------------------------------------------------ SwiGLU + 1x128 quantisation
# The MoE FFN's step between its two GEMMs is SwiGLU (es.news.hada.io/topic?id=19459,
# "Mega MoE": linear 1, SwiGLU, linear 2); its output is the down projection's A operand,
# quantised 1x128 as above. Reading: the gate+up output row holds gate in its first F
# columns and up in the last F; silu(g) = g * sigmoid(g) = g / (1 + e^-g); padding rows of
# the contiguous layout (m_indices = -1) are zeros.
def swiglu(h: np.ndarray) -> np.ndarray:
    """h [R, 2F] (float32 values) -> the SwiGLU value silu(gate) * up in FP64."""
    h = np.asarray(h, dtype=np.float32).astype(np.float64)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def swiglu_quantize_1x128(h: np.ndarray, m_indices=None):
    """(codes uint8 [R, F], scales float32 [F/128, R], y float32 [R, F]): the SwiGLU value
    rounded once to FP32, padding rows zeroed, then quantize_1x128."""
    y = swiglu(h).astype(np.float32)
    if m_indices is not None:
        y[np.asarray(m_indices)[:y.shape[0]] < 0] = 0.0
    q, s = quantize_1x128(y)
    return q, s, y


# ------------------------------------------------------------------ TN layout (dense)
# The pages list the NT, TN, NN and TT memory layouts of the dense call (es.news.hada.io/
# topic?id=19459, "Interfaz GEMM y restricciones de layout"; fp8_gemm_{nt,nn,tn,tt}).
# TN: A stored [K, M] and B stored [K, N] (K the strided axis of both), D = A^T B. The
# scales keep their logical meaning: one per (m, 128-K block) for A in sa [K/128, >=M],
# one per 128x128 block for B in sb [ceil(N/128), K/128]; BF16 output, one rounding.
def gemm_tn(A_km, sa, B_kn, sb):
    """Dense TN GEMM. Returns (bf16 bits uint16 [M, N], float64 S [M, N])."""
    A = np.asarray(A_km, dtype=np.uint8)
    B = np.asarray(B_kn, dtype=np.uint8)
    K, M = A.shape
    K2, N = B.shape
    assert K == K2 and K % BLOCK == 0
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    S = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // BLOCK):
        a = decode_e4m3(A[kb * BLOCK:(kb + 1) * BLOCK])          # [128, M]
        b = decode_e4m3(B[kb * BLOCK:(kb + 1) * BLOCK])          # [128, N]
        P = a.T @ b                                              # exact block partial
        s = sa[kb, :M].astype(np.float64)[:, None] * sb[np.arange(N) // BLOCK, kb].astype(np.float64)[None, :]
        S += P * s
    return bf16_bits_rne(S), S


# NN: A stored [M, K] (as in NT), B stored [K, N]; TT: A stored [K, M], B stored [N, K] (as
# in NT). Same scales and output as the other layouts.
def _gemm_any(a_rows, b_cols, M, N, K, sa, sb):
    """Shared by gemm_nn / gemm_tt: a_rows(kb) -> decoded A block [M, 128], b_cols(kb) ->
    decoded B block [128, N]."""
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    S = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // BLOCK):
        P = a_rows(kb) @ b_cols(kb)                              # exact block partial
        s = sa[kb, :M].astype(np.float64)[:, None] * sb[np.arange(N) // BLOCK, kb].astype(np.float64)[None, :]
        S += P * s
    return bf16_bits_rne(S), S


def gemm_nn(A_mk, sa, B_kn, sb):
    """Dense NN GEMM D = A B, A [M, K], B [K, N]. Returns (bf16 bits [M, N], float64 S)."""
    A = np.asarray(A_mk, dtype=np.uint8)
    B = np.asarray(B_kn, dtype=np.uint8)
    (M, K), N = A.shape, B.shape[1]
    assert B.shape[0] == K and K % BLOCK == 0
    return _gemm_any(lambda kb: decode_e4m3(A[:, kb * BLOCK:(kb + 1) * BLOCK]),
                     lambda kb: decode_e4m3(B[kb * BLOCK:(kb + 1) * BLOCK]), M, N, K, sa, sb)


def gemm_tt(A_km, sa, B_nk, sb):
    """Dense TT GEMM D = A^T B^T, A [K, M], B [N, K]. Returns (bf16 bits [M, N], float64 S)."""
    A = np.asarray(A_km, dtype=np.uint8)
    B = np.asarray(B_nk, dtype=np.uint8)
    (K, M), N = A.shape, B.shape[0]
    assert B.shape[1] == K and K % BLOCK == 0
    return _gemm_any(lambda kb: decode_e4m3(A[kb * BLOCK:(kb + 1) * BLOCK]).T,
                     lambda kb: decode_e4m3(B[:, kb * BLOCK:(kb + 1) * BLOCK]).T, M, N, K, sa, sb)
