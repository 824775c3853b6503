"""FP8 (e4m3) block-scaled NT GEMM for AMD MI355X: Python binding of libfp8gemm.so.

A thin ctypes layer over the C ABI declared in include/fp8gemm.h. It only
marshals torch tensors (device pointers, strides, the current HIP stream) into
the library's entry points; every step of the computation runs in the library's
HIP kernels. PyTorch supplies device memory and streams. Importing works without
a GPU; calling a GEMM needs the built library and a gfx950 device, and raises
otherwise (there is no fallback path).

Entry points (names follow the DeepGEMM pages' interface, bquan.live post
9429818 "¿Cómo usarlo?" and es.news.hada.io/topic?id=19459 "Dense y Grouped
GEMM"):
  fp8_gemm_nt                       D = A . B^T
  fp8_grouped_gemm_nt_contiguous    experts concatenated along M, m_indices per row
  fp8_grouped_gemm_nt_masked        [G, M_max, K] input, masked_m[g] live rows
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "fp8_gemm_nt", "fp8_gemm_nt_noalloc", "noalloc_scratch_bytes", "fp8_gemm_nt_ue8m0", "fp8_grouped_gemm_nt_contiguous", "fp8_grouped_gemm_nt_masked",
    "workspace_size", "make_workspace", "query_config", "force_config", "set_num_cus",
    "get_num_cus", "get_mk_alignment_for_contiguous_layout", "scale_ld", "num_tiles",
    "status_string", "lib", "LIB_PATH", "KIND_DENSE", "KIND_CONTIGUOUS", "KIND_MASKED", "KIND_LAYOUT", "quantize_1x128",
    "Fp8GemmError",
]

# FP8GEMM_LIBRARY names another build of the same library (the host-sanitizer build of
# build.py); by default the one built in this directory
LIB_PATH = os.environ.get("FP8GEMM_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libfp8gemm.so")
KIND_DENSE, KIND_CONTIGUOUS, KIND_MASKED, KIND_LAYOUT = 0, 1, 2, 3


class Fp8GemmError(RuntimeError):
    pass


class Config(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("split_k", ctypes.c_int),
                ("grid", ctypes.c_int), ("num_units", ctypes.c_int), ("full_tiles", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None
_P, _I64, _INT, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "fp8_gemm_nt": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_nt_ue8m0": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_nt_c": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_contiguous_c": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_masked_c": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P, _INT, _INT, _INT, _INT, _INT, _P, _SZ,
               _P]),
    "fp8_grouped_gemm_nt_contiguous": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_masked": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_contiguous_ue8m0": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_masked_ue8m0": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tn": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_nn": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tt": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tn_c": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_nn_c": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tt_c": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tn_ue8m0": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_nn_ue8m0": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_gemm_tt_ue8m0": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_k_grouped_gemm_tn_contiguous": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _INT, _INT, _INT, _INT, _P]),
    "fp8_k_grouped_gemm_tn_contiguous_ue8m0": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _INT, _INT, _INT, _INT, _P]),
    "fp8_gemm_workspace_size": (_SZ, [_INT, _INT, _INT, _INT, _INT, _INT]),
    "fp8_gemm_nt_noalloc": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P]),
    "fp8_gemm_nt_ue8m0_packed": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_contiguous_ue8m0_packed": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_grouped_gemm_nt_masked_ue8m0_packed": (
        _INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _INT, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "fp8_transform_sf_into_required_layout": (_INT, [_P, _I64, _INT, _INT, _INT, _INT, _P, _I64, _P]),
    "fp8_gemm_noalloc_scratch_bytes": (_SZ, []),
    "fp8_quantize_1x128": (_INT, [_P, _I64, _INT, _P, _I64, _P, _I64, _INT, _INT, _P]),
    "fp8_swiglu_quantize_1x128": (_INT, [_P, _I64, _INT, _P, _P, _I64, _P, _I64, _INT, _INT, _P]),
    "fp8_gemm_query_config": (_INT, [_INT, _INT, _INT, _INT, _INT, _INT, _SZ, ctypes.POINTER(Config)]),
    "fp8_gemm_force_config": (_INT, [ctypes.POINTER(Config)]),
    "fp8_gemm_set_num_cus": (_INT, [_INT]),
    "fp8_gemm_get_num_cus": (_INT, []),
    "fp8_gemm_get_mk_alignment_for_contiguous_layout": (_INT, []),
    "fp8_gemm_scale_ld": (_I64, [_I64]),
    "fp8_gemm_num_tiles": (_I64, [_I64, _I64, _INT, _INT]),
    "fp8_gemm_status_string": (ctypes.c_char_p, [_INT]),
}


def lib():
    """The loaded libfp8gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with moe_grouped_gemm_fp32_amd/build.py "
                              "(or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fp8_gemm_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise Fp8GemmError(f"{what}: {status_string(status)} (status {status})")


def _bytes_view(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"FP8 operand must be uint8 (e4m3 bytes) or float8_e4m3fn, got {t.dtype}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _ws(workspace):
    if workspace is None:
        return ctypes.c_void_p(0), 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def _common(A, sa, B, sb, D, rows_dim):
    A, B = _bytes_view(A), _bytes_view(B)
    dev = D.device
    _require(dev.type == "cuda", "tensors must live on a GPU")
    for name, t in (("A", A), ("sa", sa), ("B", B), ("sb", sb), ("D", D)):
        _require(t.device == dev, f"{name} is on {t.device}, D on {dev}")
        _require(t.stride(-1) == 1, f"{name} must have a unit inner stride")
    _require(sa.dtype == torch.float32 and sb.dtype == torch.float32, "scales must be float32")
    _require(D.dtype == torch.bfloat16, "D must be bfloat16")
    _require(sb.is_contiguous(), "sb must be contiguous")
    return A, B, dev


def _check_c(C, D):
    """The optional addend of D = C + A B^T: bfloat16 with D's shape, unit inner stride,
    on D's device (it may be D itself)."""
    _require(C.dtype == torch.bfloat16 and tuple(C.shape) == tuple(D.shape) and C.device == D.device
             and C.stride(-1) == 1, "C must be bfloat16 with D's shape and a unit inner stride")


def fp8_gemm_nt(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, stream=None, C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """D[M, N] = A[M, K] . B[N, K]^T with 1x128 (sa [K/128, ld_sa]) and 128x128 (sb) scales.

    A, B: e4m3 bytes (uint8 or float8_e4m3fn), row-major with unit inner stride.
    sa: float32 [K/128, ld_sa], row stride ld_sa >= M. sb: float32 [ceil(N/128), K/128].
    D: bfloat16 [M, N] (written in place and returned). workspace: optional
    zero-initialised uint8 device buffer enabling split-K (see make_workspace).
    C: optional bfloat16 addend, D = C + A B^T (fp8_gemm_nt_c); may be D itself.
    """
    A, B, dev = _common(A, sa, B, sb, D, 0)
    M, K = A.shape
    N = B.shape[0]
    _require(B.shape[1] == K and tuple(D.shape) == (M, N), "shape mismatch")
    _require(sa.dim() == 2 and sa.shape[0] == K // 128 and _ld(sa) >= M, "sa must be [K/128, >=M]")
    _require(tuple(sb.shape) == ((N + 127) // 128, K // 128), "sb must be [ceil(N/128), K/128]")
    wp, wb = _ws(workspace)
    if C is not None:
        _check_c(C, D)
        st = lib().fp8_gemm_nt_c(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                                 _ptr(C), C.stride(0), _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
        _check(st, "fp8_gemm_nt_c")
        return D
    st = lib().fp8_gemm_nt(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                           _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
    _check(st, "fp8_gemm_nt")
    return D


def fp8_gemm_nt_noalloc(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """fp8_gemm_nt without a workspace argument, for callers that cannot allocate: the
    split-K scratch is the library's own per-device array (noalloc_scratch_bytes()).
    Calls that overlap in time on one GPU must not be issued (they share the scratch)."""
    A, B, dev = _common(A, sa, B, sb, D, 0)
    M, K = A.shape
    N = B.shape[0]
    _require(B.shape[1] == K and tuple(D.shape) == (M, N), "shape mismatch")
    _require(sa.dim() == 2 and sa.shape[0] == K // 128 and _ld(sa) >= M, "sa must be [K/128, >=M]")
    _require(tuple(sb.shape) == ((N + 127) // 128, K // 128), "sb must be [ceil(N/128), K/128]")
    st = lib().fp8_gemm_nt_noalloc(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                                   _ptr(D), D.stride(0), M, N, K, _stream(dev, stream))
    _check(st, "fp8_gemm_nt_noalloc")
    return D


def noalloc_scratch_bytes() -> int:
    return int(lib().fp8_gemm_noalloc_scratch_bytes())


def fp8_gemm_nt_ue8m0(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp8_gemm_nt for UE8M0 scale factors: sa and sb (same shapes and layouts) hold
    exact powers of two; their exponents feed the block-scaled MFMA directly."""
    A, B, dev = _common(A, sa, B, sb, D, 0)
    M, K = A.shape
    N = B.shape[0]
    _require(B.shape[1] == K and tuple(D.shape) == (M, N), "shape mismatch")
    _require(sa.dim() == 2 and sa.shape[0] == K // 128 and _ld(sa) >= M, "sa must be [K/128, >=M]")
    _require(tuple(sb.shape) == ((N + 127) // 128, K // 128), "sb must be [ceil(N/128), K/128]")
    wp, wb = _ws(workspace)
    st = lib().fp8_gemm_nt_ue8m0(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                                 _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
    _check(st, "fp8_gemm_nt_ue8m0")
    return D


def _ld(t: torch.Tensor, dim: int = 0) -> int:
    """Row stride of `t` along `dim` in elements; a dimension of size 1 may carry any stride,
    so then the rows' length (the product of the later sizes) is taken."""
    if t.shape[dim] > 1:
        return t.stride(dim)
    n = 1
    for d in t.shape[dim + 1:]:
        n *= d
    return n


def _packed_common(A, sa, B, sb, D):
    A, B = _bytes_view(A), _bytes_view(B)
    dev = D.device
    _require(dev.type == "cuda", "tensors must live on a GPU")
    for name, t in (("A", A), ("sa", sa), ("B", B), ("sb", sb), ("D", D)):
        _require(t.device == dev, f"{name} is on {t.device}, D on {dev}")
        _require(t.stride(-1) == 1, f"{name} must have a unit inner stride")
    _require(sa.dtype == torch.int32 and sb.dtype == torch.int32, "packed UE8M0 scales must be int32 words")
    _require(D.dtype == torch.bfloat16, "D must be bfloat16")
    _require(sb.is_contiguous(), "sb must be contiguous")
    return A, B, dev


def fp8_gemm_nt_ue8m0_packed(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp8_gemm_nt with packed UE8M0 scales: sa int32 [ceil(K/512), ld_sa >= M] (word w of
    row m holds the codes of K blocks 4w..4w+3 in bytes 0..3), sb int32 [ceil(N/128),
    ceil(K/512)] (see transform_sf_into_required_layout)."""
    A, B, dev = _packed_common(A, sa, B, sb, D)
    M, K = A.shape
    N = B.shape[0]
    nkw = (K // 128 + 3) // 4
    _require(B.shape[1] == K and tuple(D.shape) == (M, N), "shape mismatch")
    _require(sa.dim() == 2 and sa.shape[0] == nkw and _ld(sa) >= M, "sa must be [ceil(K/512), >=M]")
    _require(tuple(sb.shape) == ((N + 127) // 128, nkw), "sb must be [ceil(N/128), ceil(K/512)]")
    wp, wb = _ws(workspace)
    st = lib().fp8_gemm_nt_ue8m0_packed(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0),
                                        _ptr(sb), _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
    _check(st, "fp8_gemm_nt_ue8m0_packed")
    return D


def fp8_grouped_gemm_nt_contiguous_ue8m0_packed(A, sa, B, sb, D, m_indices, workspace=None, stream=None):
    """The contiguous grouped GEMM with packed UE8M0 scales: sa int32 [ceil(K/512),
    >=M_total], sb int32 [G, ceil(N/128), ceil(K/512)]."""
    A, B, dev = _packed_common(A, sa, B, sb, D)
    Mt, K = A.shape
    G, N, K2 = B.shape
    nkw = (K // 128 + 3) // 4
    _require(K2 == K and tuple(D.shape) == (Mt, N) and B.is_contiguous(), "shape mismatch")
    _require(sa.dim() == 2 and sa.shape[0] == nkw and _ld(sa) >= Mt, "sa must be [ceil(K/512), >=M_total]")
    _require(tuple(sb.shape) == (G, (N + 127) // 128, nkw), "sb must be [G, ceil(N/128), ceil(K/512)]")
    _require(m_indices.dtype == torch.int32 and m_indices.numel() == Mt and m_indices.device == dev
             and m_indices.is_contiguous(), "m_indices must be a contiguous int32 [M_total] device tensor")
    wp, wb = _ws(workspace)
    st = lib().fp8_grouped_gemm_nt_contiguous_ue8m0_packed(
        _ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(1), _ptr(sb), _ptr(D), D.stride(0),
        _ptr(m_indices), Mt, N, K, G, wp, wb, _stream(dev, stream))
    _check(st, "fp8_grouped_gemm_nt_contiguous_ue8m0_packed")
    return D


def fp8_grouped_gemm_nt_masked_ue8m0_packed(A, sa, B, sb, D, masked_m, expected_m: int, stream=None):
    """The masked grouped GEMM with packed UE8M0 scales: sa int32 [G, ceil(K/512),
    >=M_max], sb int32 [G, ceil(N/128), ceil(K/512)]."""
    A, B, dev = _packed_common(A, sa, B, sb, D)
    G, M_max, K = A.shape
    G2, N, K2 = B.shape
    nkw = (K // 128 + 3) // 4
    _require(G2 == G and K2 == K and tuple(D.shape) == (G, M_max, N), "shape mismatch")
    for name, t in (("A", A), ("B", B), ("D", D), ("sa", sa)):
        _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(sa.dim() == 3 and sa.shape[0] == G and sa.shape[1] == nkw and sa.shape[2] >= M_max,
             "sa must be [G, ceil(K/512), >=M_max]")
    _require(tuple(sb.shape) == (G, (N + 127) // 128, nkw), "sb must be [G, ceil(N/128), ceil(K/512)]")
    _require(masked_m.dtype == torch.int32 and masked_m.numel() == G and masked_m.device == dev
             and masked_m.is_contiguous(), "masked_m must be a contiguous int32 [G] device tensor")
    st = lib().fp8_grouped_gemm_nt_masked_ue8m0_packed(
        _ptr(A), A.stride(1), _ptr(sa), _ld(sa, 1), _ptr(B), B.stride(1), _ptr(sb), _ptr(D), D.stride(1),
        _ptr(masked_m), G, M_max, N, K, int(expected_m), None, 0, _stream(dev, stream))
    _check(st, "fp8_grouped_gemm_nt_masked_ue8m0_packed")
    return D


def transform_sf_into_required_layout(sf: torch.Tensor, is_activation: bool, pack: bool, ld: Optional[int] = None,
                                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """FP32 scale factors given per row, sf [rows, nkb] (activation: rows = M; weight:
    rows = ceil(N/128)), into the layout the GEMMs read, computed by
    fp8_transform_sf_into_required_layout: activation -> [nkb, ld] FP32 or [ceil(nkb/4),
    ld] int32 packed UE8M0 (ld >= rows, default scale_ld(rows)); weight -> [rows, nkb]
    FP32 or [rows, ceil(nkb/4)] int32 packed."""
    _require(sf.device.type == "cuda" and sf.dtype == torch.float32 and sf.dim() == 2 and sf.stride(-1) == 1,
             "sf must be a 2-D float32 GPU tensor with unit inner stride")
    rows, nkb = sf.shape
    cols = (nkb + 3) // 4 if pack else nkb
    dt = torch.int32 if pack else torch.float32
    if out is None:
        if is_activation:
            out = torch.zeros(cols, scale_ld(rows) if ld is None else ld, dtype=dt, device=sf.device)
        else:
            out = torch.zeros(rows, cols, dtype=dt, device=sf.device)
    _require(out.dtype == dt and out.dim() == 2 and out.stride(-1) == 1 and out.device == sf.device,
             "out has the wrong type or layout")
    _require(out.shape[0] == (cols if is_activation else rows), "out has the wrong number of rows")
    st = lib().fp8_transform_sf_into_required_layout(_ptr(sf), sf.stride(0), rows, nkb, int(bool(is_activation)),
                                                     int(bool(pack)), _ptr(out), out.stride(0),
                                                     _stream(sf.device, stream))
    _check(st, "fp8_transform_sf_into_required_layout")
    return out


QUANT_BF16, QUANT_FP32 = 0, 1  # fp8_quantize_1x128 input types


def quantize_1x128(X: torch.Tensor, Q: Optional[torch.Tensor] = None, sa: Optional[torch.Tensor] = None,
                   stream=None):
    """1x128 activation quantisation of X [M, K] (bfloat16 or float32, unit inner
    stride) -> (Q e4m3 bytes [M, K] uint8, sa float32 [K/128, ld_sa]), the A operand
    layout of the GEMMs: per row and 128-column block s = amax/448 (1 if zero) and
    q = e4m3_rne(x / s), computed by fp8_quantize_1x128. Q and sa may be given
    (written in place); by default Q is [M, K] and sa is [K/128, scale_ld(M)]."""
    _require(X.device.type == "cuda" and X.dim() == 2 and X.stride(-1) == 1, "X must be a 2-D GPU tensor")
    _require(X.dtype in (torch.bfloat16, torch.float32), "X must be bfloat16 or float32")
    M, K = X.shape
    _require(K % 128 == 0, "K must be a multiple of 128")
    if Q is None:
        Q = torch.empty(M, K, dtype=torch.uint8, device=X.device)
    if sa is None:
        sa = torch.empty(K // 128, scale_ld(M), dtype=torch.float32, device=X.device)
    Q = _bytes_view(Q)
    _require(tuple(Q.shape) == (M, K) and Q.stride(-1) == 1 and Q.device == X.device, "Q must be [M, K]")
    _require(sa.dtype == torch.float32 and sa.shape[0] == K // 128 and sa.stride(-1) == 1 and _ld(sa) >= M,
             "sa must be float32 [K/128, >=M]")
    st = lib().fp8_quantize_1x128(_ptr(X), X.stride(0), QUANT_BF16 if X.dtype == torch.bfloat16 else QUANT_FP32,
                                  _ptr(Q), Q.stride(0), _ptr(sa), _ld(sa), M, K, _stream(X.device, stream))
    _check(st, "fp8_quantize_1x128")
    return Q, sa


def swiglu_quantize_1x128(H: torch.Tensor, m_indices: Optional[torch.Tensor] = None, Q: Optional[torch.Tensor] = None,
                          sa: Optional[torch.Tensor] = None, stream=None):
    """SwiGLU of a gate+up output fused with the 1x128 quantisation: H [M, 2F] (bfloat16 or
    float32, gate in the first F columns) -> (Q e4m3 bytes [M, F], sa float32 [F/128,
    ld_sa]) of y = silu(gate) * up, computed by fp8_swiglu_quantize_1x128; rows whose
    m_indices entry is -1 quantise as zeros."""
    _require(H.device.type == "cuda" and H.dim() == 2 and H.stride(-1) == 1, "H must be a 2-D GPU tensor")
    _require(H.dtype in (torch.bfloat16, torch.float32), "H must be bfloat16 or float32")
    M, F2 = H.shape
    F = F2 // 2
    _require(F2 % 2 == 0 and F % 128 == 0, "H must be [M, 2F] with F a multiple of 128")
    if Q is None:
        Q = torch.empty(M, F, dtype=torch.uint8, device=H.device)
    if sa is None:
        sa = torch.empty(F // 128, scale_ld(M), dtype=torch.float32, device=H.device)
    Q = _bytes_view(Q)
    _require(tuple(Q.shape) == (M, F) and Q.stride(-1) == 1 and Q.device == H.device, "Q must be [M, F]")
    _require(sa.dtype == torch.float32 and sa.shape[0] == F // 128 and sa.stride(-1) == 1 and _ld(sa) >= M,
             "sa must be float32 [F/128, >=M]")
    if m_indices is not None:
        _require(m_indices.dtype == torch.int32 and m_indices.numel() >= M and m_indices.device == H.device,
                 "m_indices must be int32 [>=M] on H's device")
    st = lib().fp8_swiglu_quantize_1x128(_ptr(H), H.stride(0), QUANT_BF16 if H.dtype == torch.bfloat16 else QUANT_FP32,
                                         _ptr(m_indices), _ptr(Q), Q.stride(0), _ptr(sa), _ld(sa), M, F,
                                         _stream(H.device, stream))
    _check(st, "fp8_swiglu_quantize_1x128")
    return Q, sa


def fp8_grouped_gemm_nt_contiguous(A, sa, B, sb, D, m_indices, workspace=None, stream=None, ue8m0=False, C=None):
    """M-grouped contiguous GEMM: row r of D = A[r] . B[m_indices[r]]^T; rows with -1 untouched.

    A [M_total, K]; sa float32 [K/128, >=M_total]; B [G, N, K]; sb [G, ceil(N/128), K/128];
    D bfloat16 [M_total, N]; m_indices int32 [M_total] on the device.
    ue8m0: the scales are exact powers of two (fp8_grouped_gemm_nt_contiguous_ue8m0).
    C: optional bfloat16 addend [M_total, N], D = C + A B^T on live rows (..._contiguous_c).
    """
    A, B, dev = _common(A, sa, B, sb, D, 0)
    Mt, K = A.shape
    G, N, K2 = B.shape
    _require(K2 == K and tuple(D.shape) == (Mt, N), "shape mismatch")
    _require(B.is_contiguous(), "B must be contiguous [G, N, K]")
    _require(sa.dim() == 2 and sa.shape[0] == K // 128 and _ld(sa) >= Mt, "sa must be [K/128, >=M_total]")
    _require(tuple(sb.shape) == (G, (N + 127) // 128, K // 128), "sb must be [G, ceil(N/128), K/128]")
    _require(m_indices.dtype == torch.int32 and m_indices.numel() == Mt and m_indices.device == dev
             and m_indices.is_contiguous(), "m_indices must be a contiguous int32 [M_total] device tensor")
    wp, wb = _ws(workspace)
    if C is not None:
        _require(not ue8m0, "C is supported with FP32 scales")
        _check_c(C, D)
        st = lib().fp8_grouped_gemm_nt_contiguous_c(
            _ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(1), _ptr(sb), _ptr(C), C.stride(0),
            _ptr(D), D.stride(0), _ptr(m_indices), Mt, N, K, G, wp, wb, _stream(dev, stream))
        _check(st, "fp8_grouped_gemm_nt_contiguous_c")
        return D
    name = "fp8_grouped_gemm_nt_contiguous_ue8m0" if ue8m0 else "fp8_grouped_gemm_nt_contiguous"
    st = getattr(lib(), name)(
        _ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(1), _ptr(sb), _ptr(D), D.stride(0),
        _ptr(m_indices), Mt, N, K, G, wp, wb, _stream(dev, stream))
    _check(st, name)
    return D


def fp8_grouped_gemm_nt_masked(A, sa, B, sb, D, masked_m, expected_m: int, workspace=None, stream=None,
                               ue8m0=False, C=None):
    """M-grouped masked GEMM: D[g, m] = A[g, m] . B[g]^T for m < masked_m[g]; other rows untouched.

    A [G, M_max, K]; sa float32 [G, K/128, ld_sa >= M_max]; B [G, N, K];
    sb [G, ceil(N/128), K/128]; D bfloat16 [G, M_max, N]; masked_m int32 [G] on
    the device (never read by the host); expected_m is a tiling hint.
    ue8m0: the scales are exact powers of two (fp8_grouped_gemm_nt_masked_ue8m0).
    C: optional bfloat16 addend [G, M_max, N] (contiguous), D = C + A B^T on live rows.
    """
    A, B, dev = _common(A, sa, B, sb, D, 1)
    G, M_max, K = A.shape
    G2, N, K2 = B.shape
    _require(G2 == G and K2 == K and tuple(D.shape) == (G, M_max, N), "shape mismatch")
    for name, t in (("A", A), ("B", B), ("D", D), ("sa", sa)):
        _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(sa.dim() == 3 and sa.shape[0] == G and sa.shape[1] == K // 128 and sa.shape[2] >= M_max,
             "sa must be [G, K/128, >=M_max]")
    _require(tuple(sb.shape) == (G, (N + 127) // 128, K // 128), "sb must be [G, ceil(N/128), K/128]")
    _require(masked_m.dtype == torch.int32 and masked_m.numel() == G and masked_m.device == dev
             and masked_m.is_contiguous(), "masked_m must be a contiguous int32 [G] device tensor")
    wp, wb = _ws(workspace)
    if C is not None:
        _require(not ue8m0, "C is supported with FP32 scales")
        _check_c(C, D)
        _require(C.is_contiguous(), "C must be contiguous")
        st = lib().fp8_grouped_gemm_nt_masked_c(
            _ptr(A), A.stride(1), _ptr(sa), _ld(sa, 1), _ptr(B), B.stride(1), _ptr(sb), _ptr(C), C.stride(1),
            _ptr(D), D.stride(1), _ptr(masked_m), G, M_max, N, K, int(expected_m), wp, wb, _stream(dev, stream))
        _check(st, "fp8_grouped_gemm_nt_masked_c")
        return D
    name = "fp8_grouped_gemm_nt_masked_ue8m0" if ue8m0 else "fp8_grouped_gemm_nt_masked"
    st = getattr(lib(), name)(
        _ptr(A), A.stride(1), _ptr(sa), _ld(sa, 1), _ptr(B), B.stride(1), _ptr(sb), _ptr(D), D.stride(1),
        _ptr(masked_m), G, M_max, N, K, int(expected_m), wp, wb, _stream(dev, stream))
    _check(st, name)
    return D


def _dense_layout(name, a_kmajor, b_kmajor, A, sa, B, sb, D, stream, C=None, workspace=None):
    A, B = _bytes_view(A), _bytes_view(B)
    dev = D.device
    _require(dev.type == "cuda" and all(t.device == dev for t in (A, sa, B, sb)), "tensors must share one GPU")
    _require(A.dim() == 2 and B.dim() == 2 and A.stride(-1) == 1 and B.stride(-1) == 1,
             "A and B must be 2-D with unit inner stride")
    _require(D.dtype == torch.bfloat16 and D.dim() == 2 and D.stride(-1) == 1, "D must be bfloat16 [M, N]")
    M, N = D.shape
    K = A.shape[0] if a_kmajor else A.shape[1]
    _require((A.shape[1] >= M) if a_kmajor else (A.shape[0] == M), "A does not match D's rows")
    _require((B.shape[0] == K and B.shape[1] >= N) if b_kmajor else (B.shape[1] == K and B.shape[0] == N),
             "B does not match K and D's columns")
    _require(sa.dtype == torch.float32 and sa.shape[0] == K // 128 and sa.stride(-1) == 1 and sa.shape[1] >= M,
             "sa must be float32 [K/128, >=M]")
    _require(sb.dtype == torch.float32 and sb.is_contiguous() and sb.numel() == ((N + 127) // 128) * (K // 128),
             "sb must be contiguous float32 [ceil(N/128), K/128]")
    wp, wb = _ws(workspace)
    if C is not None:
        _check_c(C, D)
        name = name + "_c"
        st = getattr(lib(), name)(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                                  _ptr(C), C.stride(0), _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
    else:
        st = getattr(lib(), name)(_ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb),
                                  _ptr(D), D.stride(0), M, N, K, wp, wb, _stream(dev, stream))
    _check(st, name)
    return D


def fp8_gemm_tn(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor, stream=None,
                ue8m0: bool = False, C: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense TN GEMM: D [M, N] (bfloat16) = A^T B with A [K, M] and B [K, N] (e4m3 bytes,
    K-major, unit inner stride), sa [K/128, >=M] and sb [ceil(N/128), K/128] as for
    fp8_gemm_nt. workspace: optional split-K workspace (make_workspace(KIND_LAYOUT, M, N,
    K)), used by the few-row shapes."""
    _require(not (ue8m0 and C is not None), "the UE8M0 form takes no C")
    return _dense_layout("fp8_gemm_tn" + ("_ue8m0" if ue8m0 else ""), True, True, A, sa, B, sb, D, stream, C,
                         workspace)


def fp8_gemm_nn(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor, stream=None,
                ue8m0: bool = False, C: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense NN GEMM: D = A B with A [M, K] (as for fp8_gemm_nt) and B [K, N] (K-major)."""
    _require(not (ue8m0 and C is not None), "the UE8M0 form takes no C")
    return _dense_layout("fp8_gemm_nn" + ("_ue8m0" if ue8m0 else ""), False, True, A, sa, B, sb, D, stream, C,
                         workspace)


def fp8_gemm_tt(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor, stream=None,
                ue8m0: bool = False, C: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense TT GEMM: D = A^T B^T with A [K, M] (K-major) and B [N, K] (as for fp8_gemm_nt)."""
    _require(not (ue8m0 and C is not None), "the UE8M0 form takes no C")
    return _dense_layout("fp8_gemm_tt" + ("_ue8m0" if ue8m0 else ""), True, False, A, sa, B, sb, D, stream, C,
                         workspace)


MAX_K_GROUPS = 256  # groups per fp8_k_grouped_gemm_tn_contiguous call


def k_grouped_fp8_gemm_tn_contiguous(A, sa, B, sb, D, ks, accumulate: bool = False, stream=None, ue8m0=False):
    """K-grouped TN GEMM (MoE weight gradient): for each group g, whose K rows are
    [sum(ks[:g]), sum(ks[:g+1])) of A [K, M] and B [K, N] (e4m3 bytes, K-major),
    D[g] (+)= sum_kb P_kb * sa[kb, m] * sb[kb, n] with sa [K/128, >=M] and sb [K/128, >=N]
    (one FP32 scale per column per 128-row block). D is float32 [G, M, N] (unit inner
    stride); accumulate adds into its old values. ks: per-group K lengths, multiples of
    128 (a list, or a CPU int tensor). ue8m0: every scale is an exact power of two (UE8M0
    values held as FP32), applied by the block-scaled MFMA."""
    A, B = _bytes_view(A), _bytes_view(B)
    dev = D.device
    ks = [int(k) for k in (ks.tolist() if isinstance(ks, torch.Tensor) else ks)]
    G = len(ks)
    _require(dev.type == "cuda" and all(t.device == dev for t in (A, sa, B, sb)), "tensors must share one GPU")
    _require(A.dim() == 2 and B.dim() == 2 and A.stride(-1) == 1 and B.stride(-1) == 1,
             "A and B must be 2-D [K, M] / [K, N] with unit inner stride")
    _require(D.dtype == torch.float32 and D.dim() == 3 and D.shape[0] == G and D.stride(-1) == 1,
             "D must be float32 [G, M, N] with unit inner stride")
    _require(sa.dtype == torch.float32 and sb.dtype == torch.float32 and sa.stride(-1) == 1 and sb.stride(-1) == 1,
             "sa and sb must be float32 with unit inner stride")
    M, N = D.shape[1], D.shape[2]
    K = sum(ks)
    _require(A.shape[0] == K and B.shape[0] == K and A.shape[1] >= M and B.shape[1] >= N,
             "A must be [sum(ks), >=M] and B [sum(ks), >=N]")
    _require(sa.shape[0] == K // 128 and sb.shape[0] == K // 128 and sa.shape[1] >= M and sb.shape[1] >= N,
             "sa must be [K/128, >=M] and sb [K/128, >=N]")
    ks_arr = (ctypes.c_int32 * max(G, 1))(*ks)
    name = "fp8_k_grouped_gemm_tn_contiguous_ue8m0" if ue8m0 else "fp8_k_grouped_gemm_tn_contiguous"
    st = getattr(lib(), name)(
        _ptr(A), A.stride(0), _ptr(sa), _ld(sa), _ptr(B), B.stride(0), _ptr(sb), sb.stride(0),
        _ptr(D), D.stride(1), D.stride(0), ctypes.cast(ks_arr, ctypes.c_void_p), G, M, N, int(bool(accumulate)),
        _stream(dev, stream))
    _check(st, name)
    return D


def workspace_size(kind: int, M: int, N: int, K: int, G: int = 1, expected_m: int = 0) -> int:
    return int(lib().fp8_gemm_workspace_size(kind, M, N, K, G, expected_m))


def make_workspace(kind: int, M: int, N: int, K: int, G: int = 1, expected_m: int = 0, device="cuda"):
    """Zero-filled split-K workspace for calls of these sizes (None if never needed)."""
    n = workspace_size(kind, M, N, K, G, expected_m)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def query_config(kind: int, M: int, N: int, K: int, G: int = 1, expected_m: int = 0,
                 workspace_bytes: int = 1 << 62) -> dict:
    cfg = Config()
    _check(lib().fp8_gemm_query_config(kind, M, N, K, G, expected_m, workspace_bytes, ctypes.byref(cfg)),
           "fp8_gemm_query_config")
    return cfg.as_dict()


@contextlib.contextmanager
def force_config(block_m: int, block_n: int, split_k: int = 1, full_tiles: int = 0):
    """Context manager forcing a tile configuration (tests and tuning); the first
    `full_tiles` tiles are computed whole, the others split `split_k` ways."""
    cfg = Config(block_m, block_n, split_k, 0, 0, full_tiles)
    _check(lib().fp8_gemm_force_config(ctypes.byref(cfg)), "fp8_gemm_force_config")
    try:
        yield
    finally:
        lib().fp8_gemm_force_config(None)


def set_num_cus(n: int) -> None:
    lib().fp8_gemm_set_num_cus(int(n))


def get_num_cus() -> int:
    return int(lib().fp8_gemm_get_num_cus())


def get_mk_alignment_for_contiguous_layout() -> int:
    return int(lib().fp8_gemm_get_mk_alignment_for_contiguous_layout())


def scale_ld(rows: int) -> int:
    return int(lib().fp8_gemm_scale_ld(rows))


def num_tiles(M: int, N: int, block_m: int, block_n: int) -> int:
    return int(lib().fp8_gemm_num_tiles(M, N, block_m, block_n))
