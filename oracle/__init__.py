"""CPU oracle (test infrastructure only; see fp8_gemm_oracle.py)."""
from .fp8_gemm_oracle import (  # noqa: F401
    BLOCK, E4M3_TABLE, decode_e4m3, bf16_bits_rne, bf16_bits_to_f64, scaled_block_sum,
    gemm_nt, gemm_nt_sampled, grouped_contiguous, grouped_masked, e4m3_rne_codes, quantize_1x128,
    ue8m0_decode, gemm_nt_ue8m0, gemm_nt_c, ue8m0_unpack, ue8m0_pack, ue8m0_from_fp32, transform_sf,
    gemm_nt_ue8m0_packed,
    k_grouped_tn_sum, k_grouped_tn, swiglu, swiglu_quantize_1x128, gemm_tn, gemm_nn, gemm_tt,
)
