// Device code of libfp8gemm's 1x128 activation quantisation: FP32 or BF16 rows to
// e4m3 codes plus one FP32 scale per row per 128-wide K block, written K-block-major
// [K/128][ld_sa] -- the operand layout of the GEMMs (one scale per row per 128-K
// block: GeekNews topic 19444, intro; the pages leave the conversion itself to the
// user, es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout").
//
// Per row and block, in FP32 with IEEE round-to-nearest-even operations:
//     s = amax(|x|) / 448   (s = 1 when that is 0),   q = e4m3_rne(x / s)
// The division is the correctly rounded one (not a reciprocal multiply), and the
// conversion is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even); a
// quotient can exceed 448 only by the rounding of x / s and then still rounds to 448.
//
// HBM-bound elementwise work: no LDS, no matrix unit. A wave takes four rows of one
// 128-column block; the 16 lanes of a row hold 8 consecutive elements each, so every
// load instruction reads whole lines and every code store writes 128 contiguous bytes
// per row. The block maximum is reduced across those 16 lanes with shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

template <typename T>  // uint16_t: BF16 bits; float
__device__ __forceinline__ void load8(const T* src, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
    x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  }
}

// SwiGLU value of one element, y = silu(g) * u with silu(g) = g / (1 + exp(-g)),
// evaluated in FP64 and rounded once to FP32: exp within an FP64 ulp or so, 1 / (1 + e)
// from the hardware reciprocal and two Newton steps (an ulp or two; 0 when exp(-g)
// overflows), so the FP64 value is within a few FP64 ulps of the exact one and the result
// is the FP32 value nearest the exact y unless that lies within ~2^-27 of an FP32 ulp of
// a rounding midpoint.
__device__ __forceinline__ float swiglu_fp64(float g, float u) {
  const double gd = g;
  const double d = 1.0 + exp(-gd);
  double r = __builtin_amdgcn_rcp(d);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  r = d < __builtin_huge_val() ? r : 0.0;  // the Newton steps turn 1 / inf into NaN
  return (float)(gd * (double)u * r);
}

// SWIGLU instances quantise y = silu(gate) * up of a row [gate (F) | up (F)] (the MoE
// down projection's input): gate at column k, up at column F + k, y from swiglu_fp64,
// so every decision is that of the FP32 value nearest the exact y (the oracle's); rows
// whose m_indices entry is -1 (contiguous-layout padding) quantise as zeros. (An FP32
// evaluation is ~25% faster on the MoE-sized input but not exact; a hybrid that
// evaluates in FP64 only the elements an FP32 estimate cannot decide measured within 4%
// of this one.)
template <typename T, bool SWIGLU = false>
__global__ void __launch_bounds__(256) quantize_1x128_kernel(const T* X, int64_t ldx, uint8_t* Q, int64_t ldq,
                                                             float* sa, int64_t ld_sa, int M, int nkb,
                                                             const int32_t* m_indices = nullptr, int F = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;  // row within the wave's four
  const int c = lane & 15;  // 8-element chunk within the block
  const int64_t items = (int64_t)((M + 3) / 4) * nkb;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < items; it += (int64_t)gridDim.x * 4) {
    const int rg = (int)(it / nkb);
    const int kb = (int)(it - (int64_t)rg * nkb);
    const int r = rg * 4 + g;
    const bool live = r < M;
    float x[8];
    if constexpr (SWIGLU) {
      if (live && !(m_indices && m_indices[r] < 0)) {
        float u[8];
        load8(X + (int64_t)r * ldx + kb * 128 + c * 8, x);
        load8(X + (int64_t)r * ldx + F + kb * 128 + c * 8, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = swiglu_fp64(x[i], u[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
      }
    } else if (live) {
      load8(X + (int64_t)r * ldx + kb * 128 + c * 8, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    float s = amax / 448.0f;
    if (!(s > 0.0f)) s = 1.0f;
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] / s, x[1] / s, w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] / s, x[3] / s, w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] / s, x[5] / s, w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] / s, x[7] / s, w1, true);
    if (live) {
      *reinterpret_cast<uint2*>(Q + (int64_t)r * ldq + kb * 128 + c * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
      if (c == 0) sa[(int64_t)kb * ld_sa + r] = s;
    }
  }
}

// UE8M0 code of a positive normal FP32 scale: the smallest power of two not below it,
// i.e. the exponent field, plus one when a mantissa bit is set (exact for powers of two).
__device__ __forceinline__ uint32_t ue8m0_code(float x) {
  const uint32_t b = __float_as_uint(x);
  return ((b >> 23) & 0xFF) + ((b & 0x7FFFFFu) != 0u ? 1u : 0u);
}

// Scale factors given per row, sf[r][kb] (row stride ld_sf), into the layout the GEMMs
// read: activation scales transposed to out[kb][r] (FP32) or out[w][r] (packed UE8M0
// words, K blocks 4w..4w+3 in bytes 0..3), weight scales kept as out[r][kb] (FP32) or
// packed to out[r][w]; out's row stride is ld_out. One 32-bit output per thread (grid-
// stride); for activation scales consecutive threads write consecutive rows, the
// output's contiguous axis.
__global__ void transform_sf_kernel(const float* __restrict__ sf, int64_t ld_sf, int rows, int nkb,
                                    int is_activation, int pack, uint32_t* __restrict__ out, int64_t ld_out) {
  const int cols = pack ? (nkb + 3) / 4 : nkb;
  const int64_t n = (int64_t)rows * cols;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int r = is_activation ? (int)(idx % rows) : (int)(idx / cols);
    const int c = is_activation ? (int)(idx / rows) : (int)(idx % cols);
    const float* src = sf + (int64_t)r * ld_sf;
    uint32_t v = 0;
    if (pack) {
      for (int j = 0; j < 4; ++j)
        if (4 * c + j < nkb) v |= ue8m0_code(src[4 * c + j]) << (8 * j);
    } else {
      v = __float_as_uint(src[c]);
    }
    if (is_activation)
      out[(int64_t)c * ld_out + r] = v;
    else
      out[(int64_t)r * ld_out + c] = v;
  }
}

}  // namespace fp8gemm
