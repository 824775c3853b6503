// K-grouped TN FP8 GEMM: the MoE weight-gradient form (DeepGEMM overview,
// es.news.hada.io/topic?id=19459, "Dense y Grouped GEMM": grouping along K with M and N
// fixed, k_grouped_fp8_gemm_tn_contiguous).
//
//   D[g][m][n] = C[g][m][n] + sum_{kb in group g} P_kb[m][n] * sa[kb][m] * sb[kb][n]
//   P_kb[m][n] = sum_{k in block kb} A[k][m] * B[k][n]
//
// A [K][M] and B [K][N] are e4m3, K-major ("TN": the K axis is the strided one for both
// operands); group g owns the K rows [128 kb_start[g], 128 kb_start[g+1]). Both operands
// carry one FP32 scale per column per 128-row K block (sa [K/128][ld_sa], sb
// [K/128][ld_sb]). D is FP32 [G][M][N]; C is the old D when accumulating, else +0.
//
// Data path per 128x128 output tile (one workgroup, 4 wave64s in 2x2, 64x64 each):
//   a 2-stage LDS ring of [128 k][128 m] A and [128 k][128 n] B tiles filled by
//   direct-to-LDS loads (16 bytes per lane, 8 lanes per 128-byte K row), plus the block's
//   256 scales. The FP8 MFMA wants each lane's 32 operand bytes to be 32 K values of one
//   row, so the fragments are read with gfx950's transposing LDS read ds_read_b64_tr_b8:
//   within each 16-lane group, output lane i gets byte (i & 7) of the 8-byte rows
//   addressed by lanes 2j + (i >> 3), j = 0..7 (lane layout measured on the device). The
//   lanes 2p and 2p+1 of a group therefore address the two 8-byte halves of one 16-column
//   chunk in K row p, and lane i receives 8 consecutive K values of column i.
//   Promotion: the per-column scales make the factor sa[kb][m] * sb[kb][n] different for
//   each element of a lane's four results (one m, four n), so it is formed per element.
#pragma once

#include "fp8gemm_kernel.hpp"

namespace fp8gemm {

constexpr int kMaxKGroups = 256;  // the K-block offsets travel in the kernel arguments

typedef int v2i_t __attribute__((ext_vector_type(2)));

struct KParams {
  const uint8_t* A;
  const float* sa;
  const uint8_t* B;
  const float* sb;
  float* D;
  int64_t lda, ld_sa, ldb, ld_sb, ldd, d_gstride;
  int M, N, G;
  int tiles_m, tiles_n;
  int accumulate;  // 1: D += result, 0: D = result
  int vec4;        // 1: D rows allow 16-byte accesses (ldd % 4 == 0, D 16-byte aligned)
  int kb_start[kMaxKGroups + 1];  // group g covers K blocks [kb_start[g], kb_start[g+1])
};

namespace kg {
constexpr int BM = 128, BN = 128;
constexpr int kTileBytes = 128 * 128;                      // one operand's K block
constexpr int kStage = 2 * kTileBytes + 2 * 128 * 4;        // A, B, sa[128], sb[128]
constexpr int kStages = 2;
constexpr int kLoadsPerStage = 9;                           // per wave: 4 A, 4 B, 1 scale

// 16-byte chunk position of logical chunk c in K row k of a staged tile. With it, the
// 32 lanes of each half-wave of a fragment read (16 K rows, both 8-byte halves of one
// chunk) touch 32 distinct 8-byte bank slots.
__device__ __forceinline__ int chunk_key(int k) { return ((k >> 1) & 3) | ((k >> 3) & 4); }
}  // namespace kg

__global__ void __launch_bounds__(256, 2) fp8_k_grouped_tn_kernel(const KParams p) {
  using namespace kg;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile of this workgroup: XCD-contiguous ranges of a group-major, rasterised order
  const int per_group = p.tiles_m * p.tiles_n;
  const int L = xcd_remap(blockIdx.x, p.G * per_group);
  const int g = L / per_group;
  int tm, tn;
  raster(L - g * per_group, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = p.kb_start[g], nkb = p.kb_start[g + 1] - kb0;

  // ---- direct-to-LDS load plan (the same per-lane offsets for every K block)
  // instruction i of this wave writes K rows 8 (4 wave + i) + lane / 8 of the tile,
  // chunk position lane % 8, which holds logical chunk (lane % 8) ^ chunk_key(row)
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ chunk_key(k);
    const int ma = m0 + 16 * c < p.M ? m0 + 16 * c : m0;   // chunks past M re-read chunk 0
    const int nb = n0 + 16 * c < p.N ? n0 + 16 * c : n0;
    a_off[i] = (uint32_t)(8 * i + (lane >> 3)) * (uint32_t)p.lda + (uint32_t)ma;
    b_off[i] = (uint32_t)(8 * i + (lane >> 3)) * (uint32_t)p.ldb + (uint32_t)nb;
  }
  // scales: wave 0/1 load sa of columns 64 (wave & 1) + lane, wave 2/3 the same of sb
  const bool s_is_a = wave < 2;
  const int s_col = (s_is_a ? m0 : n0) + 64 * (wave & 1) + lane;
  const int s_lim = (s_is_a ? p.M : p.N) - 1;
  const float* s_src = (s_is_a ? p.sa : p.sb) + (s_col < s_lim ? s_col : s_lim);
  const int64_t s_ld = s_is_a ? p.ld_sa : p.ld_sb;

  const uint32_t smem_base = lds_addr(smem);
  auto issue = [&](int kb, int slot) {
    const uint32_t st = smem_base + slot * kStage;
    const int64_t krow = (int64_t)(kb0 + kb) * kBlockK + 32 * wave;
    const uint8_t* a_base = p.A + krow * p.lda;
    const uint8_t* b_base = p.B + krow * p.ldb;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(a_base, a_off[i], st + (4 * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(b_base, b_off[i], st + kTileBytes + (4 * wave + i) * 1024);
    dma4v(s_src + (int64_t)(kb0 + kb) * s_ld, st + 2 * kTileBytes + wave * 256);
  };

  // ---- fragment read plan: lane l = 16 q + i reads, for r = 0..3, K row 32 q + 8 r + i / 2,
  // the 8-byte half i & 1 of the fragment's chunk (chunk_key depends on the lane only)
  const int q = lane >> 4, li = lane & 15;
  const int key = ((li >> 2) & 3) | ((q & 1) << 2);
  const int rd_row = 32 * q + (li >> 1);                 // + 8 r
  auto frag_off = [&](int chunk) { return rd_row * 128 + ((chunk ^ key) << 4) + 8 * (li & 1); };

  v4f acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nkb > 0) issue(0, 0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int slot = kb & 1;
    wait_vmcnt<0>();   // this wave's loads of block kb have landed
    barrier();         // everyone's have, and everyone is done reading block kb - 1
    if (kb + 1 < nkb) issue(kb + 1, slot ^ 1);

    uint8_t* st = smem + slot * kStage;
    typedef __attribute__((address_space(3))) v2i_t* lds_v2i;
    v8i fa[4], fb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint8_t* base = st + frag_off(4 * wm + t);
      v2i_t x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(v2i_t*)(base + r * 8 * 128));
      fa[t] = v8i{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint8_t* base = st + kTileBytes + frag_off(4 * wn + j);
      v2i_t x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(v2i_t*)(base + r * 8 * 128));
      fb[j] = v8i{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
    }
    const float* s_a = reinterpret_cast<const float*>(st + 2 * kTileBytes);
    const float* s_b = s_a + 128;
    float sa_t[4];
    v4f sb_j[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sa_t[t] = s_a[64 * wm + 16 * t + li];
#pragma unroll
    for (int j = 0; j < 4; ++j) sb_j[j] = *reinterpret_cast<const v4f*>(s_b + 64 * wn + 16 * j + 4 * q);

#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], fa[t], v4f{0.f, 0.f, 0.f, 0.f},
                                                                        0, 0, 0, 0, 0, 0);
        const v4f s = sb_j[j] * sa_t[t];
        acc[t][j][0] = __builtin_fmaf(r[0], s[0], acc[t][j][0]);
        acc[t][j][1] = __builtin_fmaf(r[1], s[1], acc[t][j][1]);
        acc[t][j][2] = __builtin_fmaf(r[2], s[2], acc[t][j][2]);
        acc[t][j][3] = __builtin_fmaf(r[3], s[3], acc[t][j][3]);
      }
  }

  // ---- epilogue: lane holds D[m][n .. n + 3] of each fragment
  float* Dg = p.D + (int64_t)g * p.d_gstride;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + 64 * wm + 16 * t + li;
    if (m >= p.M) continue;
    float* row = Dg + (int64_t)m * p.ldd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + 4 * q;
      v4f v = acc[t][j];
      if (p.vec4 && n + 3 < p.N) {
        v4f* dst = reinterpret_cast<v4f*>(row + n);
        if (p.accumulate) v += *dst;
        *dst = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) row[n + r] = p.accumulate ? row[n + r] + v[r] : v[r];
      }
    }
  }
}

}  // namespace fp8gemm
