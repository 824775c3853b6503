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
// Data path per BM x BN output tile (one workgroup of WAVES_M x WAVES_N wave64s, each
// computing 64 x 16 TNW outputs; instances 128x128 with 2x2 waves, 256x256 with 4x2, and
// for the dense layouts' few-row shapes 64x128 (1x4 waves) and 128x64 (2x2 waves of 64x32)):
//   a STAGES-deep LDS ring holding, per 128-row K block, the A tile as [128 k][128 m] byte
//   panels (one [128 k][64 m] panel when BM = 64), the B tile likewise, and the block's
//   BM + BN scales, filled by direct-to-LDS loads (16 bytes per lane, 8 lanes per 128-byte
//   panel row, 4 per 64-byte row; one kilobyte per load instruction, spread evenly over
//   the waves, and one scale load per wave per block). The FP8 MFMA wants each lane's 32
//   operand bytes to be 32 K values of one row, so the
//   fragments are read with gfx950's transposing LDS read ds_read_b64_tr_b8: within each
//   16-lane group, output lane i gets byte (i & 7) of the 8-byte rows addressed by lanes
//   2j + (i >> 3), j = 0..7 (lane layout measured on the device). The lanes 2p and 2p+1
//   of a group therefore address the two 8-byte halves of one 16-column chunk in K row
//   p, and lane i receives 8 consecutive K values of column i.
//   Promotion: the per-column scales make the factor sa[kb][m] * sb[kb][n] different for
//   each element of a lane's four results (one m, four n), so it is formed per element:
//   one multiply and one FMA per output element per K block, i.e. eight wave64 FP32
//   operations (32 SIMD cycles) per 16x16x128 MFMA (also 32 cycles), as long as the
//   matrix work. The dense layouts' B scale covers a whole 128-column block, so there
//   the factor is one product per row and the promotion four FMAs per MFMA.
#pragma once

#include "fp8gemm_kernel.hpp"

namespace fp8gemm {

constexpr int kMaxKGroups = 256;  // the K-block offsets travel in the kernel arguments
constexpr int kDeferCols = 2;    // B columns of a block computed after the next block's barrier

typedef int v2i_t __attribute__((ext_vector_type(2)));

struct KParams {
  const uint8_t* A;
  const float* sa;
  const uint8_t* B;
  const float* sb;
  float* D;
  uint16_t* Dh;    // BF16 output of the dense layout calls (DENSE_TN instances)
  const uint16_t* C;  // dense layout calls: optional BF16 addend of D = C + A B (may be Dh)
  int64_t ldc;
  int c_vec;          // 1: C rows allow 8-byte loads (ldc % 4 == 0, C 8-byte aligned)
  int64_t lda, ld_sa, ldb, ld_sb, ldd, d_gstride;
  int M, N, G;
  int tiles_m, tiles_n;
  int accumulate;  // 1: D += result, 0: D = result
  int vec4;        // 1: D rows allow 16-byte accesses (ldd % 4 == 0, D 16-byte aligned)
  // split-K of the dense layout calls: each tile is split_k units of kb_per_split K
  // blocks (the last may be shorter); partials and arrival counters as in the NT call
  int split_k, kb_per_split;
  float* ws;
  int32_t* counters;
  int chunk;  // K-grouped: tiles per chunk (the CUs of one XCD), see the tile mapping
  // dense layouts (ignored by the K-grouped call): 1 when one tile row covers all of M, so
  // that each B tile is read by one unit: B is then loaded with the non-temporal hint
  // (streamed past the caches, which keep A; measured on the few-row shapes: up to 22%
  // faster, where B tiles are shared up to 18% slower)
  int stream_b;
  int kb_start[kMaxKGroups + 1];  // group g covers K blocks [kb_start[g], kb_start[g+1])
};

namespace kg {
constexpr int kPanel = 128 * 128;  // one [128 k][128 columns] byte panel of a K block
// A stage holds the A tile (BM columns or rows by 128 K bytes), then B (BN by 128), then
// the scales. A K-major operand of 128 or more columns is stored as [128 k][128 columns]
// panels; one of 64 columns as a single [128 k][64 columns] panel (64-byte rows). A
// K-contiguous operand is stored as [rows][128 k] (128-row panels, or one of 64 rows).
template <int BM, int BN, int NW>
struct Layout {
  static constexpr int wa = BM < 128 ? BM : 128, wb = BN < 128 ? BN : 128;  // panel widths
  static constexpr int la = BM * kBlockK / 1024, lb = BN * kBlockK / 1024;  // 1 KB loads per block
  static constexpr int b_off = BM * kBlockK;
  static constexpr int s_off = (BM + BN) * kBlockK;  // sa[BM] then sb[BN]
  static constexpr int stage = s_off + NW * 256;     // one 64-scale load per wave
};

// 16-byte chunk position of logical chunk c in K row k of a panel: c ^ chunk_key(k) in a
// 128-wide panel, c ^ chunk_key64(k) in a 64-wide one. With it, the 32 lanes of each
// half-wave of a fragment read (16 K rows, both 8-byte halves of one chunk) touch 32
// distinct 8-byte slots of a 256-byte bank row: in a 128-wide panel the rows alternate
// between the two 128-byte halves and the key spreads the chunks; in a 64-wide panel
// four rows share a bank row and the key gives those four (rows 4 and 32 apart) four
// distinct chunk positions.
__device__ __forceinline__ int chunk_key(int k) { return ((k >> 1) & 3) | ((k >> 3) & 4); }
__device__ __forceinline__ int chunk_key64(int k) { return ((k >> 2) & 1) | ((k >> 4) & 2); }
}  // namespace kg

// E8 instances take power-of-two scales (UE8M0 values 2^(e-127) held as FP32): the
// block-scaled MFMA multiplies each 128-K block product by 2^(ea[m]-127) * 2^(eb[n]-127)
// -- one exponent per lane for its A row and one for its B row, which is exactly the
// per-column scaling of both operands -- and accumulates it itself, so no promotion
// VALU work is left.
// DENSE_TN instances are the dense call in another memory layout (one group over all of
// K): B carries one scale per 128x128 block (sb [ceil(N/128)][ld_sb = K/128]) as in the NT
// call, and the output is BF16 (round to nearest even once, from the FP32 accumulator,
// after adding the optional BF16 C of D = C + A B). They may split K: the grid is then
// split_k units per tile, numbered split-major (the units that read the same K range of
// A run next to each other, on one XCD), and the last arrival of a tile's units sums the
// FP32 partials in split order before the epilogue, as in the NT kernel.
// A_KC / B_KC make that operand K-contiguous ([rows][K], as in the NT call) instead of
// K-major: its panels hold [128 rows][128 k] in the NT kernel's swizzled row layout and
// its fragments come from two 16-byte reads per lane, with the same lane -> K order as
// the transposing read (so the two kinds of operand combine): TN = neither, NN = A_KC,
// TT = B_KC.
template <int WAVES_M, int WAVES_N, int TNW, int STAGES, bool E8 = false, bool DENSE_TN = false, bool A_KC = false,
          bool B_KC = false>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, 1) fp8_k_grouped_tn_kernel(const KParams p) {
  using namespace kg;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BM = 64 * WAVES_M, BN = 16 * TNW * WAVES_N;
  typedef Layout<BM, BN, NW> LY;
  constexpr int LPW = (LY::la + LY::lb) / NW;  // operand loads per wave
  constexpr int LPS = LPW + 1;                  // + one scale load
  static_assert(LY::la + LY::lb == LPW * NW, "operand loads spread evenly");
  static_assert(BM + BN <= 64 * NW, "at most one scale load per wave");
  static_assert(BM % 64 == 0 && (BM <= 128 || BM % 128 == 0) && BN % 64 == 0 && (BN <= 128 || BN % 128 == 0),
                "64-wide or whole 128-wide panels");
  static_assert(TNW % 4 == 0 || TNW < 4, "the E8 form reads B fragments four at a time");
  static_assert(STAGES >= 2, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * LY::stage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // tile of this workgroup. Dense layouts: XCD-contiguous ranges of a split-major
  // rasterised order. K-grouped: the groups' K lengths differ, so giving each XCD a
  // contiguous range of a group-major order would leave the XCDs with the short groups
  // idle while the one with the longest finishes (workgroup b always runs on XCD b % 8).
  // Instead each group's tiles (in raster order) form chunks of p.chunk consecutive
  // tiles, one per CU of an XCD, and the chunks, group after group, are dealt to the
  // XCDs in turn: the i-th workgroup of XCD x takes tile i % chunk of chunk
  // (i / chunk) * 8 + x. Every XCD gets a like mix of groups; the tiles that run together
  // on one XCD are neighbours of one group and share its A and B panels in L2. The grid
  // covers whole rounds of chunks; workgroups past a group's last tile exit at once.
  const int per_group = p.tiles_m * p.tiles_n;
  const int S = DENSE_TN ? p.split_k : 1;
  int g, split, tile;
  if constexpr (DENSE_TN) {
    const int L = xcd_remap(blockIdx.x, per_group * S);
    g = 0;
    split = L / per_group;
    tile = L - split * per_group;
  } else {
    const int cpg = (per_group + p.chunk - 1) / p.chunk;  // chunks per group
    const int x = blockIdx.x % kNumXcd, i = blockIdx.x / kNumXcd;
    const int k = (i / p.chunk) * kNumXcd + x;
    g = k / cpg;
    split = 0;
    tile = (k - g * cpg) * p.chunk + i % p.chunk;
    if (g >= p.G || tile >= per_group) return;  // the whole workgroup: no barrier is pending
  }
  int tm, tn;
  raster(tile, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = p.kb_start[g] + split * p.kb_per_split;
  const int nkb = S > 1 ? min(p.kb_per_split, p.kb_start[g + 1] - kb0) : p.kb_start[g + 1] - kb0;

  // ---- direct-to-LDS load plan (the same per-lane offsets for every K block). Load
  // u = LPW wave + i fills kilobyte u of the stage (A's loads first): load v of an operand
  // covers, in a 128-wide K-major panel v / 16, K rows 8 (v % 16) + lane / 8 at chunk
  // position lane % 8, which holds logical chunk (lane % 8) ^ chunk_key(k); in a 64-wide
  // one, K rows 16 v + lane / 4 at position lane % 4 (logical chunk (lane % 4) ^
  // chunk_key64(k)).
  uint32_t off[LPW];
  bool is_b[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int u = LPW * wave + i;
    is_b[i] = u >= LY::la;
    const int v = is_b[i] ? u - LY::la : u;
    const int c0 = is_b[i] ? n0 : m0, lim = is_b[i] ? p.N : p.M;
    const uint32_t ld = (uint32_t)(is_b[i] ? p.ldb : p.lda);
    if (is_b[i] ? B_KC : A_KC) {
      // K-contiguous: LDS row position 8 (v % 16) + lane / 8 of panel v / 16 holds tile
      // row row_at(.), whose logical 16-byte K chunk (lane % 8) ^ (row & 7) sits at
      // position lane % 8; rows past M / N re-read the tile's first row. Offset from the
      // tile's first row.
      const int row = 128 * (v >> 4) + row_at(8 * (v & 15) + (lane >> 3));
      const int c = (lane & 7) ^ (row & 7);
      off[i] = (c0 + row < lim ? (uint32_t)row : 0u) * ld + (uint32_t)(16 * c);
    } else {
      int k, col;
      if ((is_b[i] ? LY::wb : LY::wa) == 128) {
        k = 8 * (v & 15) + (lane >> 3);
        col = 128 * (v >> 4) + 16 * ((lane & 7) ^ chunk_key(k));
      } else {
        k = 16 * v + (lane >> 2);
        col = 16 * ((lane & 3) ^ chunk_key64(k));
      }
      const int col_g = c0 + col < lim ? c0 + col : c0;   // chunks past M / N re-read the first
      off[i] = (uint32_t)k * ld + (uint32_t)col_g;
    }
  }
  // scales: wave w loads entry 64 w + lane of [sa of the BM columns | sb of the BN columns];
  // waves past the BM + BN entries re-load the last sb entries into their own unused slot,
  // so that every wave issues LPS loads per block
  const bool s_is_a = 64 * wave < BM;
  const int s_col = s_is_a ? m0 + 64 * wave + lane : n0 + min(64 * wave - BM, BN - 64) + lane;
  const int s_lim = (s_is_a ? p.M : p.N) - 1;
  const int s_c = s_col < s_lim ? s_col : s_lim;
  // column-scale layouts advance one row per K block; the 128x128 block layout of B
  // holds a K block's scale of column n at [n / 128][kb]
  const float* s_src = s_is_a ? p.sa + s_c : (DENSE_TN ? p.sb + (int64_t)(s_c >> 7) * p.ld_sb : p.sb + s_c);
  const int64_t s_ld = s_is_a ? p.ld_sa : (DENSE_TN ? 1 : p.ld_sb);

  const uint32_t smem_base = lds_addr(smem);
  auto issue = [&](int kb, int slot) {
    const uint32_t st = smem_base + slot * LY::stage;
    const int64_t krow = (int64_t)(kb0 + kb) * kBlockK;
    const uint8_t* a_base = A_KC ? p.A + (int64_t)m0 * p.lda + krow : p.A + krow * p.lda;
    const uint8_t* b_base = B_KC ? p.B + (int64_t)n0 * p.ldb + krow : p.B + krow * p.ldb;
    if (DENSE_TN && p.stream_b) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        if (is_b[i])
          dma16nt(b_base, off[i], st + (LPW * wave + i) * 1024);
        else
          dma16(a_base, off[i], st + (LPW * wave + i) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma16(is_b[i] ? b_base : a_base, off[i], st + (LPW * wave + i) * 1024);
    }
    dma4v(s_src + (int64_t)(kb0 + kb) * s_ld, st + LY::s_off + wave * 256);
  };

  // ---- fragment read plan: lane l = 16 q + i reads, for r = 0..3, K row 32 q + 8 r + i / 2,
  // the 8-byte half i & 1 of the fragment's chunk (chunk_key depends on the lane only)
  const int q = lane >> 4, li = lane & 15;
  // chunk_key / chunk_key64 of the lane's K rows (the same for its four reads)
  const int key = ((li >> 2) & 3) | ((q & 1) << 2), key64 = ((li >> 3) & 1) | ((q & 1) << 1);
  const int rd_row = 32 * q + (li >> 1);                 // + 8 r
  // byte offset of logical chunk c (16 columns) of an operand tile of panel width W
  auto frag_off = [&](int c, int W) {
    return W == 128 ? (c >> 3) * kPanel + rd_row * 128 + (((c & 7) ^ key) << 4) + 8 * (li & 1)
                    : rd_row * 64 + (((c & 3) ^ key64) << 4) + 8 * (li & 1);
  };
  typedef __attribute__((address_space(3))) v2i_t* lds_v2i;
  // A fragment is read by RA (A) or RB (B) instructions: four transposing 8-byte reads
  // of a K-major operand, or two 16-byte reads of a K-contiguous one. Read r fills
  // elements [8 r / R, 8 (r + 1) / R) of the fragment.
  constexpr int RA = A_KC ? 2 : 4, RB = B_KC ? 2 : 4;
  // K-contiguous operand: 16-row chunk c of the tile; lane 16 q + i takes row 16 c + i,
  // K bytes 32 q .. 32 q + 31 (logical 16-byte chunks 2q and 2q + 1)
  auto read_part = [&](uint8_t* tile, int c, int r, bool kc, int W, v8i& f) {
    if (kc) {
      const int row = 16 * (c & 7) + li;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + (c >> 3) * kPanel + swz(row, 2 * q + r));
      f[4 * r] = (int)v.x, f[4 * r + 1] = (int)v.y, f[4 * r + 2] = (int)v.z, f[4 * r + 3] = (int)v.w;
    } else {
      const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(v2i_t*)(tile + frag_off(c, W) + r * 8 * W));
      f[2 * r] = x[0], f[2 * r + 1] = x[1];
    }
  };
  auto part_a = [&](uint8_t* st, int c, int r, v8i& f) { read_part(st, c, r, A_KC, LY::wa, f); };
  auto part_b = [&](uint8_t* st, int c, int r, v8i& f) { read_part(st + LY::b_off, c, r, B_KC, LY::wb, f); };

  v4f acc[4][TNW];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[t][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- K loop. Per block a wave issues 4 TNW MFMAs, B column chunk j (TNW wn + j)
  // against its four A fragments t.
  // FP32 scales: the B fragments stream. While the MFMAs of column j run, the wave reads
  // column j + 1. The last ND columns of a block are deferred past the next block's
  // barrier: their MFMAs then run while the new block's A fragments are read (each
  // replacing an A fragment once the deferred MFMAs have consumed it). Each MFMA is one
  // slot: the MFMA, its share of the reads, then the promotion of the MFMA two slots back,
  // whose result is ready by then; scheduling barriers keep the slots in order. Before the
  // first block the deferred columns are all zero operands with zero scales, so they add
  // +0 exactly.
  // E8 (no promotion): the wave reads its A fragments, then four B fragments at a time
  // and issues their 16 MFMAs; left to the compiler's schedule this measured faster than
  // the streamed order.
  constexpr int ND = kDeferCols < TNW ? kDeferCols : TNW - 1;
  constexpr int NMF = 4 * TNW, NDS = 4 * ND;  // slots per block, deferred slots
  const int cb0 = TNW * wn;  // the wave's first 16-column chunk of the B tile
  v8i fa[4], fb_last[ND];
#pragma unroll
  for (int t = 0; t < 4; ++t) fa[t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int d = 0; d < ND; ++d) fb_last[d] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  // scales of the deferred columns: the per-row factors (the product with the B scale
  // for the dense layouts, the A scale alone for the K-grouped form, whose B scales are
  // per column, sb_last)
  float s_last[4] = {0.f, 0.f, 0.f, 0.f};
  v4f sb_last[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) sb_last[d] = v4f{0.f, 0.f, 0.f, 0.f};
  // slot u: A fragment t and B column j (deferred: column TNW - ND + d of the last block)
  auto slot_t = [](int u) { return u < NDS ? u / ND : (u - NDS) & 3; };
  auto slot_j = [](int u) { return u < NDS ? TNW - ND + u % ND : (u - NDS) >> 2; };

  // STAGES-deep ring: blocks kb + 1 .. kb + STAGES - 2 stay in flight while block kb is
  // computed, and block kb + STAGES - 1 refills the slot of block kb - 1
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkb) issue(s, s);
  int slot = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    wait_stages<LPS, STAGES - 2>(nkb - 1 - kb);  // this wave's loads of block kb have landed
    wait_lgkmcnt0();   // and its reads of block kb - 1 (the deferred columns' B fragments)
    barrier();         // everyone's have, and everyone is done reading block kb - 1
    if (kb + STAGES - 1 < nkb) issue(kb + STAGES - 1, slot == 0 ? STAGES - 1 : slot - 1);

    uint8_t* st = smem + slot * LY::stage;
    slot = slot == STAGES - 1 ? 0 : slot + 1;
    const float* s_a = reinterpret_cast<const float*>(st + LY::s_off);
    const float* s_b = s_a + BM;
    float sa_t[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sa_t[t] = s_a[64 * wm + 16 * t + li];

    if constexpr (E8) {
      // operand scales: lane l carries the exponent of its A row 16 t + l % 16 and of its
      // B row 16 j + l % 16 (the same for its four 32-K chunks: one block scale)
      int ea[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < RA; ++r) part_a(st, 4 * wm + t, r, fa[t]);
        ea[t] = (__float_as_int(sa_t[t]) >> 23) & 0xFF;
      }
      constexpr int GB = TNW < 4 ? TNW : 4;
#pragma unroll
      for (int jh = 0; jh < TNW / GB; ++jh) {
        v8i fb[GB];
        int eb[GB];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
#pragma unroll
          for (int r = 0; r < RB; ++r) part_b(st, cb0 + GB * jh + j, r, fb[j]);
          eb[j] = (__float_as_int(s_b[16 * (cb0 + GB * jh + j) + li]) >> 23) & 0xFF;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < GB; ++j)
            acc[t][GB * jh + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fb[j], fa[t], acc[t][GB * jh + j], 0, 0, 0, eb[j], 0, ea[t]);
      }
      continue;
    }

    // dense layouts: the wave's 16 TNW columns lie in one 128-column block of B, whose
    // scale every column entry repeats
    const float sbw = DENSE_TN ? s_b[16 * cb0] : 0.f;
    v4f sbc[TNW];   // K-grouped form: B scales of the lane's four columns of chunk j
    v8i fb[TNW];
#pragma unroll
    for (int r = 0; r < RB; ++r) part_b(st, cb0, r, fb[0]);
    auto col_scale = [&](int j) {
      if constexpr (!DENSE_TN) sbc[j] = *reinterpret_cast<const v4f*>(s_b + 16 * (cb0 + j) + 4 * q);
    };
    col_scale(0);

    v4f res[NMF];
    auto promote = [&](int u) {
      const v4f v = res[u];
      const bool def = u < NDS;
      const int t = slot_t(u), j = slot_j(u);
      v4f s;
      if constexpr (DENSE_TN) {
        const float f = def ? s_last[t] : sa_t[t] * sbw;
        s = v4f{f, f, f, f};
      } else {
        s = def ? sb_last[u % ND] * s_last[t] : sbc[j] * sa_t[t];
      }
      v4f& a = acc[t][j];
      a[0] = __builtin_fmaf(v[0], s[0], a[0]);
      a[1] = __builtin_fmaf(v[1], s[1], a[1]);
      a[2] = __builtin_fmaf(v[2], s[2], a[2]);
      a[3] = __builtin_fmaf(v[3], s[3], a[3]);
    };
#pragma unroll
    for (int u = 0; u < NMF; ++u) {
      const bool def = u < NDS;
      const int t = slot_t(u), j = slot_j(u);
      res[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(def ? fb_last[u % ND] : fb[j], fa[t],
                                                                v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      if (def) {
        // the last deferred MFMA of A fragment t has read it: read this block's
        if (u % ND == ND - 1) {
#pragma unroll
          for (int r = 0; r < RA; ++r) part_a(st, 4 * wm + t, r, fa[t]);
        }
      } else {
        // column j reads column j + 1, the last regular column also the deferred ones;
        // their parts go out in the first three slots (the first takes the extra), so the
        // last lands two MFMAs before its first use
        const int c1 = j + 1, c2 = j == TNW - ND - 1 ? TNW - 1 : j + 1;
        const int nparts = (c2 - c1 + 1) * RB;
#pragma unroll
        for (int p = 0; p < nparts; ++p)
          if (p * 3 / nparts == t) part_b(st, cb0 + c1 + p / RB, p % RB, fb[c1 + p / RB]);
        if (t == 2)
#pragma unroll
          for (int c = c1; c <= c2; ++c) col_scale(c);
      }
      if (u >= 2) promote(u - 2);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    promote(NMF - 2);
    promote(NMF - 1);
    // the last ND columns wait for the next block (or the drain below)
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      fb_last[d] = fb[TNW - ND + d];
      if constexpr (!DENSE_TN) sb_last[d] = sbc[TNW - ND + d];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) s_last[t] = DENSE_TN ? sa_t[t] * sbw : sa_t[t];
  }
  // drain: the deferred columns of the last block
  if constexpr (!E8) {
#pragma unroll
    for (int u = 0; u < NDS; ++u) {
      const int t = slot_t(u), j = slot_j(u), d = u % ND;
      const v4f v = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb_last[d], fa[t], v4f{0.f, 0.f, 0.f, 0.f}, 0,
                                                                     0, 0, 0, 0, 0);
      const v4f s = DENSE_TN ? v4f{s_last[t], s_last[t], s_last[t], s_last[t]} : sb_last[d] * s_last[t];
      v4f& a = acc[t][j];
      a[0] = __builtin_fmaf(v[0], s[0], a[0]);
      a[1] = __builtin_fmaf(v[1], s[1], a[1]);
      a[2] = __builtin_fmaf(v[2], s[2], a[2]);
      a[3] = __builtin_fmaf(v[3], s[3], a[3]);
    }
  }

  // ---- epilogue: lane holds D[m][n .. n + 3] of each fragment
  if constexpr (DENSE_TN) {
    __shared__ int s_last;
    // fragments of this wave whose rows start below M (the few-row shapes leave whole
    // fragments past M)
    const int live_t = max(0, min(4, (p.M - m0 - 64 * wm + 15) >> 4));
    // (K is split only with 64x64 or 64x32 wave tiles: the reduce of a 64x128 one would spill)
    if constexpr (TNW <= 4) {
      if (S > 1 && !reduce_splits(p.ws, p.counters, acc, tile, split, S, (wave * 4 * TNW) * 64 + lane, BM * BN, tid,
                                  &s_last, live_t))
        return;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + 64 * wm + 16 * t + li;
      if (m >= p.M) continue;
      uint16_t* row = p.Dh + (int64_t)m * p.ldd;
#pragma unroll
      for (int j = 0; j < TNW; ++j) {
        const int n = n0 + 16 * (TNW * wn + j) + 4 * q;
        v4f v = acc[t][j];
        if (p.C) {  // each lane reads the C elements of exactly the D elements it writes
          const uint16_t* crow = p.C + (int64_t)m * p.ldc + n;
          if (p.c_vec && n + 3 < p.N) {
            const uint2 cw = *reinterpret_cast<const uint2*>(crow);
            v[0] += bf16_value(cw.x & 0xFFFF), v[1] += bf16_value(cw.x >> 16);
            v[2] += bf16_value(cw.y & 0xFFFF), v[3] += bf16_value(cw.y >> 16);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.N) v[r] += bf16_value(crow[r]);
          }
        }
        const uint32_t lo = bf16x2_bits(v[0], v[1]), hi = bf16x2_bits(v[2], v[3]);
        if (p.vec4 && n + 3 < p.N) {
          *reinterpret_cast<uint2*>(row + n) = make_uint2(lo, hi);
        } else {
          const uint32_t w[2] = {lo, hi};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) row[n + r] = (uint16_t)(w[r >> 1] >> (16 * (r & 1)));
        }
      }
    }
    return;
  }
  float* Dg = p.D + (int64_t)g * p.d_gstride;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + 64 * wm + 16 * t + li;
    if (m >= p.M) continue;
    float* row = Dg + (int64_t)m * p.ldd;
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const int n = n0 + 16 * (TNW * wn + j) + 4 * q;
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
