// Device code of libfp8gemm: one kernel template serves the dense, M-grouped
// contiguous and M-grouped masked FP8 NT GEMMs (DeepGEMM overview page,
// deepep.org/zh/deepgemm, 核心优化技术: one scheduler for grouped and non-grouped
// kernels, rasterised for L2 reuse).
//
// Per work unit (one BM x BN output tile, or one K-slice of it under split-K):
//   for every 128-wide K block kb (one scale block, one MFMA deep):
//     stage A[BM x 128] and B[BN x 128] bytes HBM -> registers -> LDS (2 stages,
//       XOR-swizzled 16-byte chunks so fragment reads spread over the banks);
//     t = v_mfma_f32_16x16x128_f8f6f4(B frag, A frag, 0)      -- exact FP8 products
//     acc += t * (sa[kb][m] * sb[n/128][kb])                   -- FP32 promotion
//   then round acc to BF16 (nearest-even) and store live rows.
// The promotion step is the pages' two-level accumulation (GeekNews topic 19444,
// intro; bquan.live post 9429818, "Comprender profundamente DeepGEMM"): every
// 128-K partial is scaled and added into an FP32 accumulator outside the matrix
// unit.
//
// MFMA operand roles: the MFMA's first operand carries 16 rows of B (n) and the
// second 16 rows of A (m), so lane l of the 16x16 result holds
// D[m0 + l%16][n0 + 4*(l/16) + r], r = 0..3: four consecutive columns of one row
// (one 8-byte BF16 store) and a single activation scale per lane. Both operands
// use the same lane->K assignment, so the K order inside the MFMA is irrelevant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

constexpr int kBlockK = 128;   // K extent of a scale block and of one MFMA
constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kMaxGroups = 1024;
constexpr int kNumXcd = 8;     // MI355X: 8 XCDs, workgroups dispatched round-robin

enum : int { kDense = 0, kContiguous = 1, kMasked = 2 };

struct Params {
  const uint8_t* A;
  const float* sa;
  const uint8_t* B;
  const float* sb;
  uint16_t* D;
  int64_t lda, ld_sa, ldb, ldd;
  int64_t a_gstride, sa_gstride, b_gstride, sb_gstride, d_gstride;  // per group (masked / B)
  const int32_t* m_indices;  // contiguous
  const int32_t* masked_m;   // masked
  int M;        // rows: M (dense), M_total (contiguous), M_max (masked)
  int N, K, G;
  int kind;
  int tiles_m, tiles_n;      // tiles_m per group for masked
  int split_k, kb_per_split, num_kb;
  int num_units;             // dense / contiguous: tiles * split_k (masked: computed on device)
  int group_m;               // raster group height in tiles
  int vec_store;             // D rows allow 8-byte stores (ldd % 4 == 0, D 8-byte aligned)
  float* ws;                 // split-K partials [tile][split][BM*BN]
  int32_t* counters;         // split-K arrival counters [tile]
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// FP32 -> BF16 bits, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Bijection on [0, U) that gives each XCD one contiguous range of logical units:
// unit u runs on XCD u % 8 (when the grid is a multiple of 8), so units that share
// an XCD's L2 become neighbours in the rasterised order.
__device__ __forceinline__ int xcd_remap(int u, int U) {
  const int per = (U + kNumXcd - 1) / kNumXcd;
  const int full = U - (per - 1) * kNumXcd;  // XCDs holding `per` units
  const int x = u % kNumXcd, i = u / kNumXcd;
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

// Grouped rasterisation: walk `gm` tile rows at a time so concurrently running
// tiles share both A row blocks and B column blocks in L2.
__device__ __forceinline__ void raster(int L, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int per_group = gm * tiles_n;
  const int grp = L / per_group;
  const int first = grp * gm;
  const int gs = min(tiles_m - first, gm);
  const int r = L - grp * per_group;
  tm = first + r % gs;
  tn = r / gs;
}

// Swizzled byte offset of 16-byte chunk `c` (0..7) of LDS row `row` (128 bytes/row).
__device__ __forceinline__ int swz(int row, int c) { return row * kBlockK + ((c ^ (row & 7)) << 4); }

template <int BM, int BN, int WAVES_M, int WAVES_N, int OCC>
__global__ void __launch_bounds__(kThreads, OCC) fp8_gemm_kernel(const Params p) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per workgroup");
  constexpr int WTM = BM / WAVES_M;  // wave tile rows
  constexpr int WTN = BN / WAVES_N;  // wave tile cols
  constexpr int TM = WTM / 16;
  constexpr int TN = WTN / 16;
  static_assert(TM >= 1 && TN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(kBlockK % WTN == 0, "a wave's columns must share one 128-column scale block");
  constexpr int A_BYTES = BM * kBlockK;
  constexpr int B_BYTES = BN * kBlockK;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LD = A_BYTES / (16 * kThreads);  // 16-byte chunks per thread per kb
  constexpr int B_LD = B_BYTES / (16 * kThreads);
  static_assert(A_LD * 16 * kThreads == A_BYTES && B_LD * 16 * kThreads == B_BYTES, "tile load split");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int s_pre[kMaxGroups + 1];  // masked: prefix sums of live m-tiles per group
  __shared__ int s_info;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int S = p.split_k;

  // ---- masked: live m-tiles per group, exclusive prefix sum in LDS
  int num_units = p.num_units;
  if (p.kind == kMasked) {
    constexpr int PER = (kMaxGroups + kThreads - 1) / kThreads;
    int local[PER];
    int run = 0;
    for (int q = 0; q < PER; ++q) {
      const int g = tid * PER + q;
      int t = 0;
      if (g < p.G) {
        const int live = min(max(p.masked_m[g], 0), p.M);
        t = (live + BM - 1) / BM;
      }
      local[q] = run;
      run += t;
    }
    // inclusive scan of per-thread totals (Hillis-Steele over 256 entries)
    __shared__ int s_scan[kThreads];
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int base = s_scan[tid] - run;
    for (int q = 0; q < PER; ++q) {
      const int g = tid * PER + q;
      if (g <= p.G && g < kMaxGroups + 1) s_pre[g] = base + local[q];
    }
    if (tid == kThreads - 1) s_pre[min(p.G, kMaxGroups)] = s_scan[kThreads - 1];
    __syncthreads();
    num_units = s_pre[p.G] * p.tiles_n * S;
  }

  for (int u = blockIdx.x; u < num_units; u += gridDim.x) {
    const int L = xcd_remap(u, num_units);
    int g = 0, tm, tn, split, tile_id;
    if (p.kind == kMasked) {
      // units of one (group, n-tile) are contiguous: the group's B tile is reused
      int lo = 0, hi = p.G;  // largest g with s_pre[g] * tiles_n * S <= L
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] * p.tiles_n * S <= L) lo = mid; else hi = mid;
      }
      g = lo;
      const int live_tiles = s_pre[g + 1] - s_pre[g];
      const int local = L - s_pre[g] * p.tiles_n * S;
      tn = local / (live_tiles * S);
      const int r = local - tn * live_tiles * S;
      tm = r / S;
      split = r - tm * S;
      tile_id = (s_pre[g] + tm) * p.tiles_n + tn;
    } else {
      const int tile = L / S;
      split = L - tile * S;
      raster(tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
      tile_id = tm * p.tiles_n + tn;
    }
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // ---- contiguous: expert of this row block (-1 everywhere = nothing to do)
    if (p.kind == kContiguous) {
      if (tid == 0) s_info = -1;
      __syncthreads();
      if (tid < BM && m0 + tid < p.M) {
        const int e = p.m_indices[m0 + tid];
        if (e >= 0) atomicMax(&s_info, e);
      }
      __syncthreads();
      g = s_info;
      __syncthreads();
      if (g < 0 || g >= p.G) continue;  // all padding (or an invalid id): nothing to write
    }

    const int kb0 = split * p.kb_per_split;
    const int kb1 = min(p.num_kb, kb0 + p.kb_per_split);
    const uint8_t* Ag = p.A + (p.kind == kMasked ? (int64_t)g * p.a_gstride : 0);
    const float* sag = p.sa + (p.kind == kMasked ? (int64_t)g * p.sa_gstride : 0);
    const uint8_t* Bg = p.B + (int64_t)g * p.b_gstride;
    const float* sbg = p.sb + (int64_t)g * p.sb_gstride;

    // ---- global -> LDS copy plan: thread owns fixed 16-byte chunks of each tile
    const uint8_t* a_src[A_LD];
    int a_dst[A_LD];
#pragma unroll
    for (int r = 0; r < A_LD; ++r) {
      const int q = tid + r * kThreads;
      const int row = q >> 3, c = q & 7;
      const int grow = min(m0 + row, p.M - 1);  // rows past the end: clamped, results unused
      a_src[r] = Ag + (int64_t)grow * p.lda + c * 16;
      a_dst[r] = swz(row, c);
    }
    const uint8_t* b_src[B_LD];
    int b_dst[B_LD];
#pragma unroll
    for (int r = 0; r < B_LD; ++r) {
      const int q = tid + r * kThreads;
      const int row = q >> 3, c = q & 7;
      const int grow = min(n0 + row, p.N - 1);
      b_src[r] = Bg + (int64_t)grow * p.ldb + c * 16;
      b_dst[r] = A_BYTES + swz(row, c);
    }

    // rows / scale indices of this lane
    int sa_row[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_row[i] = min(m0 + wm * WTM + 16 * i + (lane & 15), p.M - 1);
    const int sb_row = min(n0 + wn * WTN, p.N - 1) / kBlockK;
    const float* sb_ptr = sbg + (int64_t)sb_row * p.num_kb;

    v4i ra[A_LD], rb[B_LD];
    float sa_next[TM], sb_next;
    auto gload = [&](int kb) {
#pragma unroll
      for (int r = 0; r < A_LD; ++r) ra[r] = *reinterpret_cast<const v4i*>(a_src[r] + (int64_t)kb * kBlockK);
#pragma unroll
      for (int r = 0; r < B_LD; ++r) rb[r] = *reinterpret_cast<const v4i*>(b_src[r] + (int64_t)kb * kBlockK);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_next[i] = sag[(int64_t)kb * p.ld_sa + sa_row[i]];
      sb_next = sb_ptr[kb];
    };
    auto lstore = [&](int stage) {
      uint8_t* base = smem + stage * STAGE;
#pragma unroll
      for (int r = 0; r < A_LD; ++r) *reinterpret_cast<v4i*>(base + a_dst[r]) = ra[r];
#pragma unroll
      for (int r = 0; r < B_LD; ++r) *reinterpret_cast<v4i*>(base + b_dst[r]) = rb[r];
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (kb0 < kb1) {
      gload(kb0);
      lstore(0);
    }
    __syncthreads();

    const int frow = lane & 15;        // fragment row within a 16-row subtile
    const int fchunk = (lane >> 4) * 2;  // first of the lane's two 16-byte K chunks
    for (int kb = kb0; kb < kb1; ++kb) {
      const int cur = (kb - kb0) & 1;
      float s[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) s[i] = sa_next[i] * sb_next;
      if (kb + 1 < kb1) gload(kb + 1);

      const uint8_t* sA = smem + cur * STAGE;
      const uint8_t* sB = sA + A_BYTES;
      v8i fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + 16 * i + frow;
        const v4i lo = *reinterpret_cast<const v4i*>(sA + swz(row, fchunk));
        const v4i hi = *reinterpret_cast<const v4i*>(sA + swz(row, fchunk + 1));
        fa[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WTN + 16 * j + frow;
        const v4i lo = *reinterpret_cast<const v4i*>(sB + swz(row, fchunk));
        const v4i hi = *reinterpret_cast<const v4i*>(sB + swz(row, fchunk + 1));
        fb[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fb[j], fa[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          acc[i][j][0] = __builtin_fmaf(t[0], s[i], acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(t[1], s[i], acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(t[2], s[i], acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(t[3], s[i], acc[i][j][3]);
        }
      }
      if (kb + 1 < kb1) lstore(cur ^ 1);
      __syncthreads();
    }

    // ---- split-K: publish the partial; the last of the S arrivals reduces in order
    if (S > 1) {
      const int64_t tile_base = (int64_t)tile_id * S * (BM * BN);
      const int frag_base = (wave * TM * TN) * 64 + lane;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          *reinterpret_cast<v4f*>(p.ws + tile_base + (int64_t)split * (BM * BN) +
                                  (int64_t)(frag_base + (i * TN + j) * 64) * 4) = acc[i][j];
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const int old = atomicAdd(&p.counters[tile_id], 1);
        s_info = (old == S - 1);
      }
      __syncthreads();
      const int last = s_info;
      __syncthreads();
      if (!last) continue;
      __threadfence();
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
          for (int q = 0; q < S; ++q) {
            const v4f part = q == split ? acc[i][j]
                : *reinterpret_cast<const v4f*>(p.ws + tile_base + (int64_t)q * (BM * BN) +
                                                (int64_t)(frag_base + (i * TN + j) * 64) * 4);
            sum += part;
          }
          acc[i][j] = sum;
        }
      if (tid == 0) p.counters[tile_id] = 0;  // ready for the next call
    }

    // ---- epilogue: BF16 round-to-nearest-even, live rows only
    uint16_t* Dg = p.D + (p.kind == kMasked ? (int64_t)g * p.d_gstride : 0);
    int live_rows = p.M;
    if (p.kind == kMasked) live_rows = min(max(p.masked_m[g], 0), p.M);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WTM + 16 * i + (lane & 15);
      bool ok = m < live_rows;
      if (ok && p.kind == kContiguous) ok = p.m_indices[m] >= 0;
      if (!ok) continue;
      uint16_t* drow = Dg + (int64_t)m * p.ldd;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + 16 * j + 4 * (lane >> 4);
        const v4f v = acc[i][j];
        if (p.vec_store && n + 3 < p.N) {
          const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
          const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(drow + n) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) drow[n + r] = (uint16_t)bf16_bits(v[r]);
        }
      }
    }
  }
}

}  // namespace fp8gemm
