// Device code of libfp8gemm: one kernel template serves the dense, M-grouped
// contiguous and M-grouped masked FP8 NT GEMMs (DeepGEMM overview page,
// deepep.org/zh/deepgemm, 核心优化技术: one scheduler for grouped and non-grouped
// kernels, rasterised for L2 reuse).
//
// Per work unit (one BM x BN output tile, or one K-slice of it under split-K):
//   a STAGES-deep ring of LDS stages, each holding one 128-wide K block: the A tile
//   [BM x 128 B], the B tile [BN x 128 B] and that block's scales. Stages are filled
//   by gfx950 direct-to-LDS loads (global_load_lds_dwordx4 / _dword), so up to
//   STAGES-1 K blocks are in flight per workgroup without holding any registers;
//   completion is tracked with explicit vmcnt waits and raw s_barrier.
//   For every K block kb:
//     t = v_mfma_f32_16x16x128_f8f6f4(B frag, A frag, 0)      -- exact FP8 products
//     acc += t * (sa[kb][m] * sb[n/128][kb])                   -- FP32 promotion
//   then round acc to BF16 (nearest-even) and store live rows.
// The promotion step is the pages' two-level accumulation (GeekNews topic 19444,
// intro; bquan.live post 9429818, "Comprender profundamente DeepGEMM"): every
// 128-K partial is scaled and added into an FP32 accumulator outside the matrix
// unit.
//
// MFMA operand roles: the MFMA's first operand carries 16 rows of B (n) and the
// second 16 rows of A (m), so lane l of a 16x16 result holds four B rows 4*(l/16)+r
// of one A row l%16: a single activation scale per lane. B rows are placed so that
// the lane's results of subtiles 2h and 2h+1 are eight consecutive output columns
// (b_col): one 16-byte BF16 store per lane, 64 contiguous bytes per row. Both
// operands use the same lane->K assignment, so the K order inside the MFMA is
// irrelevant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8gemm {

constexpr int kBlockK = 128;   // K extent of a scale block and of one MFMA
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
  int full_tiles;            // dense / contiguous: leading tiles of the work order computed
                             // whole; each later tile is split_k units (split-K)
  int num_units;             // dense / contiguous: tiles * split_k (masked: computed on device)
  int group_m;               // raster group height in tiles
  int vec_store;             // widest D store: 2 = 16 bytes (ldd % 8 == 0, D 16-byte aligned),
                             // 1 = 8 bytes (ldd % 4 == 0, D 8-byte aligned), 0 = 2 bytes
  const uint16_t* C;         // optional BF16 addend of D = C + A B^T (nullptr: none); may alias D
  int64_t ldc, c_gstride;    // C row stride, per-group stride (masked)
  int c_vec;                 // 1: C rows allow 16-byte loads (ldc % 8 == 0, C 16-byte aligned)
  int sf_packed;             // E8: sa / sb hold packed UE8M0 words (the codes of K blocks 4w..4w+3
                             // in bytes 0..3 of word w) instead of FP32 powers of two
  int sb_kstride;            // entries per weight-scale row: K/128 (FP32) or ceil(K/512) (packed)
  float* ws;                 // split-K partials [split tile][split][BM*BN]
  int32_t* counters;         // split-K arrival counters [split tile]
  int ws_tiles;              // split tiles the workspace holds (masked: a call whose live tiles exceed
                             // it runs unsplit)
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Two FP32 values to packed BF16 bits (a in the low half), rounded to nearest even by
// one v_cvt_pk_bf16_f32. The kernel's float mode keeps FP32 denormals, so subnormal
// results round like normal ones; values past the BF16 range become infinities. (NaN
// inputs are outside the interface contract.)
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
}

// Eight BF16 values (packed in w, lowest column first) to dst[0..7], of which only the
// first `left` columns exist; `vec` is the widest store the row alignment allows.
__device__ __forceinline__ void store_edge(uint16_t* dst, uint4 w, int left, int vec) {
  if (left >= 8 && vec == 2) {
    *reinterpret_cast<uint4*>(dst) = w;
  } else if (left >= 8 && vec == 1) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);
    *reinterpret_cast<uint2*>(dst + 4) = make_uint2(w.z, w.w);
  } else {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < left) dst[c] = (uint16_t)(d[c >> 1] >> (16 * (c & 1)));
  }
}

// D = C + A B^T: add the BF16 addend of eight consecutive output columns (the lane's
// u = columns 0..3, v = columns 4..7) of which only the first `left` exist; `vec` allows
// one 16-byte load. Each lane reads only the C elements of the D elements it writes, so
// C may be D itself.
__device__ __forceinline__ float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ void add_c(v4f& u, v4f& v, const uint16_t* src, int left, int vec) {
  if (left >= 8 && vec) {
    const uint4 c = *reinterpret_cast<const uint4*>(src);
    u[0] += bf16_value(c.x & 0xFFFF), u[1] += bf16_value(c.x >> 16);
    u[2] += bf16_value(c.y & 0xFFFF), u[3] += bf16_value(c.y >> 16);
    v[0] += bf16_value(c.z & 0xFFFF), v[1] += bf16_value(c.z >> 16);
    v[2] += bf16_value(c.w & 0xFFFF), v[3] += bf16_value(c.w >> 16);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < left) u[c] += bf16_value(src[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c + 4 < left) v[c] += bf16_value(src[c + 4]);
  }
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

// LDS layout of the 128-byte operand rows of a stage. A fragment read (ds_read_b128)
// has 16 lanes fetch the same logical 16-byte chunk of 16 consecutive rows. Measured
// on gfx950 with the bank-conflict counter: such a read is conflict-free when each
// 8-lane half of the 16 lanes stays within one half of the 256-byte bank row
// (address bit 7), the two halves take opposite halves, and the lanes of a half use
// distinct 16-byte positions. So within every block of 16 rows, rows 0-7 are stored
// at the even row positions and rows 8-15 at the odd ones (lds_row), and chunk c of
// row r sits at chunk position c ^ (r & 7).
__device__ __forceinline__ int lds_row(int r) { return (r & ~15) | ((r & 7) << 1) | ((r >> 3) & 1); }
// output column (within the tile) of logical B row x: inside each 32-row group,
// row 16j' + 4q + r (j' = 0, 1) holds column 8q + 4j' + r, so a lane's four rows of
// subtile 2h and of 2h+1 are the eight columns 32h + 8q .. 32h + 8q + 7
__device__ __forceinline__ int b_col(int x) {
  return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
// the logical row stored at LDS row position R (inverse of lds_row)
__device__ __forceinline__ int row_at(int R) { return (R & ~15) | ((R >> 1) & 7) | ((R & 1) << 3); }
__device__ __forceinline__ int swz_key(int row) { return row & 7; }
__device__ __forceinline__ int swz(int row, int c) { return lds_row(row) * kBlockK + ((c ^ swz_key(row)) << 4); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima). The s_waitcnt builtin
// orders nothing for the compiler, so every wait sits between scheduling barriers
// (no instruction moves across) and memory clobbers: work written before the wait
// in source order executes before it, work written after it executes after it.
__device__ __forceinline__ void fence_schedule() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  fence_schedule();
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  fence_schedule();
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  fence_schedule();
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
  fence_schedule();
}

// Workgroup barrier without the memory fence of __syncthreads (which would drain
// every outstanding load); the empty asm keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier() {
  fence_schedule();
  __builtin_amdgcn_s_barrier();
  fence_schedule();
}

// 32-bit LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wave-uniform copies of values the compiler cannot prove uniform (a value read from
// LDS, an index derived from threadIdx.x >> 6), so they and everything computed from
// them live in scalar registers; a no-op on values already known to be uniform.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ const T* uni(const T* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Direct-to-LDS loads: every lane reads `bytes` from its own global address and the
// wave writes them to LDS at m0 + lane * bytes. Issued as asm so the compiler does
// not treat them as LDS stores it must drain before every LDS read; completion is
// tracked by the caller's explicit vmcnt waits. The address is a wave-uniform base
// in scalar registers plus a per-lane 32-bit byte offset, so advancing a K block
// and setting m0 cost only scalar instructions.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(uni(base)), "s"(uni((int)lds)) : "memory");
}
// The same with the non-temporal hint: lines streamed through once (an operand that no
// other tile reads) need not displace reusable lines from the caches.
__device__ __forceinline__ void dma16nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(uni(base)), "s"(uni((int)lds)) : "memory");
}
// 4-byte loads with a per-lane 64-bit address (the scale loads, whose lanes read
// scattered rows)
__device__ __forceinline__ void dma4v(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(uni((int)lds)) : "memory");
}

// Wait until at most min(n, MAXN) groups of LPS loads are outstanding.
template <int LPS, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<LPS * MAXN>();
    else wait_stages<LPS, MAXN - 1>(n);
  }
}

// Split-K: publish this split's partial (acc, each 16x16 result stored lane-major at
// frag_base + (t * TN + j) * 64 in units of 4 floats) and count the arrival; the last
// of the S arrivals reads the other partials and sums all S in split order into acc,
// then resets the counter. Returns true for the workgroup that writes the tile.
// Every thread of the workgroup calls it (it contains workgroup barriers).
// Partials move as device-coherent (sc1) 16-byte buffer accesses, one kilobyte of
// contiguous lines per instruction; the last arrival issues all loads of a partial
// before adding any of them, so each partial costs one round trip.
// ws: the partials [split tile][S][tile_floats]; counters: one per split tile.
// live_t (wave-uniform): only the fragments of rows t < live_t hold output rows, the
// others lie past M; they are neither published nor read (their sums are never stored).
template <int TM, int TN>
__device__ __forceinline__ bool reduce_splits(float* ws, int32_t* counters, v4f (&acc)[TM][TN], int ws_id,
                                              int split, int S, int frag_base, int tile_floats, int tid,
                                              int* s_flag, int live_t = TM) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  constexpr int kDeviceScope = 16;       // buffer cache policy: sc1
  constexpr int kRawDword3 = 0x00020000;  // buffer descriptor word 3: 32-bit data, untyped access
  float* tile_ws = const_cast<float*>(uni((const float*)(ws + (int64_t)ws_id * S * tile_floats)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(tile_ws, 0, S * tile_floats * 4, kRawDword3);
  auto offset = [&](int q, int t, int j) { return (q * tile_floats + (frag_base + (t * TN + j) * 64) * 4) * 4; };
#pragma unroll
  for (int t = 0; t < TM; ++t)
    if (t < live_t)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[t][j]), rs, offset(split, t, j), 0,
                                               kDeviceScope);
  wait_vmcnt<0>();  // the partial has reached the device-coherent level
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[ws_id], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old == S - 1);
  }
  __syncthreads();
  const int last = *s_flag;
  __syncthreads();
  if (!last) return false;
  v4f sum[TM][TN];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int j = 0; j < TN; ++j) sum[t][j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < S; ++q) {
    if (q == split) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j) sum[t][j] += acc[t][j];
    } else {
      v4f part[TM][TN];
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          part[t][j] = t < live_t ? __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                                rs, offset(q, t, j), 0, kDeviceScope))
                                  : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j) sum[t][j] += part[t][j];
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[t][j] = sum[t][j];
  if (tid == 0) __hip_atomic_store(&counters[ws_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// BM x BN tile, WAVES_M x WAVES_N wave64s (4 or 8), STAGES-deep LDS ring; MASKED
// instances carry the per-group live-tile table.
// E8 instances take power-of-two scales (UE8M0 values 2^(e-127) held as FP32) and give
// their 8-bit exponents to gfx950's block-scaled MFMA, which multiplies each 128-K
// block product by 2^(ea-127) * 2^(eb-127) and adds it to the FP32 accumulator itself:
// the promotion needs no separate FMAs.
// HAS_C instances add the BF16 C of D = C + A B^T in the epilogue (p.C non-null).
// STREAM_B instances load B with the non-temporal hint, for calls where one tile row
// covers all of M, so that every B tile is read by exactly one work unit: streaming it
// past the caches keeps A's lines, which every unit reads, resident (measured on the
// few-row shapes: up to 22% faster; where B tiles are shared it is slower).
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool MASKED, bool E8 = false, bool HAS_C = false,
          bool STREAM_B = false>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, 1) fp8_gemm_kernel(const Params p) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int NT = NW * 64;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  constexpr int WTM = BM / WAVES_M;  // wave tile rows
  constexpr int WTN = BN / WAVES_N;  // wave tile cols
  constexpr int TM = WTM / 16;
  constexpr int TN = WTN / 16;
  static_assert(TM >= 1 && TN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(TN % 2 == 0, "subtiles pair up into 16-byte stores");
  // Weight scales per wave and K block: one when the wave's columns lie in one 128-column
  // scale block (tile widths that are multiples or divisors of 128). Other widths (block
  // sizes not aligned to the scale blocks, as on the DeepGEMM overview page,
  // deepep.org/zh/deepgemm, 非对齐块大小: 96 columns make 256 tiles of N=24576) start
  // tiles inside a scale block; there each 32-column pair of subtiles takes its own scale
  // (32 divides both the tile width and 128, so a pair never straddles two blocks).
  constexpr bool SB_ONE = (BN % kBlockK == 0 || kBlockK % BN == 0) && kBlockK % WTN == 0;
  constexpr int NSB = SB_ONE ? 1 : TN / 2;
  static_assert(SB_ONE || BN % 32 == 0, "unaligned tile widths are multiples of 32");
  static_assert((BM * kBlockK) % (1024 * NW) == 0 && (BN * kBlockK) % (1024 * NW) == 0, "tile load split");
  static_assert(STAGES >= 2, "pipeline depth");
  constexpr int A_BYTES = BM * kBlockK;
  constexpr int B_BYTES = BN * kBlockK;
  // Scales of a stage: the BM activation scales, ordered so that the TM scales a lane
  // needs (rows wm*WTM + 16t + frow, t < TM) are adjacent (one vector read), then 64
  // slots for the weight scales of the tile's 128-column blocks. Waves below SA_WAVES
  // each load 64 activation scales, the others the weight scales (identical copies),
  // so every wave issues one scale load per stage.
  constexpr int SA_WAVES = BM / 64;
  static_assert(BM % 64 == 0 && SA_WAVES < NW, "scale loads");
  static_assert(TM == 1 || TM == 2 || TM == 4, "activation scales per lane: one vector read");
  constexpr int SC_FLOATS = BM + 64;
  constexpr int STAGE = A_BYTES + B_BYTES + SC_FLOATS * 4;
  constexpr int A_INSTR = A_BYTES / (1024 * NW);    // 1 KB direct-to-LDS loads per wave per stage
  constexpr int B_INSTR = B_BYTES / (1024 * NW);
  constexpr int LPS = A_INSTR + B_INSTR + 1;
  static_assert(LPS * (STAGES - 1) < 64, "vmcnt capacity");

  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * STAGE];
  __shared__ int s_pre[MASKED ? kMaxGroups + 1 : 1];  // masked: prefix sums of live m-tiles per group
  __shared__ int s_info;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  int S = p.split_k;

  // ---- masked: live m-tiles per group, exclusive prefix sum in LDS
  int num_units = p.num_units;
  if constexpr (MASKED) {
    constexpr int PER = (kMaxGroups + NT - 1) / NT;
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
    __shared__ int s_scan[NT];
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
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
    if (tid == NT - 1) s_pre[min(p.G, kMaxGroups)] = s_scan[NT - 1];
    __syncthreads();
    // the live tiles are known only here: split K only if the workspace holds them all
    // (the same decision in every workgroup)
    const int live_total = uni(s_pre[p.G]) * p.tiles_n;
    if (S > 1 && live_total > p.ws_tiles) S = 1;
    num_units = live_total * S;
  }

  for (int u = blockIdx.x; u < num_units; u += gridDim.x) {
    // whole tiles and split units are remapped separately, so the split units (a
    // last, partial round of tiles cut into K slices) stay in the last round
    int L;
    if (!MASKED && p.full_tiles > 0 && p.full_tiles < num_units)
      L = u < p.full_tiles ? xcd_remap(u, p.full_tiles)
                           : p.full_tiles + xcd_remap(u - p.full_tiles, num_units - p.full_tiles);
    else
      L = xcd_remap(u, num_units);
    int g = 0, tm, tn, split;
    int S_u = S;       // splits of this unit's tile
    int ws_id = 0;     // slot of a split tile in the workspace
    if constexpr (MASKED) {
      // units of one (group, n-tile) are contiguous: the group's B tile is reused
      int lo = 0, hi = p.G;  // largest g with s_pre[g] * tiles_n * S <= L
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] * p.tiles_n * S <= L) lo = mid; else hi = mid;
      }
      g = uni(lo);
      const int pre = uni(s_pre[g]);
      const int live_tiles = uni(s_pre[g + 1]) - pre;
      const int local = L - pre * p.tiles_n * S;
      tn = local / (live_tiles * S);
      const int r = local - tn * live_tiles * S;
      tm = r / S;
      split = r - tm * S;
      ws_id = pre * p.tiles_n + tn * live_tiles + tm;  // this live tile's slot, < live_total
    } else {
      // the first full_tiles tiles are single units; each later one is S units, so a
      // last partial round of tiles can be spread over all CUs as K slices. Split
      // units are numbered split-major: the units next to each other (on one XCD)
      // are neighbouring tiles at the same K slice, which share A and B rows in L2
      // as the tiles of a whole round do.
      int tile;
      if (L < p.full_tiles) {
        tile = L;
        split = 0;
        S_u = 1;
      } else {
        const int split_tiles = (num_units - p.full_tiles) / S;
        const int l = L - p.full_tiles;
        split = l / split_tiles;
        ws_id = l - split * split_tiles;
        tile = p.full_tiles + ws_id;
      }
      raster(tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    }
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // ---- contiguous: expert of this row block, the largest m_indices entry of its rows
    // (-1 everywhere = padding only: nothing to do). Each wave reduces it on its own, with
    // cross-lane shuffles: no LDS and no workgroup barrier.
    if (p.kind == kContiguous) {
      int e = -1;
      for (int r = lane; r < BM; r += 64)
        if (m0 + r < p.M) e = max(e, p.m_indices[m0 + r]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) e = max(e, __shfl_xor(e, off, 64));
      g = uni(e);
      if (g < 0 || g >= p.G) continue;  // all padding (or an invalid id): nothing to write
    }

    const int kb0 = S_u > 1 ? split * p.kb_per_split : 0;
    const int nk = S_u > 1 ? min(p.num_kb, kb0 + p.kb_per_split) - kb0 : p.num_kb;
    const uint8_t* Ag = uni(p.A + (MASKED ? (int64_t)g * p.a_gstride : 0) + (int64_t)kb0 * kBlockK);
    // scale rows: one per K block (FP32), or one word row per four K blocks (packed UE8M0)
    const bool packed = E8 && p.sf_packed;
    const int kw0 = packed ? kb0 >> 2 : kb0;
    const float* sag = uni(p.sa + (MASKED ? (int64_t)g * p.sa_gstride : 0) + (int64_t)kw0 * p.ld_sa);
    const uint8_t* Bg = uni(p.B + (int64_t)g * p.b_gstride + (int64_t)kb0 * kBlockK);
    const float* sbg = uni(p.sb + (int64_t)g * p.sb_gstride + kw0);

    // ---- direct-to-LDS load plan. Load instruction r of this wave fills LDS row
    // positions 8*grp .. 8*grp+7 (1 KB) of a stage: lane l writes chunk position l & 7
    // of position 8*grp + l/8, so it brings the row stored there (row_at) and that
    // row's logical chunk (l & 7) ^ swz_key(row) (the layout above).
    const int lrow = lane >> 3;
    uint32_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
    for (int r = 0; r < A_INSTR; ++r) {
      const int row = row_at((r * NW + wave) * 8 + lrow);
      const int grow = min(m0 + row, p.M - 1);  // rows past the end: clamped, results unused
      a_off[r] = (uint32_t)(grow * p.lda) + (((lane & 7) ^ swz_key(row)) << 4);
    }
#pragma unroll
    for (int r = 0; r < B_INSTR; ++r) {
      const int row = row_at((r * NW + wave) * 8 + lrow);
      const int grow = min(n0 + b_col(row), p.N - 1);
      b_off[r] = (uint32_t)(grow * p.ldb) + (((lane & 7) ^ swz_key(row)) << 4);
    }
    // scale load of this wave (layout above): lane l of activation-scale wave w fills
    // slot 64w + l, which holds row wm*WTM + 16t + frow for slot wm*WTM + frow*TM + t;
    // lane l of a weight-scale wave brings the scale of the tile's 128-column block l
    // (spare lanes repeat the last block)
    const float* sc_src;
    int64_t sc_step;  // per K block
    if (wave < SA_WAVES) {
      const int slot = wave * 64 + lane;
      const int rem = slot % WTM;
      const int row = (slot / WTM) * WTM + 16 * (rem % TM) + rem / TM;
      sc_src = sag + min(m0 + row, p.M - 1);
      sc_step = p.ld_sa;
    } else {
      // the scale blocks the tile's columns touch: BN / 128, or, where a tile may start
      // inside a block, one more than the blocks its width spans (slot nb holds block
      // n0 / 128 + nb)
      constexpr int NB = SB_ONE ? (BN >= kBlockK ? BN / kBlockK : 1) : (BN + kBlockK - 1) / kBlockK + 1;
      const int nb = min(lane, NB - 1);
      sc_src = sbg + (int64_t)(min(n0 + nb * kBlockK, p.N - 1) / kBlockK) * p.sb_kstride;
      sc_step = 1;
    }

    const uint32_t ring = lds_addr(smem);
    // load item q (0 <= q < LPS) of K block kb0 + i into `stage`: A rows, B rows, scales
    auto issue_item = [&](int i, int stage, int q) {
      const uint32_t base = ring + stage * STAGE;
      if (q < A_INSTR) {
        dma16(Ag + (int64_t)i * kBlockK, a_off[q], base + (q * NW + wave) * 1024);
      } else if (q < A_INSTR + B_INSTR) {
        const int r = q - A_INSTR;
        if constexpr (STREAM_B)
          dma16nt(Bg + (int64_t)i * kBlockK, b_off[r], base + A_BYTES + (r * NW + wave) * 1024);
        else
          dma16(Bg + (int64_t)i * kBlockK, b_off[r], base + A_BYTES + (r * NW + wave) * 1024);
      } else {
        dma4v(sc_src + (packed ? ((kb0 + i) >> 2) - kw0 : i) * sc_step,
              base + A_BYTES + B_BYTES + (wave < SA_WAVES ? wave * 256 : BM * 4));
      }
    };
    auto issue = [&](int i, int stage) {
#pragma unroll
      for (int q = 0; q < LPS; ++q) issue_item(i, stage, q);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;          // fragment row within a 16-row subtile
    const int fchunk = (lane >> 4) * 2;  // first of the lane's two 16-byte K chunks
    // fragments and scales of one stage, read from LDS into registers. Read item q:
    // B fragments first, then the scales, then the A fragments, so a compute that
    // starts before all reads have landed needs only the oldest ones.
    // Double-buffered fragments only where the registers allow it (4 waves with
    // wave tiles up to 64x64); otherwise one buffer read just before its compute.
    constexpr bool DB = NW == 4 && TM * TN <= 16;
    constexpr int NBUF = DB ? 2 : 1;
    constexpr int NREAD = TN + 1 + TM;
    v8i fa[NBUF][TM], fb[NBUF][TN];
    float sa_r[NBUF][TM], sb_r[NBUF][NSB];  // raw scales; multiplied only once the stage is consumed
    auto read_item = [&](int stage, auto buf_c, int q) {
      constexpr int buf = decltype(buf_c)::value;
      const uint8_t* sA = smem + stage * STAGE;
      const uint8_t* sB = sA + A_BYTES;
      const float* sS = reinterpret_cast<const float*>(sB + B_BYTES);
      if (q < TN) {
        const int row = wn * WTN + 16 * q + frow;
        const v4i lo = *reinterpret_cast<const v4i*>(sB + swz(row, fchunk));
        const v4i hi = *reinterpret_cast<const v4i*>(sB + swz(row, fchunk + 1));
        fb[buf][q] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else if (q == TN) {
        if constexpr (SB_ONE) {
          sb_r[buf][0] = sS[BM + (wn * WTN) / kBlockK];
        } else {
#pragma unroll
          for (int h = 0; h < NSB; ++h) sb_r[buf][h] = sS[BM + ((n0 + wn * WTN + 32 * h) >> 7) - (n0 >> 7)];
        }
        const float* sa_p = sS + wm * WTM + frow * TM;
        if constexpr (TM == 4) {
          const v4f v = *reinterpret_cast<const v4f*>(sa_p);
#pragma unroll
          for (int t = 0; t < TM; ++t) sa_r[buf][t] = v[t];
        } else if constexpr (TM == 2) {
          const float2 v = *reinterpret_cast<const float2*>(sa_p);
          sa_r[buf][0] = v.x;
          sa_r[buf][1] = v.y;
        } else {
          sa_r[buf][0] = sa_p[0];
        }
      } else {
        const int t = q - TN - 1;
        const int row = wm * WTM + 16 * t + frow;
        const v4i lo = *reinterpret_cast<const v4i*>(sA + swz(row, fchunk));
        const v4i hi = *reinterpret_cast<const v4i*>(sA + swz(row, fchunk + 1));
        fa[buf][t] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    auto read_stage = [&](int stage, auto buf_c) {
#pragma unroll
      for (int q = 0; q < NREAD; ++q) read_item(stage, buf_c, q);
    };
    // One K block from registers, as TM*TN slots. Slot k issues MFMA k (A subtile
    // k / TN, B subtile k % TN), then `side(k)` (this slot's share of the global and
    // LDS traffic of the iteration), then the promotion FMAs of MFMA k-2, whose
    // result is ready by then. Scheduling barriers keep the slots in this order so
    // the load traffic runs in the matrix unit's shadow.
    constexpr int NMF = TM * TN;
    // kbi: the computed stage's K block, counted from kb0 (selects a packed code's byte)
    auto compute = [&](auto buf_c, auto&& side, int kbi) {
      constexpr int buf = decltype(buf_c)::value;
      if constexpr (E8) {
        // scale operands: the exponent byte of each power-of-two scale (the E8M0 code);
        // the first MFMA operand (B rows) takes the tile's weight scale, the second
        // (A rows) the activation scale of the lane's row
        // (an FP32 power of two carries its code in the exponent field, bits 23..30; a
        // packed word carries K block 4w + j's code in byte j)
        const int sh = packed ? 8 * ((kb0 + kbi) & 3) : 23;
        int ea[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) ea[t] = (__float_as_int(sa_r[buf][t]) >> sh) & 0xFF;
        int eb[NSB];
#pragma unroll
        for (int h = 0; h < NSB; ++h) eb[h] = (__float_as_int(sb_r[buf][h]) >> sh) & 0xFF;
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          const int t = k / TN, j = k % TN;
          acc[t][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[buf][j], fa[buf][t], acc[t][j], 0, 0,
                                                                       0, eb[SB_ONE ? 0 : j / 2], 0, ea[t]);
          side(k);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      float sc[TM][NSB];
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int h = 0; h < NSB; ++h) sc[t][h] = sa_r[buf][t] * sb_r[buf][h];
      v4f r[NMF];
      auto promote = [&](int k) {
        const int t = k / TN, j = k % TN;
        const float f = sc[t][SB_ONE ? 0 : j / 2];
        const v4f v = r[k];
        acc[t][j][0] = __builtin_fmaf(v[0], f, acc[t][j][0]);
        acc[t][j][1] = __builtin_fmaf(v[1], f, acc[t][j][1]);
        acc[t][j][2] = __builtin_fmaf(v[2], f, acc[t][j][2]);
        acc[t][j][3] = __builtin_fmaf(v[3], f, acc[t][j][3]);
      };
#pragma unroll
      for (int k = 0; k < NMF; ++k) {
        r[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[buf][k % TN], fa[buf][k / TN], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        side(k);
        if (k >= 2) promote(k - 2);
        // within the slot the MFMA issues first and the promotion FMAs after it, two
        // MFMAs behind the result they read (left to itself the scheduler hoists them
        // above the MFMA, and a single wave then waits on every result)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (NMF >= 2) promote(NMF - 2);
      promote(NMF - 1);
    };
    // slot k of NMF gets items [k*n/NMF, (k+1)*n/NMF) of a list of n
    auto share = [](int k, int n, auto&& f) {
#pragma unroll
      for (int q = k * n / NMF; q < (k + 1) * n / NMF; ++q) f(q);
    };

    // all waves are done with the LDS ring of the previous unit before it is refilled
    wait_lgkmcnt0();
    barrier();
    if constexpr (DB) {
      // Fragments double-buffered in registers. Stage i lives in
      // slot i % STAGES; while computing stage i (from registers) the wave reads
      // stage i+1 into its other buffer, and the slot of stage i (already in
      // registers everywhere) is refilled with stage i + STAGES.
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s < nk) issue(s, s);
      wait_stages<LPS, STAGES - 1>(nk - 1);
      barrier();
      read_stage(0, std::integral_constant<int, 0>{});
      wait_lgkmcnt0();
      // MORE: stage i+1 exists (read it); REFILL: stage i+STAGES exists (load it).
      // Every step is one basic block: its waits have compile-time counts and nothing
      // in it branches. (Across a branch the compiler sinks a step's promotions, which
      // keeps every MFMA result live, and where differently compiled steps join it
      // copies the accumulators.)
      auto step_body = [&](int i, auto cur_c, auto more_c, auto refill_c) {
        constexpr int nxt = decltype(cur_c)::value ^ 1;
        constexpr bool MORE = decltype(more_c)::value;
        constexpr bool REFILL = decltype(refill_c)::value;
        if constexpr (MORE) {
          // stage i+1 is complete once at most min(STAGES-2, nk-2-i) later stages are
          // pending; with REFILL that is STAGES-2. Without, all loads were issued at
          // least STAGES-1 steps ago, so waiting for every one of them costs little.
          if constexpr (REFILL) wait_vmcnt<LPS * (STAGES - 2)>();
          else wait_vmcnt<0>();
          barrier();
        }
        const int rs = (i + 1) % STAGES, ws = i % STAGES;
        compute(cur_c, [&](int k) {
          if constexpr (REFILL) share(k, LPS, [&](int q) { issue_item(i + STAGES, ws, q); });
          if constexpr (MORE) share(k, NREAD, [&](int q) { read_item(rs, std::integral_constant<int, nxt>{}, q); });
        }, i);
        wait_lgkmcnt0();
      };
      using T = std::true_type;
      using F = std::false_type;
      // the steps after the last refill, starting from buffer parity P
      auto finish = [&](int i, auto par_c) {
        constexpr int P = decltype(par_c)::value;
        using C0 = std::integral_constant<int, P>;
        using C1 = std::integral_constant<int, P ^ 1>;
        for (; i + 2 < nk; i += 2) {
          step_body(i, C0{}, T{}, F{});
          step_body(i + 1, C1{}, T{}, F{});
        }
        if (i + 1 < nk) {
          step_body(i, C0{}, T{}, F{});
          step_body(i + 1, C1{}, F{}, F{});
        } else {
          step_body(i, C0{}, F{}, F{});
        }
      };
      int i = 0;
      for (; i + 1 + STAGES < nk; i += 2) {
        step_body(i, std::integral_constant<int, 0>{}, T{}, T{});
        step_body(i + 1, std::integral_constant<int, 1>{}, T{}, T{});
      }
      if (i + STAGES < nk) {  // one refilling step is left
        step_body(i, std::integral_constant<int, 0>{}, T{}, T{});
        finish(i + 1, std::integral_constant<int, 1>{});
      } else {
        finish(i, std::integral_constant<int, 0>{});
      }
    } else {
      // One register buffer per wave, 8 waves: ping-pong. Waves w and w + 4 share a
      // SIMD; group A (waves 0-3) and group B (waves 4-7) run half a step apart,
      // with a workgroup barrier between phases, so that in every phase one wave of
      // each SIMD computes a stage from registers (MFMAs and promotions only) while
      // the other reads its next stage from LDS and issues its share of the loads
      // of a later stage (a single computing wave is limited by its own instruction
      // issue, so everything else goes to the reading wave). Group B passes one
      // extra barrier before its K loop and group A one after it, so both pass
      // 2 nk + 1 barriers per unit. Phases, with BAR(n) the n-th barrier of the unit
      // and S = STAGES:
      //   A: wait(j) BAR(2j+1) read(j)+load(j+S-1) BAR(2j+2) compute(j)
      //   B: BAR(2j+2) read(j)+load(j+S-1) wait(j+1) BAR(2j+3) compute(j)
      // Stage j is read by A between BAR(2j+1) and BAR(2j+2) and by B between
      // BAR(2j+2) and BAR(2j+3); every wave has waited for its own loads of stage j
      // before BAR(2j+1). Stage j+S-1 goes to the slot of stage j-1, which both
      // groups finished reading by BAR(2j+1). Both prologues load stages
      // 0 .. S-2, so each wave's wait leaves exactly its S - 2 later stages in
      // flight in the steady state.
      static_assert(NW == 8, "single-buffered tiles use 8 waves");
      const bool group_b = wave >= NW / 2;
      using C0 = std::integral_constant<int, 0>;
      // read stage j into registers and, with REFILL, load stage `ld` of this wave
      auto phase_read = [&](int j, int ld, auto refill_c) {
        constexpr bool REFILL = decltype(refill_c)::value;
        read_stage(j % STAGES, C0{});
        if constexpr (REFILL) issue(ld, ld % STAGES);
        wait_lgkmcnt0();
      };
      auto phase_compute = [&](int j) { compute(C0{}, [](int) {}, j); };
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s, s);
      if (!group_b) {
        // stage j is complete once min(STAGES-2, nk-1-j) later stages of this wave are
        // pending: STAGES-2 while refills continue, else wait for all (one basic block
        // per phase, as in the double-buffered path)
        int j = 0;
        for (; j + STAGES - 1 < nk; ++j) {
          wait_vmcnt<LPS * (STAGES - 2)>();
          barrier();
          phase_read(j, j + STAGES - 1, std::true_type{});
          barrier();
          phase_compute(j);
        }
        for (; j < nk; ++j) {
          wait_vmcnt<0>();
          barrier();
          phase_read(j, 0, std::false_type{});
          barrier();
          phase_compute(j);
        }
        barrier();
      } else {
        wait_stages<LPS, STAGES - 2>(nk - 1);  // stage 0
        barrier();
        int j = 0;
        for (; j + STAGES - 1 < nk; ++j) {
          barrier();
          phase_read(j, j + STAGES - 1, std::true_type{});
          wait_vmcnt<LPS * (STAGES - 2)>();  // stage j + 1
          barrier();
          phase_compute(j);
        }
        for (; j < nk; ++j) {
          barrier();
          phase_read(j, 0, std::false_type{});
          wait_vmcnt<0>();
          barrier();
          phase_compute(j);
        }
      }
    }

    // ---- split-K: the last of the S arrivals writes the tile
    if (S_u > 1 && !reduce_splits(p.ws, p.counters, acc, ws_id, split, S_u, (wave * TM * TN) * 64 + lane, BM * BN, tid, &s_info))
      continue;

    // ---- epilogue: BF16 round-to-nearest-even, live rows only; subtiles 2h and 2h+1
    // of a lane are eight consecutive columns (b_col)
    uint16_t* Dg = p.D + (MASKED ? (int64_t)g * p.d_gstride : 0);
    const uint16_t* Cg = HAS_C ? p.C + (MASKED ? (int64_t)g * p.c_gstride : 0) : nullptr;
    int live_rows = p.M;
    if (MASKED) live_rows = min(max(p.masked_m[g], 0), p.M);
    const bool full = p.vec_store == 2 && n0 + BN <= p.N;  // no column edge in this tile
    const int ncol = n0 + wn * WTN + 8 * (lane >> 4);
    if constexpr (HAS_C) {
      bool okv[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = m0 + wm * WTM + 16 * t + (lane & 15);
        bool ok = m < live_rows;
        if (ok && p.kind == kContiguous) ok = p.m_indices[m] >= 0;
        okv[t] = ok;
      }
      // a lane issues all of its 16-byte C loads before any of its stores (C may be D,
      // so the compiler would otherwise keep each load behind the previous store); edge
      // tiles and unaligned C load element by element in add_c
      const bool cfast = full && p.c_vec;
      uint4 cv[TM][TN / 2];
      if (cfast) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
          if (okv[t]) {
            const uint16_t* crow = Cg + (int64_t)(m0 + wm * WTM + 16 * t + (lane & 15)) * p.ldc + ncol;
#pragma unroll
            for (int h = 0; h < TN / 2; ++h) cv[t][h] = *reinterpret_cast<const uint4*>(crow + 32 * h);
          }
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = m0 + wm * WTM + 16 * t + (lane & 15);
        if (!okv[t]) continue;
        uint16_t* drow = Dg + (int64_t)m * p.ldd + ncol;
#pragma unroll
        for (int h = 0; h < TN / 2; ++h) {
          v4f u = acc[t][2 * h], v = acc[t][2 * h + 1];
          if (cfast) {
            const uint4 c = cv[t][h];
            u[0] += bf16_value(c.x & 0xFFFF), u[1] += bf16_value(c.x >> 16);
            u[2] += bf16_value(c.y & 0xFFFF), u[3] += bf16_value(c.y >> 16);
            v[0] += bf16_value(c.z & 0xFFFF), v[1] += bf16_value(c.z >> 16);
            v[2] += bf16_value(c.w & 0xFFFF), v[3] += bf16_value(c.w >> 16);
          } else {
            add_c(u, v, Cg + (int64_t)m * p.ldc + ncol + 32 * h, p.N - (ncol + 32 * h), p.c_vec);
          }
          const uint4 w = make_uint4(bf16x2_bits(u[0], u[1]), bf16x2_bits(u[2], u[3]), bf16x2_bits(v[0], v[1]),
                                     bf16x2_bits(v[2], v[3]));
          if (full)
            *reinterpret_cast<uint4*>(drow + 32 * h) = w;
          else
            store_edge(drow + 32 * h, w, p.N - (ncol + 32 * h), p.vec_store);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = m0 + wm * WTM + 16 * t + (lane & 15);
        bool ok = m < live_rows;
        if (ok && p.kind == kContiguous) ok = p.m_indices[m] >= 0;
        if (!ok) continue;
        uint16_t* drow = Dg + (int64_t)m * p.ldd + ncol;
#pragma unroll
        for (int h = 0; h < TN / 2; ++h) {
          const v4f u = acc[t][2 * h], v = acc[t][2 * h + 1];
          const uint4 w = make_uint4(bf16x2_bits(u[0], u[1]), bf16x2_bits(u[2], u[3]), bf16x2_bits(v[0], v[1]),
                                     bf16x2_bits(v[2], v[3]));
          if (full)
            *reinterpret_cast<uint4*>(drow + 32 * h) = w;
          else
            store_edge(drow + 32 * h, w, p.N - (ncol + 32 * h), p.vec_store);
        }
      }
    }
  }
}

}  // namespace fp8gemm
