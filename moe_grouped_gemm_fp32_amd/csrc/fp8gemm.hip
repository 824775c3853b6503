// Host side of libfp8gemm: argument checks, tile/split selection, persistent-grid
// sizing and launch of the gfx950 kernels behind the C ABI in include/fp8gemm.h.
//
// Tile selection follows the pages' point that block shape, stage count and grid
// should be chosen per shape so every compute unit has work (bquan.live post
// 9429818, "¿Cómo usarlo?": dynamic block size / pipeline stage choice;
// deepep.org/zh/deepgemm, 非对齐块大小: pick tiles that keep more SMs busy). On
// MI355X that means filling 256 CUs: small-M shapes split K across workgroups and
// reduce the FP32 partials in a fixed order; large shapes use 128x128 tiles.
#include "fp8gemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "fp8gemm_kernel.hpp"
#include "fp8kgroup_kernel.hpp"
#include "fp8quant_kernel.hpp"

namespace {

using fp8gemm::Params;

constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256;

struct DeviceInfo {
  int cus = 0;
  int status = 1;          // 1 = not queried, FP8GEMM_OK or FP8GEMM_ERR_DEVICE
  void* scratch = nullptr;  // device address of this device's copy of `scratch` (set up on first use)
};
DeviceInfo g_devices[kMaxDevices];
std::mutex g_dev_mutex;
std::atomic<int> g_num_cus_override{0};
bool g_forced = false;
fp8gemm_config_t g_forced_cfg{};
std::atomic<uint32_t> g_forced_epoch{0};  // advanced by every fp8_gemm_force_config call

int query_device(int* cus_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8GEMM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& d = g_devices[dev];
  if (d.status == 1) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      d.status = FP8GEMM_ERR_DEVICE;
    } else {
      d.cus = prop.multiProcessorCount;
      d.status = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? FP8GEMM_OK : FP8GEMM_ERR_DEVICE;
    }
  }
  *cus_out = d.cus;
  return d.status;
}

// CU count used for sizing: the override if set, else the device's (or the
// MI355X default when no device is current, e.g. for host-only queries).
int effective_cus(bool need_device, int* status) {
  *status = FP8GEMM_OK;
  int cus = 0;
  if (need_device) {
    *status = query_device(&cus);
    if (*status != FP8GEMM_OK) return 0;
  }
  const int ov = g_num_cus_override.load();
  if (ov > 0) return need_device ? std::min(ov, cus) : ov;
  return cus > 0 ? cus : kDefaultCus;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K scratch of fp8_gemm_nt_noalloc, for callers that cannot allocate: one copy per
// device, held until the process ends. Its first kCounterBytes are the arrival counters
// (the workspace layout below), the rest holds FP32 partials. In host code `scratch`
// names only a host-side stand-in: kernels get the device address that
// hipGetSymbolAddress returns (cached per device in DeviceInfo::scratch).
constexpr size_t kScratchPartialBytes = (size_t)32 << 20;  // covers every plan of the dense configurations


struct Plan {
  int bm = 128, bn = 128, split = 1, kbps = 1, tiles_m = 0, tiles_n = 0;
  int64_t ws_tiles = 0;  // split tiles the workspace is sized for
  int64_t full = 0;  // leading tiles computed whole (the others are split `split` ways)
  int64_t units = 0;
  int grid = 0;
  size_t ws_bytes = 0;
};

// Compiled variants: tile shape, wave layout (4 or 8 wave64s) and LDS ring depth. One
// workgroup runs per CU (the persistent grid has one per CU). Most rings fill the LDS;
// the 64x64 and 128x96 tiles, which serve few-row calls whose units hold few K blocks,
// keep 4 and 3 stages: with the full 8 and 5, each unit's first stage waits behind more
// loads issued at once (measured on the six 64x64 and two 128x96 few-row shapes: 3-6%
// faster with the shallower rings).
struct Variant {
  int bm, bn, waves_m, waves_n, stages;
};
// The 96-column tiles (4 waves stacked along M) make 256 tiles of N=24576.
constexpr Variant kVariants[] = {
    {64, 64, 2, 2, 4},  {128, 64, 2, 2, 6},  {64, 128, 2, 2, 6},  {128, 128, 2, 2, 4},
    {256, 128, 4, 2, 3}, {128, 256, 2, 4, 3}, {64, 96, 4, 1, 7},   {128, 96, 4, 1, 3}};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
constexpr int kOccupancy = 1;

bool has_kernel(int bm, int bn) {
  for (const auto& v : kVariants)
    if (v.bm == bm && v.bn == bn) return true;
  return false;
}

// Split-K workspace layout: a fixed block of kMaxSplitTiles int32 arrival counters at
// offset 0, then the FP32 partials [split tile][split][BM*BN]. The counters sit at the
// same place whatever the plan, so calls of different shapes (different tiles and
// splits) can share one workspace: every counter is zero before a call and is zero again
// when it completes (the last arrival resets it). The partials need no initial value:
// each call writes a partial before any workgroup reads it.
constexpr int64_t kMaxSplitTiles = 4096;
constexpr size_t kCounterBytes = (size_t)kMaxSplitTiles * sizeof(int32_t);  // 16 KiB
static_assert(kCounterBytes % 256 == 0, "partials start 256-byte aligned");

constexpr size_t kScratchBytes = kCounterBytes + kScratchPartialBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Device address of the current device's scratch. On a device's first call it is
// looked up once (hipGetSymbolAddress, with that device current) and its counter block
// is cleared by a small kernel on `stream` (a kernel, not a memset, so the call may be
// captured into a graph); every later call that completes leaves the counters zero.
int scratch_for_current_device(void** out, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8GEMM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& d = g_devices[dev];
  if (!d.scratch) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP8GEMM_ERR_DEVICE;
    hipLaunchKernelGGL(zero_words, dim3(16), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                       (int)(kCounterBytes / sizeof(uint32_t)));
    if (hipGetLastError() != hipSuccess) return FP8GEMM_ERR_LAUNCH;
    d.scratch = ptr;
  }
  *out = d.scratch;
  return FP8GEMM_OK;
}

size_t split_ws_bytes(int64_t split_tiles, int split, int bm, int bn) {
  if (split <= 1) return 0;
  return kCounterBytes + (size_t)split_tiles * split * bm * bn * sizeof(float);
}

// Cost model of the planner (microseconds, fitted to timings on MI355X): per tile
// variant, the fixed cost of a work unit (pipeline fill and epilogue) and the time of
// one 128-wide K block, plus the extra cost of a split-K unit (publishing its partial,
// plus the last arrival reading the other partials). A call's estimate is
// rounds * (unit cost) with rounds = ceil(units / CUs), so the planner trades tile
// efficiency against filling all CUs (the unaligned-block argument of the pages:
// deepep.org/zh/deepgemm, 非对齐块大小).
// The constants were fitted to measured timings of every tile / split / whole-tile-round
// candidate of the 18 dense DeepSeek-V3-like shapes and the 10 masked decode cases, each
// timed inside the benchmark's sequence of calls (two runs averaged; bench.py --plan-sweep,
// the table in profiles/planner_sweep.json): with them the chosen plan is within 2.5% of
// the fastest measured one in all 28 cases.
constexpr double kSplitUnitUs = 3.0;
constexpr double kSplitReadUsPerKB = 0.03;
// A call also takes at least its HBM traffic (A, B and D once, plus the split-K
// partials, written and read once each) over an effective read rate, fitted like the
// constants above: 4.2 TB/s for dense calls, whose few-row shapes stream B once at up to
// 3.8-4.4 TB/s between back-to-back GEMMs, and 3.5 TB/s for the grouped calls. For the
// few-row shapes this bound decides between tiles and splits that the per-unit costs
// rank wrongly.
constexpr double kHbmBytesPerUs = 3.5e6;
constexpr double kDenseHbmBytesPerUs = 4.2e6;
constexpr int kMaxSplit = 8;
// Extra live M tiles per group the planner assumes for masked calls with several
// groups: their live rows differ, so ceil(masked_m / BM) averages above expected_m / BM
// (by half a tile for masked_m spread over [179, 333]); a quarter because the round-based
// estimate over-charges a nearly empty last round.
constexpr double kMaskedTileSlack = 0.25;
struct UnitCost {
  double fixed_us, kb_us;
};
UnitCost unit_cost(int bm, int bn) {
  if (bm == 64 && bn == 64) return {4.4, 0.37};
  if (bm == 128 && bn == 128) return {8.7, 0.64};
  if (bm == 128 && bn == 64) return {5.0, 0.60};
  if (bm == 64 && bn == 128) return {4.2, 0.59};
  if (bm == 256 && bn == 128) return {7.8, 0.85};
  if (bm == 64 && bn == 96) return {5.0, 0.49};
  if (bm == 128 && bn == 96) return {4.0, 0.56};
  return {8.3, 0.88};  // 128x256
}

// Masked calls learn their live rows on the device; their split-K workspace is sized for
// up to twice expected_m rows per group (masked_m spread around expected_m), and a call
// with more live tiles than that runs unsplit (the kernel decides).
int64_t masked_capacity_tiles(int G, int M_max, int N, int expected_m, int bm, int bn) {
  const int64_t rows = std::min<int64_t>(M_max, 2 * (int64_t)std::max(expected_m > 0 ? expected_m : M_max, 1));
  return (int64_t)G * ceil_div(rows, bm) * ceil_div(N, bn);
}

// Choose tile shape and split for a call. `rows` is M (dense), M_total
// (contiguous) or M_max (masked, where expected_m estimates the live rows).
Plan choose_uncached(int kind, int rows, int N, int K, int G, int expected_m, int cus, size_t ws_avail) {
  Plan pl;
  const int num_kb = K / fp8gemm::kBlockK;
  if (g_forced) {
    pl.bm = g_forced_cfg.block_m;
    pl.bn = g_forced_cfg.block_n;
    pl.split = std::max(1, g_forced_cfg.split_k);
    pl.full = std::max(0, g_forced_cfg.full_tiles);
  } else {
    double best = 1e30, best_units = 1e30;
    const bool masked = kind == FP8GEMM_KIND_MASKED;
    const int live = masked ? std::max(1, std::min(expected_m > 0 ? expected_m : rows, rows)) : rows;
    // candidate: `full` tiles computed whole, the other tiles split `split` ways
    auto consider = [&](const Variant& v, int64_t tiles, int split, int64_t full) {
      const int kbps = (int)ceil_div(num_kb, split);
      const int64_t split_tiles = split > 1 ? tiles - full : 0;
      // masked: the workspace must hold the live tiles of up to twice expected_m rows per group
      const int64_t ws_tiles = masked ? masked_capacity_tiles(G, rows, N, expected_m, v.bm, v.bn) : split_tiles;
      if (split > 1 && (ws_tiles > kMaxSplitTiles || split_ws_bytes(ws_tiles, split, v.bm, v.bn) > ws_avail))
        return;
      const UnitCost c = unit_cost(v.bm, v.bn);
      const double reduce =
          split > 1 ? kSplitUnitUs + kSplitReadUsPerKB * (split - 1) * (v.bm * v.bn * 4.0 / 1024.0) : 0.0;
      double t_units;
      if (split > 1 && full > 0) {  // whole tiles fill full / cus rounds, the split tiles one more
        t_units = (double)(full / cus) * (c.fixed_us + num_kb * c.kb_us) + (c.fixed_us + kbps * c.kb_us + reduce);
      } else {
        const int64_t units = split > 1 ? tiles * split : tiles;
        t_units = (double)ceil_div(units, cus) * (c.fixed_us + (split > 1 ? kbps : num_kb) * c.kb_us + reduce);
      }
      const double rows_live = masked ? (double)live * G : (double)rows;
      const double hbm_bytes = rows_live * K + (double)N * K * (kind == FP8GEMM_KIND_DENSE ? 1 : G) +
                               2.0 * rows_live * N +
                               8.0 * split * split_tiles * v.bm * v.bn;
      const double t =
          std::max(t_units, hbm_bytes / (kind == FP8GEMM_KIND_DENSE ? kDenseHbmBytesPerUs : kHbmBytesPerUs));
      // ties of the bound (calls that stream the same bytes) go to the faster units
      if (t < best * 0.999 || (t < best * 1.001 && t_units < best_units)) {
        best = t;
        best_units = t_units;
        pl.bm = v.bm;
        pl.bn = v.bn;
        pl.split = split;
        pl.full = split > 1 ? full : tiles;
      }
    };
    for (const auto& v : kVariants) {
      if (kind == FP8GEMM_KIND_CONTIGUOUS && 128 % v.bm != 0) continue;  // one expert per tile
      // the 96-column tiles measure faster only on few-row dense calls (grouped calls: never)
      if (kind != FP8GEMM_KIND_DENSE && v.bn % 128 != 0 && 128 % v.bn != 0) continue;
      if (v.bm >= 2 * 128 && live <= 128) continue;                      // mostly empty tiles
      // masked with several groups: their live rows differ, so the live M tiles per
      // group average more than expected_m / BM (by up to half a tile)
      const int64_t tiles =
          kind == FP8GEMM_KIND_MASKED && G > 1
              ? (int64_t)std::ceil((double)G * ceil_div(N, v.bn) * ((double)live / v.bm + kMaskedTileSlack))
              : ceil_div(live, v.bm) * ceil_div(N, v.bn) * (kind == FP8GEMM_KIND_MASKED ? G : 1);
      const int max_split = std::min(num_kb, kMaxSplit);
      const int64_t rem = tiles % cus;  // tiles of a last, partial round
      for (int sp = 1; sp <= max_split; ++sp) {
        if ((int)ceil_div(num_kb, ceil_div(num_kb, sp)) != sp) continue;  // same as a smaller split
        consider(v, tiles, sp, 0);
        // whole tiles for the full rounds, the last partial round split over the CUs
        if (!masked && sp > 1 && tiles > cus && rem > 0 && rem * sp <= cus) consider(v, tiles, sp, tiles - rem);
      }
    }
  }
  pl.kbps = (int)ceil_div(num_kb, pl.split);
  pl.split = (int)ceil_div(num_kb, pl.kbps);  // no empty splits
  pl.tiles_n = (int)ceil_div(N, pl.bn);
  pl.tiles_m = (int)ceil_div(rows, pl.bm);
  const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n * (kind == FP8GEMM_KIND_MASKED ? G : 1);
  // masked: every tile is split (no whole-tile rounds); the tile count is an upper bound
  pl.full = pl.split > 1 ? (kind == FP8GEMM_KIND_MASKED ? 0 : std::min<int64_t>(pl.full, tiles)) : tiles;
  pl.ws_tiles = kind == FP8GEMM_KIND_MASKED ? masked_capacity_tiles(G, rows, N, expected_m, pl.bm, pl.bn)
                                            : tiles - pl.full;
  pl.ws_bytes = split_ws_bytes(pl.ws_tiles, pl.split, pl.bm, pl.bn);
  if (pl.split > 1 && (pl.ws_bytes > ws_avail || pl.ws_tiles > kMaxSplitTiles) && !g_forced) {
    pl.split = 1;
    pl.kbps = num_kb;
    pl.full = tiles;
    pl.ws_bytes = 0;
  }
  pl.units = pl.full + (tiles - pl.full) * pl.split;
  const int64_t cap = (int64_t)cus * kOccupancy;
  int64_t grid = std::min<int64_t>(pl.units, cap);
  // A grid-stride loop keeps each workgroup on one XCD (workgroup b runs on XCD b % 8)
  // only if the grid is a multiple of 8. When every unit has a workgroup of its own (one
  // round), no rounding: rounding 231 units down to 224 workgroups would run 7 of them
  // in a second round. Masked calls learn their unit count on the device, so they
  // always round.
  if ((pl.units > cap || kind == FP8GEMM_KIND_MASKED) && grid > fp8gemm::kNumXcd)
    grid = grid / fp8gemm::kNumXcd * fp8gemm::kNumXcd;
  pl.grid = (int)std::max<int64_t>(grid, 1);
  return pl;
}

// The plan of a call depends only on its arguments below, so repeated calls of one shape
// (a serving loop) take it from a small per-thread cache instead of re-running the
// planner, which costs about a microsecond of host time per call.
Plan choose(int kind, int rows, int N, int K, int G, int expected_m, int cus, size_t ws_avail) {
  struct Entry {
    int kind, rows, N, K, G, expected_m, cus;
    uint32_t epoch;
    size_t ws_avail;
    bool valid;
    Plan plan;
  };
  constexpr int kEntries = 16;
  thread_local Entry cache[kEntries] = {};
  const uint32_t epoch = g_forced_epoch.load(std::memory_order_acquire);
  const uint64_t h = ((uint64_t)(uint32_t)rows * 0x9E3779B1u) ^ ((uint64_t)(uint32_t)N * 0x85EBCA77u) ^
                     ((uint64_t)(uint32_t)K * 0xC2B2AE3Du) ^ (uint64_t)(kind * 31 + G);
  Entry& e = cache[(h ^ (h >> 17)) % kEntries];
  if (e.valid && e.kind == kind && e.rows == rows && e.N == N && e.K == K && e.G == G &&
      e.expected_m == expected_m && e.cus == cus && e.epoch == epoch && e.ws_avail == ws_avail)
    return e.plan;
  const Plan pl = choose_uncached(kind, rows, N, K, G, expected_m, cus, ws_avail);
  e = Entry{kind, rows, N, K, G, expected_m, cus, epoch, ws_avail, true, pl};
  return pl;
}

template <int I, bool MASKED, bool E8 = false, bool HAS_C = false, bool STREAM_B = false>
hipError_t launch_variant(const Params& p, int grid, hipStream_t stream) {
  constexpr Variant v = kVariants[I];
  hipLaunchKernelGGL(
      (fp8gemm::fp8_gemm_kernel<v.bm, v.bn, v.waves_m, v.waves_n, v.stages, MASKED, E8, HAS_C, STREAM_B>),
      dim3(grid), dim3(v.waves_m * v.waves_n * 64), 0, stream, p);
  return hipGetLastError();
}

// Instances with non-temporal B loads exist for the 4-wave tiles (the few-row shapes)
// of the dense and contiguous forms.
template <int I>
constexpr bool kHasStreamB = kVariants[I].waves_m * kVariants[I].waves_n == 4;

// e8: power-of-two scales through the block-scaled MFMA; stream_b: B tiles read once
template <int I = 0>
hipError_t launch(const Plan& pl, const Params& p, hipStream_t stream, bool e8, bool stream_b) {
  if constexpr (I < kNumVariants) {
    if (kVariants[I].bm == pl.bm && kVariants[I].bn == pl.bn) {
      const bool masked = p.kind == FP8GEMM_KIND_MASKED;
      if constexpr (kHasStreamB<I>) {
        if (stream_b && !masked) {
          if (e8) return launch_variant<I, false, true, false, true>(p, pl.grid, stream);
          if (p.C) return launch_variant<I, false, false, true, true>(p, pl.grid, stream);
          return launch_variant<I, false, false, false, true>(p, pl.grid, stream);
        }
      }
      if (e8)
        return masked ? launch_variant<I, true, true>(p, pl.grid, stream)
                      : launch_variant<I, false, true>(p, pl.grid, stream);
      if (p.C)  // D = C + A B^T (FP32 scales)
        return masked ? launch_variant<I, true, false, true>(p, pl.grid, stream)
                      : launch_variant<I, false, false, true>(p, pl.grid, stream);
      return masked ? launch_variant<I, true>(p, pl.grid, stream) : launch_variant<I, false>(p, pl.grid, stream);
    }
    return launch<I + 1>(pl, p, stream, e8, stream_b);
  } else {
    return hipErrorInvalidValue;
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_common(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                 const float* sb, void* D, int64_t ldd, int rows, int N, int K) {
  if (!A || !sa || !B || !sb || !D) return FP8GEMM_ERR_NULL;
  if (rows < 0 || N <= 0 || K <= 0 || K % fp8gemm::kBlockK != 0) return FP8GEMM_ERR_SHAPE;
  if (lda < K || lda % 16 || ldb < K || ldb % 16) return FP8GEMM_ERR_LAYOUT;
  if (ldd < N) return FP8GEMM_ERR_LAYOUT;
  if (ld_sa < rows || ld_sa % 4) return FP8GEMM_ERR_LAYOUT;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 2) || !aligned(sa, 4) || !aligned(sb, 4))
    return FP8GEMM_ERR_LAYOUT;
  // the kernels address rows of one operand (one group) with 32-bit byte offsets
  if ((int64_t)std::max(rows - 1, 0) * lda + K > (int64_t)UINT32_MAX) return FP8GEMM_ERR_SHAPE;
  if ((int64_t)(N - 1) * ldb + K > (int64_t)UINT32_MAX) return FP8GEMM_ERR_SHAPE;
  return FP8GEMM_OK;
}

// optional addend C (BF16, D's shape): row stride and element alignment
int check_c(const void* C, int64_t ldc, int N) {
  if (!C) return FP8GEMM_OK;
  if (ldc < N || !aligned(C, 2)) return FP8GEMM_ERR_LAYOUT;
  return FP8GEMM_OK;
}

void maybe_print(const char* what, int rows, int N, int K, int G, const Plan& pl) {
  static const bool on = [] {
    const char* e = std::getenv("FP8GEMM_PRINT_CONFIGS");
    return e && *e && *e != '0';
  }();
  if (!on) return;
  std::fprintf(stderr, "[fp8gemm] %s M=%d N=%d K=%d G=%d -> tile %dx%d split %d grid %d units %lld\n", what,
               rows, N, K, G, pl.bm, pl.bn, pl.split, pl.grid, (long long)pl.units);
}

int run(int kind, const char* name, Params& p, int rows, int N, int K, int G, int expected_m, void* workspace,
        size_t workspace_bytes, hipStream_t stream, bool e8 = false) {
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  if (workspace && !aligned(workspace, 16)) return FP8GEMM_ERR_LAYOUT;
  const size_t ws_avail = workspace ? workspace_bytes : 0;
  Plan pl = choose(kind, rows, N, K, G, expected_m, cus, ws_avail);
  if (!has_kernel(pl.bm, pl.bn)) return FP8GEMM_ERR_CONFIG;
  if (pl.split > 1 && pl.ws_tiles > kMaxSplitTiles) return FP8GEMM_ERR_CONFIG;
  if (pl.split > 1 && pl.ws_bytes > ws_avail) return FP8GEMM_ERR_WORKSPACE;
  maybe_print(name, rows, N, K, G, pl);
  p.N = N;
  p.K = K;
  p.G = G;
  p.kind = kind;
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.split_k = pl.split;
  p.kb_per_split = pl.kbps;
  p.num_kb = K / fp8gemm::kBlockK;
  p.sb_kstride = p.sf_packed ? (p.num_kb + 3) / 4 : p.num_kb;
  p.num_units = (int)pl.units;
  p.full_tiles = (int)pl.full;
  // Raster width (M tiles walked at a time). Dense calls with at most 16 K blocks walk
  // one M-tile row at a time: their time goes largely into writing D, and the tiles that
  // run together then cover whole output rows (measured: 4096x32768x512 8% faster,
  // 4096x24576x1536 and 4096x7168x2048 3-5%). Longer K and the contiguous form keep 8,
  // the better width for their operand reuse in L2 (with one row: 4096x4096x7168 3%
  // slower, contiguous 8x4096 rows with K=2048 16% slower).
  p.group_m = kind == FP8GEMM_KIND_DENSE && p.num_kb <= 16 ? 1 : 8;
  p.vec_store = (p.ldd % 8 == 0 && aligned(p.D, 16)) ? 2 : (p.ldd % 4 == 0 && aligned(p.D, 8)) ? 1 : 0;
  p.c_vec = p.C && p.ldc % 8 == 0 && aligned(p.C, 16) ? 1 : 0;
  if (pl.split > 1) {
    p.counters = static_cast<int32_t*>(workspace);
    p.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    p.ws_tiles = (int)pl.ws_tiles;
  }
  if (pl.units == 0) return FP8GEMM_OK;
  // one tile row covers all of M (dense): each B tile is read by one unit only
  const bool stream_b = kind == FP8GEMM_KIND_DENSE && pl.tiles_m == 1;
  return launch(pl, p, stream, e8, stream_b) == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}

Params base_params(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                   const float* sb, void* D, int64_t ldd) {
  Params p{};
  p.A = static_cast<const uint8_t*>(A);
  p.sa = sa;
  p.B = static_cast<const uint8_t*>(B);
  p.sb = sb;
  p.D = static_cast<uint16_t*>(D);
  p.lda = lda;
  p.ld_sa = ld_sa;
  p.ldb = ldb;
  p.ldd = ldd;
  return p;
}

// Scale entries per 128-row weight block per group: K/128 FP32 values, or ceil(K/512)
// packed UE8M0 words.
int64_t scale_kstride(int K, bool packed) {
  const int nkb = K / fp8gemm::kBlockK;
  return packed ? (nkb + 3) / 4 : nkb;
}

int grouped_contiguous(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                       const float* sb, void* D, int64_t ldd, const int32_t* m_indices, int M_total, int N, int K,
                       int G, void* workspace, size_t workspace_bytes, hipStream_t stream, bool e8,
                       const void* C = nullptr, int64_t ldc = 0, bool packed = false) {
  int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M_total, N, K);
  if (st == FP8GEMM_OK) st = check_c(C, ldc, N);
  if (st != FP8GEMM_OK) return st;
  if (!m_indices) return FP8GEMM_ERR_NULL;
  if (G <= 0) return FP8GEMM_ERR_SHAPE;
  if (M_total == 0) return FP8GEMM_OK;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M_total;
  p.m_indices = m_indices;
  p.C = static_cast<const uint16_t*>(C);
  p.ldc = ldc;
  p.b_gstride = (int64_t)N * ldb;
  p.sf_packed = packed ? 1 : 0;
  p.sb_gstride = ceil_div(N, 128) * scale_kstride(K, packed);
  // tiles must not straddle two 128-row expert blocks
  if (g_forced && 128 % g_forced_cfg.block_m != 0) return FP8GEMM_ERR_CONFIG;
  return run(FP8GEMM_KIND_CONTIGUOUS, e8 ? (packed ? "contiguous ue8m0 packed" : "contiguous ue8m0") : "contiguous",
             p, M_total, N, K, G, 0, workspace,
             workspace_bytes, stream, e8);
}

int grouped_masked(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                   const float* sb, void* D, int64_t ldd, const int32_t* masked_m, int G, int M_max, int N, int K,
                   int expected_m, void* workspace, size_t workspace_bytes, hipStream_t stream, bool e8,
                   const void* C = nullptr, int64_t ldc = 0, bool packed = false) {
  int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M_max, N, K);
  if (st == FP8GEMM_OK) st = check_c(C, ldc, N);
  if (st != FP8GEMM_OK) return st;
  if (!masked_m) return FP8GEMM_ERR_NULL;
  if (G <= 0 || G > fp8gemm::kMaxGroups || M_max <= 0) return FP8GEMM_ERR_SHAPE;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M_max;
  p.masked_m = masked_m;
  p.a_gstride = (int64_t)M_max * lda;
  p.sf_packed = packed ? 1 : 0;
  p.sa_gstride = scale_kstride(K, packed) * ld_sa;
  p.b_gstride = (int64_t)N * ldb;
  p.sb_gstride = ceil_div(N, 128) * scale_kstride(K, packed);
  p.d_gstride = (int64_t)M_max * ldd;
  p.C = static_cast<const uint16_t*>(C);
  p.ldc = ldc;
  p.c_gstride = (int64_t)M_max * ldc;
  return run(FP8GEMM_KIND_MASKED, e8 ? (packed ? "masked ue8m0 packed" : "masked ue8m0") : "masked", p, M_max, N,
             K, G, expected_m, workspace, workspace_bytes, stream, e8);
}

}  // namespace

extern "C" {

int fp8_gemm_nt(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  const int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M;
  return run(FP8GEMM_KIND_DENSE, "dense", p, M, N, K, 1, 0, workspace, workspace_bytes, stream);
}

int fp8_gemm_nt_noalloc(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                        const float* sb, void* D, int64_t ldd, int M, int N, int K, hipStream_t stream) {
  const int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  int dst;
  effective_cus(true, &dst);
  if (dst != FP8GEMM_OK) return dst;
  void* ws = nullptr;
  const int sst = scratch_for_current_device(&ws, stream);
  if (sst != FP8GEMM_OK) return sst;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M;
  // the planner fits its split-K plan into the scratch; a forced plan that needs more
  // is rejected with FP8GEMM_ERR_WORKSPACE before any launch
  return run(FP8GEMM_KIND_DENSE, "dense noalloc", p, M, N, K, 1, 0, ws, kScratchBytes, stream);
}

size_t fp8_gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fp8_gemm_nt_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                  const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K);
  if (st == FP8GEMM_OK) st = check_c(C, ldc, N);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M;
  p.C = static_cast<const uint16_t*>(C);
  p.ldc = ldc;
  return run(FP8GEMM_KIND_DENSE, C ? "dense +C" : "dense", p, M, N, K, 1, 0, workspace, workspace_bytes, stream);
}

int fp8_gemm_nt_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                      const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const int st = check_common(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  Params p = base_params(A, lda, sa, ld_sa, B, ldb, sb, D, ldd);
  p.M = M;
  return run(FP8GEMM_KIND_DENSE, "dense ue8m0", p, M, N, K, 1, 0, workspace, workspace_bytes, stream, true);
}

int fp8_gemm_nt_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa, const void* B, int64_t ldb,
                             const int32_t* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  const float* saf = reinterpret_cast<const float*>(sa);
  const float* sbf = reinterpret_cast<const float*>(sb);
  const int st = check_common(A, lda, saf, ld_sa, B, ldb, sbf, D, ldd, M, N, K);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  Params p = base_params(A, lda, saf, ld_sa, B, ldb, sbf, D, ldd);
  p.M = M;
  p.sf_packed = 1;
  return run(FP8GEMM_KIND_DENSE, "dense ue8m0 packed", p, M, N, K, 1, 0, workspace, workspace_bytes, stream, true);
}

int fp8_grouped_gemm_nt_contiguous_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                                                const void* B, int64_t ldb, const int32_t* sb, void* D, int64_t ldd,
                                                const int32_t* m_indices, int M_total, int N, int K, int G,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return grouped_contiguous(A, lda, reinterpret_cast<const float*>(sa), ld_sa, B, ldb,
                            reinterpret_cast<const float*>(sb), D, ldd, m_indices, M_total, N, K, G, workspace,
                            workspace_bytes, stream, true, nullptr, 0, true);
}

int fp8_grouped_gemm_nt_masked_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                                            const void* B, int64_t ldb, const int32_t* sb, void* D, int64_t ldd,
                                            const int32_t* masked_m, int G, int M_max, int N, int K, int expected_m,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return grouped_masked(A, lda, reinterpret_cast<const float*>(sa), ld_sa, B, ldb, reinterpret_cast<const float*>(sb),
                        D, ldd, masked_m, G, M_max, N, K, expected_m, workspace, workspace_bytes, stream, true, nullptr,
                        0, true);
}

int fp8_grouped_gemm_nt_contiguous(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                   int64_t ldb, const float* sb, void* D, int64_t ldd, const int32_t* m_indices,
                                   int M_total, int N, int K, int G, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return grouped_contiguous(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, m_indices, M_total, N, K, G, workspace,
                            workspace_bytes, stream, false);
}

int fp8_grouped_gemm_nt_contiguous_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                         int64_t ldb, const float* sb, void* D, int64_t ldd,
                                         const int32_t* m_indices, int M_total, int N, int K, int G,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return grouped_contiguous(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, m_indices, M_total, N, K, G, workspace,
                            workspace_bytes, stream, true);
}

int fp8_grouped_gemm_nt_contiguous_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                     int64_t ldb, const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd,
                                     const int32_t* m_indices, int M_total, int N, int K, int G, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return grouped_contiguous(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, m_indices, M_total, N, K, G, workspace,
                            workspace_bytes, stream, false, C, ldc);
}

int fp8_grouped_gemm_nt_masked_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                 int64_t ldb, const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd,
                                 const int32_t* masked_m, int G, int M_max, int N, int K, int expected_m,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return grouped_masked(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, masked_m, G, M_max, N, K, expected_m, workspace,
                        workspace_bytes, stream, false,
                        C, ldc);
}

int fp8_grouped_gemm_nt_masked(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                               int64_t ldb, const float* sb, void* D, int64_t ldd, const int32_t* masked_m, int G,
                               int M_max, int N, int K, int expected_m, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return grouped_masked(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, masked_m, G, M_max, N, K, expected_m, workspace,
                        workspace_bytes, stream, false);
}

int fp8_grouped_gemm_nt_masked_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                     int64_t ldb, const float* sb, void* D, int64_t ldd, const int32_t* masked_m,
                                     int G, int M_max, int N, int K, int expected_m, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return grouped_masked(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, masked_m, G, M_max, N, K, expected_m, workspace,
                        workspace_bytes, stream, true);
}

int fp8_quantize_1x128(const void* X, int64_t ldx, int x_dtype, void* Q, int64_t ldq, float* sa, int64_t ld_sa, int M,
                       int K, hipStream_t stream) {
  if (!X || !Q || !sa) return FP8GEMM_ERR_NULL;
  if (M < 0 || K <= 0 || K % fp8gemm::kBlockK != 0) return FP8GEMM_ERR_SHAPE;
  if (x_dtype != FP8GEMM_QUANT_BF16 && x_dtype != FP8GEMM_QUANT_FP32) return FP8GEMM_ERR_LAYOUT;
  const int64_t x_align = x_dtype == FP8GEMM_QUANT_BF16 ? 8 : 4;  // elements per 16 bytes
  if (ldx < K || ldx % x_align != 0 || ldq < K || ldq % 8 != 0 || ld_sa < M || ld_sa % 4 != 0)
    return FP8GEMM_ERR_LAYOUT;
  if (!aligned(X, 16) || !aligned(Q, 8) || !aligned(sa, 4)) return FP8GEMM_ERR_LAYOUT;
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  const int nkb = K / fp8gemm::kBlockK;
  const int64_t items = ceil_div(M, 4) * nkb;  // one wave each
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 4), (int64_t)cus * 8));
  if (x_dtype == FP8GEMM_QUANT_BF16)
    hipLaunchKernelGGL(fp8gemm::quantize_1x128_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(X), ldx, static_cast<uint8_t*>(Q), ldq, sa, ld_sa, M, nkb);
  else
    hipLaunchKernelGGL(fp8gemm::quantize_1x128_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const float*>(X), ldx, static_cast<uint8_t*>(Q), ldq, sa, ld_sa, M, nkb);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}

}  // extern "C"

namespace {
int k_grouped_tn(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                 const float* sb, int64_t ld_sb, float* D, int64_t ldd, int64_t d_gstride, const int32_t* ks, int G,
                 int M, int N, int accumulate, hipStream_t stream, bool e8) {
  if (!A || !sa || !B || !sb || !D || !ks) return FP8GEMM_ERR_NULL;
  if (G <= 0 || G > fp8gemm::kMaxKGroups || M <= 0 || N <= 0) return FP8GEMM_ERR_SHAPE;
  fp8gemm::KParams p{};
  int64_t kb = 0;
  for (int g = 0; g < G; ++g) {
    if (ks[g] < 0 || ks[g] % fp8gemm::kBlockK != 0) return FP8GEMM_ERR_SHAPE;
    kb += ks[g] / fp8gemm::kBlockK;
    if (kb * fp8gemm::kBlockK > INT32_MAX) return FP8GEMM_ERR_SHAPE;
    p.kb_start[g + 1] = (int)kb;
  }
  // 16-byte row chunks; 128 rows of either operand addressed with 32-bit lane offsets
  if (lda < M || lda % 16 != 0 || ldb < N || ldb % 16 != 0 || lda > (1 << 24) || ldb > (1 << 24))
    return FP8GEMM_ERR_LAYOUT;
  if (ld_sa < M || ld_sb < N || ldd < N || (G > 1 && d_gstride < (int64_t)(M - 1) * ldd + N))
    return FP8GEMM_ERR_LAYOUT;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(D, 4))
    return FP8GEMM_ERR_LAYOUT;
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  p.A = static_cast<const uint8_t*>(A);
  p.sa = sa;
  p.B = static_cast<const uint8_t*>(B);
  p.sb = sb;
  p.D = D;
  p.lda = lda, p.ld_sa = ld_sa, p.ldb = ldb, p.ld_sb = ld_sb, p.ldd = ldd, p.d_gstride = d_gstride;
  p.M = M, p.N = N, p.G = G;
  p.accumulate = accumulate ? 1 : 0;
  p.vec4 = (ldd % 4 == 0 && (G == 1 || d_gstride % 4 == 0) && aligned(D, 16)) ? 1 : 0;
  // 256x256 tiles (8 waves of 64x128) once they alone give every CU a tile; else 128x128
  // (4 waves of 64x64, two workgroups per CU). Both use a 2-stage ring: a 3-stage 256x128
  // instance (64x64 per wave) measured slower than the 256x256 one on the weight-gradient
  // shapes, whose per-flop LDS reads are 25% lower.
  const bool big = (int64_t)G * ceil_div(M, 256) * ceil_div(N, 256) >= cus;
  const int bm = big ? 256 : 128, bn = big ? 256 : 128;
  p.tiles_m = (int)ceil_div(M, bm);
  p.tiles_n = (int)ceil_div(N, bn);
  // chunks of one XCD's CUs worth of tiles, dealt to the XCDs in turn (the kernel's tile
  // mapping); the grid covers whole rounds of chunks
  p.chunk = std::max(1, std::min(cus / fp8gemm::kNumXcd, 64));
  const int64_t chunks = (int64_t)G * ceil_div((int64_t)p.tiles_m * p.tiles_n, p.chunk);
  const int64_t tiles = ceil_div(chunks, fp8gemm::kNumXcd) * fp8gemm::kNumXcd * p.chunk;
  if (tiles > INT32_MAX) return FP8GEMM_ERR_SHAPE;
  if (big && e8)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<4, 2, 8, 2, true>), dim3((unsigned)tiles), dim3(512), 0,
                       stream, p);
  else if (big)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<4, 2, 8, 2>), dim3((unsigned)tiles), dim3(512), 0, stream, p);
  else if (e8)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<2, 2, 4, 2, true>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<2, 2, 4, 2>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}
}  // namespace

extern "C" {

int fp8_k_grouped_gemm_tn_contiguous(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B,
                                     int64_t ldb, const float* sb, int64_t ld_sb, float* D, int64_t ldd,
                                     int64_t d_gstride, const int32_t* ks, int G, int M, int N, int accumulate,
                                     hipStream_t stream) {
  return k_grouped_tn(A, lda, sa, ld_sa, B, ldb, sb, ld_sb, D, ldd, d_gstride, ks, G, M, N, accumulate, stream,
                      false);
}

int fp8_k_grouped_gemm_tn_contiguous_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                           const void* B, int64_t ldb, const float* sb, int64_t ld_sb, float* D,
                                           int64_t ldd, int64_t d_gstride, const int32_t* ks, int G, int M, int N,
                                           int accumulate, hipStream_t stream) {
  return k_grouped_tn(A, lda, sa, ld_sa, B, ldb, sb, ld_sb, D, ldd, d_gstride, ks, G, M, N, accumulate, stream,
                      true);
}

}  // extern "C"

namespace {
// Tile plans of the dense layout calls (TN, NN, TT). Instances: 256x256 tiles (8 waves of
// 64x128, a 2-stage ring); 128x128 tiles (4 waves of 64x64) with a 2-stage ring, of
// which two workgroups share a CU, or a 4-stage ring (one workgroup per CU, more bytes
// in flight per unit) for plans whose units all run in one round; 64x128 and 128x64
// tiles (4 waves of 64x32; one operand in a 64-wide panel) with a 6-stage ring.
struct LayoutPlan {
  int bm = 128, bn = 128, split = 1, kbps = 0, stages = 2;
  int64_t tiles = 0, units = 0;
  size_t ws_bytes = 0;
};

bool is_layout_tile(int bm, int bn) {
  return (bm == 128 && bn == 128) || (bm == 256 && bn == 256) || (bm == 64 && bn == 128) || (bm == 128 && bn == 64);
}

// 256x256 tiles once they give at least half the CUs a tile and pad the output by at most
// a quarter: a CU computes a 256x256 tile ~20% faster than two co-resident 128x128 ones
// (measured: 4096x2112x7168, 144 such tiles, 99 vs 120 us), but a few-row shape would
// compute its padding. Otherwise the tile (128x128, 64x128 or 128x64) and the K split
// with the least modelled time. These calls are bound by what each CU streams: a unit
// costs kLayoutUsPerLoadByte per byte of its K blocks' loads (the whole tile, rows past
// M included) plus kLayoutUnitUs, per round of units, and the last arrival
// kLayoutUsPerPartialByte per byte of each further partial it reads (live rows only).
// Constants fitted to bench.py --plan-sweep layout (every tile and split of the 12 few-row
// shapes; the choice is within 5% of the fastest measured plan on each). K is split only
// as far as all units run in one round, each keeps at least kLayoutMinKbps K blocks (with
// fewer, its fixed cost is not amortised) and the workspace holds the partials.
constexpr int kLayoutMaxSplit = 16;
constexpr int kLayoutMinKbps = 5;
constexpr double kLayoutUsPerLoadByte = 2.57e-5;
constexpr double kLayoutUsPerPartialByte = 2.72e-5;
constexpr double kLayoutUnitUs = 8.66;
LayoutPlan choose_layout(int M, int N, int K, int cus, size_t ws_avail) {
  LayoutPlan pl;
  const int num_kb = K / fp8gemm::kBlockK;
  if (g_forced) {
    pl.bm = g_forced_cfg.block_m;
    pl.bn = g_forced_cfg.block_n;
    pl.split = std::max(1, std::min(g_forced_cfg.split_k, num_kb));
  } else if (2 * ceil_div(M, 256) * ceil_div(N, 256) >= cus &&
             (double)(ceil_div(M, 256) * 256) * (double)(ceil_div(N, 256) * 256) <= 1.25 * (double)M * N) {
    pl.bm = pl.bn = 256;
  } else {
    static const int kTiles[3][2] = {{128, 128}, {64, 128}, {128, 64}};
    double best = 1e30;
    for (const auto& tl : kTiles) {
      const int bm = tl[0], bn = tl[1];
      const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
      for (int sp = 1; sp <= std::min(num_kb, kLayoutMaxSplit); ++sp) {
        const int kbps = (int)ceil_div(num_kb, sp);
        if (ceil_div(num_kb, kbps) != sp) continue;  // the same as a smaller split
        if (sp > 1 && (kbps < kLayoutMinKbps || tiles * sp > cus || tiles > kMaxSplitTiles ||
                       split_ws_bytes(tiles, sp, bm, bn) > ws_avail))
          continue;
        const int64_t units = tiles * sp;
        // two 2-stage 128x128 workgroups share a CU; the 6-stage narrow tiles take one
        const int per_cu = (bm == 128 && bn == 128 && units > cus) ? 2 : 1;
        const double rounds = (double)ceil_div(units, (int64_t)cus * per_cu);
        const double t = rounds * ((double)kbps * (bm + bn) * fp8gemm::kBlockK * kLayoutUsPerLoadByte + kLayoutUnitUs) +
                         (sp - 1) * (double)std::min(bm, M) * bn * 4 * kLayoutUsPerPartialByte;
        if (t < best) {
          best = t;
          pl.bm = bm, pl.bn = bn, pl.split = sp;
        }
      }
    }
  }
  pl.kbps = (int)ceil_div(num_kb, pl.split);
  pl.split = (int)ceil_div(num_kb, pl.kbps);  // no empty splits
  pl.tiles = ceil_div(M, pl.bm) * ceil_div(N, pl.bn);
  pl.units = pl.tiles * pl.split;
  pl.ws_bytes = split_ws_bytes(pl.tiles, pl.split, pl.bm, pl.bn);
  pl.stages = pl.bm == 256 ? 2 : pl.bm == 64 || pl.bn == 64 ? 6 : pl.units <= cus ? 4 : 2;
  return pl;
}

template <bool E8, bool A_KC, bool B_KC>
void launch_dense_layout(const fp8gemm::KParams& p, const LayoutPlan& pl, hipStream_t stream) {
  const dim3 grid((unsigned)pl.units);
  if (pl.bm == 256)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<4, 2, 8, 2, E8, true, A_KC, B_KC>), grid, dim3(512), 0,
                       stream, p);
  else if (pl.bm == 64)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<1, 4, 2, 6, E8, true, A_KC, B_KC>), grid, dim3(256), 0,
                       stream, p);
  else if (pl.bn == 64)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<2, 2, 2, 6, E8, true, A_KC, B_KC>), grid, dim3(256), 0,
                       stream, p);
  else if (pl.stages == 4)
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<2, 2, 4, 4, E8, true, A_KC, B_KC>), grid, dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fp8gemm::fp8_k_grouped_tn_kernel<2, 2, 4, 2, E8, true, A_KC, B_KC>), grid, dim3(256), 0,
                       stream, p);
}
template <bool E8>
void launch_dense_layout(const fp8gemm::KParams& p, const LayoutPlan& pl, hipStream_t stream, bool a_kc,
                         bool b_kc) {
  if (a_kc)
    launch_dense_layout<E8, true, false>(p, pl, stream);
  else if (b_kc)
    launch_dense_layout<E8, false, true>(p, pl, stream);
  else
    launch_dense_layout<E8, false, false>(p, pl, stream);
}

// The dense call in the TN (a_kc = b_kc = false), NN (a_kc) and TT (b_kc) layouts: a
// K-contiguous operand is [rows][ld >= K], a K-major one [K][ld >= rows]. e8: UE8M0
// (power-of-two) scales applied by the block-scaled MFMA.
int dense_layout(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                 const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                 size_t workspace_bytes, hipStream_t stream, bool a_kc, bool b_kc, bool e8 = false,
                 const void* C = nullptr, int64_t ldc = 0) {
  if (!A || !sa || !B || !sb || !D) return FP8GEMM_ERR_NULL;
  if (M < 0 || N <= 0 || K <= 0 || K % fp8gemm::kBlockK != 0) return FP8GEMM_ERR_SHAPE;
  // 16-byte row chunks; 128 rows of either operand addressed with 32-bit lane offsets
  if (lda < (a_kc ? K : M) || lda % 16 != 0 || ldb < (b_kc ? K : N) || ldb % 16 != 0 || lda > (1 << 24) ||
      ldb > (1 << 24))
    return FP8GEMM_ERR_LAYOUT;
  if (ld_sa < M || ld_sa % 4 != 0 || ldd < N) return FP8GEMM_ERR_LAYOUT;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(D, 2))
    return FP8GEMM_ERR_LAYOUT;
  if (C && (ldc < N || !aligned(C, 2))) return FP8GEMM_ERR_LAYOUT;
  if (workspace && !aligned(workspace, 16)) return FP8GEMM_ERR_LAYOUT;
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  if (g_forced && !is_layout_tile(g_forced_cfg.block_m, g_forced_cfg.block_n)) return FP8GEMM_ERR_CONFIG;
  if (M == 0) return FP8GEMM_OK;
  const size_t ws_avail = workspace ? workspace_bytes : 0;
  const LayoutPlan pl = choose_layout(M, N, K, cus, ws_avail);
  // the 256x256 tiles do not split K
  if (pl.split > 1 && (pl.tiles > kMaxSplitTiles || pl.bm == 256)) return FP8GEMM_ERR_CONFIG;
  if (pl.split > 1 && pl.ws_bytes > ws_avail) return FP8GEMM_ERR_WORKSPACE;
  if (pl.units > INT32_MAX) return FP8GEMM_ERR_SHAPE;
  fp8gemm::KParams p{};
  p.C = static_cast<const uint16_t*>(C);
  p.ldc = ldc;
  p.c_vec = (C && ldc % 4 == 0 && aligned(C, 8)) ? 1 : 0;
  p.A = static_cast<const uint8_t*>(A);
  p.sa = sa;
  p.B = static_cast<const uint8_t*>(B);
  p.sb = sb;
  p.Dh = static_cast<uint16_t*>(D);
  p.lda = lda, p.ld_sa = ld_sa, p.ldb = ldb, p.ld_sb = K / fp8gemm::kBlockK, p.ldd = ldd;
  p.M = M, p.N = N, p.G = 1;
  p.kb_start[0] = 0;
  p.kb_start[1] = K / fp8gemm::kBlockK;
  p.vec4 = (ldd % 4 == 0 && aligned(D, 8)) ? 1 : 0;
  p.tiles_m = (int)ceil_div(M, pl.bm);
  p.tiles_n = (int)ceil_div(N, pl.bn);
  p.stream_b = p.tiles_m == 1 ? 1 : 0;
  p.split_k = pl.split;
  p.kb_per_split = pl.kbps;
  if (pl.split > 1) {
    p.counters = static_cast<int32_t*>(workspace);
    p.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
  }
  if (e8)
    launch_dense_layout<true>(p, pl, stream, a_kc, b_kc);
  else
    launch_dense_layout<false>(p, pl, stream, a_kc, b_kc);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}
}  // namespace

extern "C" {

int fp8_gemm_tn(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      false);
}

int fp8_gemm_nn(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, true,
                      false);
}

int fp8_gemm_tt(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      true);
}

int fp8_gemm_tn_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                  const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!C) return FP8GEMM_ERR_NULL;
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      false, false, C, ldc);
}

int fp8_gemm_nn_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                  const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!C) return FP8GEMM_ERR_NULL;
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, true,
                      false, false, C, ldc);
}

int fp8_gemm_tt_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                  const float* sb, const void* C, int64_t ldc, void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!C) return FP8GEMM_ERR_NULL;
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      true, false, C, ldc);
}

int fp8_gemm_tn_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                      const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      false, true);
}

int fp8_gemm_nn_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                      const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, true,
                      false, true);
}

int fp8_gemm_tt_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa, const void* B, int64_t ldb,
                      const float* sb, void* D, int64_t ldd, int M, int N, int K, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return dense_layout(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace, workspace_bytes, stream, false,
                      true, true);
}

int fp8_swiglu_quantize_1x128(const void* H, int64_t ldh, int h_dtype, const int32_t* m_indices, void* Q,
                              int64_t ldq, float* sa, int64_t ld_sa, int M, int F, hipStream_t stream) {
  if (!H || !Q || !sa) return FP8GEMM_ERR_NULL;
  if (M < 0 || F <= 0 || F % fp8gemm::kBlockK != 0) return FP8GEMM_ERR_SHAPE;
  if (h_dtype != FP8GEMM_QUANT_BF16 && h_dtype != FP8GEMM_QUANT_FP32) return FP8GEMM_ERR_LAYOUT;
  const int64_t h_align = h_dtype == FP8GEMM_QUANT_BF16 ? 8 : 4;  // elements per 16 bytes
  if (ldh < 2 * (int64_t)F || ldh % h_align != 0 || ldq < F || ldq % 8 != 0 || ld_sa < M || ld_sa % 4 != 0)
    return FP8GEMM_ERR_LAYOUT;
  if (!aligned(H, 16) || !aligned(Q, 8) || !aligned(sa, 4) || !aligned(m_indices, 4)) return FP8GEMM_ERR_LAYOUT;
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  if (M == 0) return FP8GEMM_OK;
  const int nkb = F / fp8gemm::kBlockK;
  const int64_t items = ceil_div(M, 4) * nkb;  // one wave each
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 4), (int64_t)cus * 8));
  if (h_dtype == FP8GEMM_QUANT_BF16)
    hipLaunchKernelGGL((fp8gemm::quantize_1x128_kernel<uint16_t, true>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(H), ldh, static_cast<uint8_t*>(Q), ldq, sa, ld_sa, M, nkb,
                       m_indices, F);
  else
    hipLaunchKernelGGL((fp8gemm::quantize_1x128_kernel<float, true>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const float*>(H), ldh, static_cast<uint8_t*>(Q), ldq, sa, ld_sa, M, nkb,
                       m_indices, F);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}

int fp8_transform_sf_into_required_layout(const float* sf, int64_t ld_sf, int rows, int nkb, int is_activation,
                                          int pack, void* out, int64_t ld_out, hipStream_t stream) {
  if (!sf || !out) return FP8GEMM_ERR_NULL;
  if (rows < 0 || nkb <= 0) return FP8GEMM_ERR_SHAPE;
  const int64_t cols = pack ? (nkb + 3) / 4 : nkb;
  if (ld_sf < nkb || !aligned(sf, 4) || !aligned(out, 4)) return FP8GEMM_ERR_LAYOUT;
  if (is_activation ? (ld_out < rows || ld_out % 4 != 0) : ld_out < cols) return FP8GEMM_ERR_LAYOUT;
  if ((int64_t)rows * cols > INT32_MAX) return FP8GEMM_ERR_SHAPE;
  int st;
  const int cus = effective_cus(true, &st);
  if (st != FP8GEMM_OK) return st;
  if (rows == 0) return FP8GEMM_OK;
  const int64_t n = (int64_t)rows * cols;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, 256), (int64_t)cus * 8));
  hipLaunchKernelGGL(fp8gemm::transform_sf_kernel, dim3(grid), dim3(256), 0, stream, sf, ld_sf, rows, nkb,
                     is_activation ? 1 : 0, pack ? 1 : 0, static_cast<uint32_t*>(out), ld_out);
  return hipGetLastError() == hipSuccess ? FP8GEMM_OK : FP8GEMM_ERR_LAUNCH;
}

size_t fp8_gemm_workspace_size(int kind, int M, int N, int K, int G, int expected_m) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return 0;
  int st;
  const int cus = effective_cus(false, &st);
  if (kind == FP8GEMM_KIND_LAYOUT) {
    const LayoutPlan pl = choose_layout(M, N, K, cus, SIZE_MAX);
    return pl.split > 1 ? pl.ws_bytes : 0;
  }
  const Plan pl = choose(kind, M, N, K, std::max(G, 1), expected_m, cus, SIZE_MAX);
  return pl.split > 1 ? pl.ws_bytes : 0;
}

int fp8_gemm_query_config(int kind, int M, int N, int K, int G, int expected_m, size_t workspace_bytes,
                          fp8gemm_config_t* out) {
  if (!out) return FP8GEMM_ERR_NULL;
  if (M < 0 || N <= 0 || K <= 0 || K % 128 || G <= 0) return FP8GEMM_ERR_SHAPE;
  int st;
  const int cus = effective_cus(false, &st);
  if (kind == FP8GEMM_KIND_LAYOUT) {
    const LayoutPlan pl = choose_layout(M, N, K, cus, workspace_bytes);
    out->block_m = pl.bm;
    out->block_n = pl.bn;
    out->split_k = pl.split;
    out->grid = (int)pl.units;
    out->num_units = (int)pl.units;
    out->full_tiles = pl.split > 1 ? 0 : (int)pl.tiles;
    return FP8GEMM_OK;
  }
  const Plan pl = choose(kind, M, N, K, G, expected_m, cus, workspace_bytes);
  out->block_m = pl.bm;
  out->block_n = pl.bn;
  out->split_k = pl.split;
  out->grid = pl.grid;
  out->num_units = (int)pl.units;
  out->full_tiles = (int)pl.full;
  return FP8GEMM_OK;
}

int fp8_gemm_force_config(const fp8gemm_config_t* cfg) {
  if (!cfg) {
    g_forced = false;
    g_forced_epoch.fetch_add(1, std::memory_order_acq_rel);  // cached plans are stale
    return FP8GEMM_OK;
  }
  if (!(has_kernel(cfg->block_m, cfg->block_n) || is_layout_tile(cfg->block_m, cfg->block_n)) || cfg->split_k < 1)
    return FP8GEMM_ERR_CONFIG;
  g_forced_cfg = *cfg;
  g_forced = true;
  g_forced_epoch.fetch_add(1, std::memory_order_acq_rel);
  return FP8GEMM_OK;
}

int fp8_gemm_set_num_cus(int n) {
  g_num_cus_override.store(n > 0 ? n : 0);
  return FP8GEMM_OK;
}

int fp8_gemm_get_num_cus(void) {
  const int ov = g_num_cus_override.load();
  if (ov > 0) return ov;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  return g_devices[dev].status == FP8GEMM_OK ? g_devices[dev].cus : 0;
}

int fp8_gemm_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int64_t fp8_gemm_scale_ld(int64_t rows) { return rows <= 0 ? 0 : (rows + 3) / 4 * 4; }

int64_t fp8_gemm_num_tiles(int64_t M, int64_t N, int block_m, int block_n) {
  if (M <= 0 || N <= 0 || block_m <= 0 || block_n <= 0) return 0;
  return ceil_div(M, block_m) * ceil_div(N, block_n);
}

const char* fp8_gemm_status_string(int status) {
  switch (status) {
    case FP8GEMM_OK: return "ok";
    case FP8GEMM_ERR_NULL: return "null pointer argument";
    case FP8GEMM_ERR_SHAPE: return "invalid shape (sizes must be positive, K a multiple of 128)";
    case FP8GEMM_ERR_LAYOUT: return "invalid stride, leading dimension or alignment";
    case FP8GEMM_ERR_WORKSPACE: return "workspace too small for the forced split-K configuration";
    case FP8GEMM_ERR_DEVICE: return "current device is not gfx950 or cannot be queried";
    case FP8GEMM_ERR_LAUNCH: return "kernel launch failed";
    case FP8GEMM_ERR_CONFIG: return "invalid forced tile configuration";
    default: return "unknown status";
  }
}

}  // extern "C"
