/*
 * fp8gemm.h -- C ABI of libfp8gemm.so: FP8 (e4m3) NT GEMM with fine-grained FP32
 * block scaling and BF16 output, dense and M-grouped (MoE), for AMD MI355X (gfx950).
 *
 * Operation (all three entry points):
 *
 *     D[m, n] = bf16( sum_kb  P_kb[m, n] * sa[kb][m] * sb[n / 128][kb] )
 *     P_kb[m, n] = sum_{k = 128 kb}^{128 kb + 127}  A[m, k] * B[n, k]
 *
 * i.e. D = A . B^T ("NT": A row-major [M, K], B row-major [N, K] = B^T column-major),
 * with each 128-wide K block's partial product promoted into an FP32 accumulator
 * after multiplying it by the activation scale sa (one per row per 128 K) and the
 * weight scale sb (one per 128x128 block). Sources: DeepGEMM pages --
 * es.news.hada.io/topic?id=19444 (intro: FP8 GEMM with DeepSeek-V3 fine-grained
 * scaling; two-level "promotion" accumulation), bquan.live post 9429818
 * ("¿Cómo usarlo?": NT format, BF16 output, dense / contiguous / masked entry
 * points), es.news.hada.io/topic?id=19459 ("Interfaz GEMM y restricciones de
 * layout": NT only, LHS scales transposed and FP32; "Dense y Grouped GEMM":
 * M-grouped contiguous and masked layouts), deepep.org/zh/deepgemm (接口设计).
 * The pages name the scaling scheme but not its block sizes; 1x128 (A) and
 * 128x128 (B) are the DeepSeek-V3 granularity they refer to.
 *
 * Beside the three NT calls (each also in a UE8M0-scale form *_ue8m0 and an
 * accumulate form *_c, D = C + A B^T), the library has the dense call in the TN, NN
 * and TT layouts (fp8_gemm_tn / _nn / _tt, also _ue8m0 and _c), the K-grouped TN GEMM of the MoE weight
 * gradient with FP32 output (fp8_k_grouped_gemm_tn_contiguous, also _ue8m0), and the
 * 1x128 activation quantiser (fp8_quantize_1x128, fp8_swiglu_quantize_1x128); each
 * declaration below states its own operation and layouts where they differ from the
 * conventions here (the leading-dimension rule, for one, follows each operand's
 * layout).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *    allocates, frees or synchronises, and never reads device memory from the host.
 *  - Work is enqueued on `stream` (NULL = the default stream); buffers must stay
 *    valid until that work completes. Calls are asynchronous.
 *  - e4m3 = OCP E4M3FN bytes (max 448; 0x7F/0xFF are NaN). bf16 = uint16 bits.
 *  - Strides are in ELEMENTS of the pointed-to type. K % 128 == 0.
 *    lda, ldb >= K and multiples of 16; ldd >= N; ld_sa >= the number of rows it
 *    covers and a multiple of 4; A, B 16-byte aligned, D 2-byte aligned (the
 *    fastest, 16-byte stores need D 16-byte aligned and ldd % 8 == 0; 8-byte
 *    stores D 8-byte aligned and ldd % 4 == 0), sa / sb 4-byte aligned.
 *  - Rounding: FP32 accumulation, one round-to-nearest-even to BF16 per output.
 *  - Return value: FP8GEMM_OK (0) or a negative FP8GEMM_ERR_* code. On an
 *    argument error nothing is launched. No exception crosses the ABI.
 *  - Preconditions on device data (cannot be checked from the host): no e4m3 NaN
 *    codes in live rows; m_indices / masked_m as documented per call.
 *  - Split-K workspace: optional, 16-byte aligned. When `workspace` is NULL or smaller
 *    than fp8_gemm_workspace_size(...), the call runs without split-K (or with fewer
 *    split tiles). Layout: the first 16 KiB hold 4096 int32 arrival counters, the
 *    rest FP32 partial sums. The counters must be zero before the workspace's first
 *    use (zero-fill the buffer once); every call that completes leaves them zero
 *    again. The partials need no initial value. So one workspace may serve any
 *    sequence of calls of any shapes, one after another on a stream. Calls that may
 *    run concurrently (other streams) must not share a workspace.
 */
#ifndef FP8GEMM_H_
#define FP8GEMM_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP8GEMM_OK = 0,
  FP8GEMM_ERR_NULL = -1,      /* a required pointer is NULL                          */
  FP8GEMM_ERR_SHAPE = -2,     /* M, N, K, G <= 0 (M may be 0 where noted), K % 128   */
  FP8GEMM_ERR_LAYOUT = -3,    /* stride / leading dimension / alignment violated     */
  FP8GEMM_ERR_WORKSPACE = -4, /* forced split-K config needs more workspace          */
  FP8GEMM_ERR_DEVICE = -5,    /* current device is not gfx950 / cannot be queried    */
  FP8GEMM_ERR_LAUNCH = -6,    /* the HIP launch reported an error                    */
  FP8GEMM_ERR_CONFIG = -7     /* an invalid forced tile configuration                */
};

/* Call kinds of the planner queries (fp8_gemm_workspace_size, fp8_gemm_query_config):
 * the dense NT call, the two M-grouped calls, and the dense TN / NN / TT calls, which
 * share one plan. */
enum { FP8GEMM_KIND_DENSE = 0, FP8GEMM_KIND_CONTIGUOUS = 1, FP8GEMM_KIND_MASKED = 2, FP8GEMM_KIND_LAYOUT = 3 };

/* Tile configuration chosen for (or forced on) a call. */
typedef struct {
  int block_m;    /* output rows per work unit                                   */
  int block_n;    /* output columns per work unit                                */
  int split_k;    /* K splits per output tile (1 = none; > 1 uses the workspace) */
  int grid;       /* workgroups launched (persistent loop over work units)       */
  int num_units;  /* work units; an upper bound for masked                       */
  int full_tiles; /* tiles computed whole, the first in the order of work; each  */
                  /* other tile is split_k units. A last, partial round of tiles */
                  /* is split this way so that it occupies every CU.            */
} fp8gemm_config_t;

/*
 * Dense D[M, N] = A[M, K] . B[N, K]^T: the normal (non-grouped) GEMM of the pages
 * (bquan.live post 9429818, "¿Cómo usarlo?"; es.news.hada.io/topic?id=19459,
 * "Interfaz GEMM y restricciones de layout": fp8_gemm_nt, the NT layout, FP32 LHS
 * scales in a transposed layout).
 *   A  e4m3 [M, K] row-major, row stride lda.
 *   sa fp32 [K/128][ld_sa]: sa[kb * ld_sa + m] scales row m of K block kb
 *      (the transposed, M-contiguous layout), ld_sa >= M.
 *   B  e4m3 [N, K] row-major, row stride ldb.
 *   sb fp32 [ceil(N/128)][K/128]: sb[(n/128) * (K/128) + kb]; a last partial block
 *      of columns (N % 128 != 0) has its own scale row.
 *   D  bf16 [M, N] row-major, row stride ldd; fully overwritten. M == 0 is a no-op.
 */
int fp8_gemm_nt(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                const void* B, int64_t ldb, const float* sb,
                void* D, int64_t ldd, int M, int N, int K,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_gemm_nt for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same operation,
 * layouts and errors as fp8_gemm_nt, without the workspace arguments: the split-K
 * partials and arrival counters live in a scratch array inside the library, one copy
 * per device, of fp8_gemm_noalloc_scratch_bytes() bytes (32 MiB + 16 KiB), held from the
 * first call on a device until the process ends. The call allocates nothing (no
 * hipMalloc, no allocating library routine); the first call on a device looks the
 * array up and clears its counter block with a small kernel on `stream`; every call
 * that completes leaves the counters zero again. The planner fits its split-K plan into
 * the scratch; a forced configuration (fp8_gemm_force_config) whose plan needs more
 * returns FP8GEMM_ERR_WORKSPACE before any launch. All calls on one GPU share its
 * scratch: calls that may overlap in time (other streams, other host threads) race and
 * must not be issued; calls in order on one stream are safe.
 */
int fp8_gemm_nt_noalloc(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                        const void* B, int64_t ldb, const float* sb,
                        void* D, int64_t ldd, int M, int N, int K, hipStream_t stream);
/* Size in bytes of the per-device scratch of fp8_gemm_nt_noalloc (the same for every
 * device; a constant of the library), for the callers that cannot allocate. */
size_t fp8_gemm_noalloc_scratch_bytes(void);

/*
 * D = C + A B^T (the pages' naming convention for every GEMM: fp8_gemm_nt computes
 * D = C + A @ B.T; es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de
 * layout"). The three calls below are fp8_gemm_nt, fp8_grouped_gemm_nt_contiguous and
 * fp8_grouped_gemm_nt_masked with an optional addend:
 *   C  bf16 with D's shape and layout conventions (row stride ldc >= N, 2-byte aligned;
 *      masked: [G, M_max, N] with group stride M_max * ldc), read only where D is
 *      written; D = bf16_rne(C + the FP32 accumulation). C == NULL is the plain call.
 *      C may be D itself (in-place accumulation: each element is read before it is
 *      written, by the same lane); other overlaps of C and D are undefined.
 * Errors as for the plain calls, plus FP8GEMM_ERR_LAYOUT for ldc < N or a misaligned C.
 */
int fp8_gemm_nt_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                  const void* B, int64_t ldb, const float* sb,
                  const void* C, int64_t ldc, void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_grouped_gemm_nt_contiguous_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                     const void* B, int64_t ldb, const float* sb,
                                     const void* C, int64_t ldc, void* D, int64_t ldd,
                                     const int32_t* m_indices, int M_total, int N, int K, int G,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_grouped_gemm_nt_masked_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                 const void* B, int64_t ldb, const float* sb,
                                 const void* C, int64_t ldc, void* D, int64_t ldd,
                                 const int32_t* masked_m, int G, int M_max, int N, int K, int expected_m,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense NT GEMM with UE8M0 scale factors: the same operation, layouts, workspace and
 * errors as fp8_gemm_nt, for scales that are powers of two (the UE8M0 scale format
 * the pages list among DeepGEMM's scale-factor options: es.news.hada.io/topic?id=19459,
 * "Interfaz GEMM y restricciones de layout"). sa and sb hold each scale as the FP32
 * value 2^(e-127) of its E8M0 code e (1 <= e <= 254); only the exponent field is read.
 * The kernel passes the codes to gfx950's block-scaled MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4), which scales each 128-K block product and
 * accumulates it in FP32 itself, so no promotion FMAs run.
 * Precondition (device data, not checked): every scale is an exact normal power of
 * two; a mantissa would be ignored.
 */
int fp8_gemm_nt_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const void* B, int64_t ldb, const float* sb,
                      void* D, int64_t ldd, int M, int N, int K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The three NT calls with packed UE8M0 scale factors: the pages' newer API takes UE8M0
 * scales packed four to a 32-bit int (es.news.hada.io/topic?id=19459, "Interfaz GEMM y
 * restricciones de layout"). Same operations, shapes, preconditions and errors as
 * fp8_gemm_nt_ue8m0 and the grouped *_ue8m0 calls; only the scale layouts differ (the
 * pages give no axis or byte order; the reading implemented):
 *   sa int32 [ceil(K/512)][ld_sa] (masked: [G][ceil(K/512)][ld_sa]): word w of row m
 *      holds the E8M0 codes of row m's K blocks 4w, 4w+1, 4w+2, 4w+3 in bytes 0..3
 *      (bits 8j..8j+7); ld_sa >= rows, ld_sa % 4 == 0, 4-byte aligned.
 *   sb int32 [ceil(N/128)][ceil(K/512)] (grouped: [G][ceil(N/128)][ceil(K/512)]), the
 *      same packing of each 128x128 block row's codes.
 * Each scale is 2^(code - 127); codes 1..254 (0 and 255 are outside the contract).
 * Bytes of the last word past K/128 are not read. fp8_transform_sf_into_required_layout
 * produces both layouts from FP32 scales.
 */
int fp8_gemm_nt_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                             const void* B, int64_t ldb, const int32_t* sb,
                             void* D, int64_t ldd, int M, int N, int K,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_grouped_gemm_nt_contiguous_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                                                const void* B, int64_t ldb, const int32_t* sb,
                                                void* D, int64_t ldd, const int32_t* m_indices,
                                                int M_total, int N, int K, int G,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_grouped_gemm_nt_masked_ue8m0_packed(const void* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                                            const void* B, int64_t ldb, const int32_t* sb,
                                            void* D, int64_t ldd, const int32_t* masked_m,
                                            int G, int M_max, int N, int K, int expected_m,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Scale factors into the layout the GEMMs read: the analog of the pages'
 * transform_sf_into_required_layout (es.news.hada.io/topic?id=19459, "Utilidades y
 * variables de entorno"; the LHS scales must be aligned and transposed, "Interfaz GEMM y
 * restricciones de layout"). Input: FP32 scales given per row, sf[r][kb] (row stride
 * ld_sf >= nkb), as a quantiser produces them: rows = M for activation scales (one per
 * row per 128-wide K block), rows = ceil(N/128) for weight scales (one per 128x128
 * block). Output (out, row stride ld_out, in 32-bit entries):
 *   is_activation, !pack: FP32 [nkb][ld_out], out[kb][r] = sf[r][kb] (ld_out >= rows, % 4 == 0)
 *   is_activation,  pack: int32 [ceil(nkb/4)][ld_out], packed UE8M0 words as above
 *   !is_activation, !pack: FP32 [rows][ld_out], a copy (ld_out >= nkb)
 *   !is_activation,  pack: int32 [rows][ld_out] packed words (ld_out >= ceil(nkb/4))
 * Packing takes the UE8M0 code of each scale: the smallest power of two not below it
 * (exact for powers of two; other values round up). Precondition (device data): every
 * scale is a positive normal FP32 value of at most 2^127. Entries of out beyond the
 * rows x columns written are untouched. Device pointers owned by the caller; the work
 * is enqueued on `stream`. Errors: FP8GEMM_ERR_NULL, _SHAPE (rows < 0, nkb <= 0),
 * _LAYOUT (strides, 4-byte alignment), _DEVICE, _LAUNCH; rows == 0 is a no-op.
 */
int fp8_transform_sf_into_required_layout(const float* sf, int64_t ld_sf, int rows, int nkb, int is_activation,
                                          int pack, void* out, int64_t ld_out, hipStream_t stream);

/*
 * M-grouped contiguous GEMM (MoE training forward / inference prefill; pages:
 * es.news.hada.io/topic?id=19459 "Dense y Grouped GEMM", contiguous layout).
 * The tokens of all G experts are concatenated along M; each expert segment is
 * padded to a multiple of fp8_gemm_get_mk_alignment_for_contiguous_layout() (128)
 * rows, and N and K are shared by all experts.
 *   A  e4m3 [M_total, K] (stride lda); sa fp32 [K/128][ld_sa], ld_sa >= M_total.
 *   B  e4m3 [G, N, K]: expert g at B + g * N * ldb; sb fp32 [G][ceil(N/128)][K/128].
 *   D  bf16 [M_total, N] (stride ldd).
 *   m_indices int32 [M_total] on the device: expert of row r, or -1 for a padding
 *      row. Precondition: within every 128-row block all entries other than -1
 *      are equal and < G. Rows with -1 are not written (D keeps its contents).
 *      Blocks made only of -1 rows cost no compute.
 */
int fp8_grouped_gemm_nt_contiguous(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                   const void* B, int64_t ldb, const float* sb,
                                   void* D, int64_t ldd, const int32_t* m_indices,
                                   int M_total, int N, int K, int G,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * M-grouped masked GEMM (MoE decode under graph capture; pages:
 * es.news.hada.io/topic?id=19459 "Dense y Grouped GEMM", masked layout: with a
 * mask tensor only the valid regions are computed; GeekNews topic 19444: the CPU
 * does not know the per-expert token counts).
 *   A  e4m3 [G, M_max, K]: group g at A + g * M_max * lda.
 *   sa fp32 [G][K/128][ld_sa], ld_sa >= M_max.
 *   B  e4m3 [G, N, K]; sb fp32 [G][ceil(N/128)][K/128].
 *   D  bf16 [G, M_max, N]: group g at D + g * M_max * ldd.
 *   masked_m int32 [G] on the device: rows [0, masked_m[g]) of group g are
 *      computed; rows at or beyond it are not written. Values are clamped to
 *      [0, M_max]. The host never reads masked_m, so the call is graph-capturable.
 *   expected_m: host-side hint of the typical masked_m (tile choice and split-K
 *      workspace size).
 *   G <= 1024.
 * Split-K workspace: optional, as for the other calls. Its partials are sized for the
 * live tiles of up to twice expected_m rows per group (fp8_gemm_workspace_size with
 * FP8GEMM_KIND_MASKED and the same expected_m); a call whose masked_m hold more live
 * tiles than the workspace fits runs without split-K (decided on the device; the
 * results do not depend on it beyond FP32 summation order).
 */
int fp8_grouped_gemm_nt_masked(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                               const void* B, int64_t ldb, const float* sb,
                               void* D, int64_t ldd, const int32_t* masked_m,
                               int G, int M_max, int N, int K, int expected_m,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The M-grouped calls with UE8M0 scale factors (the UE8M0 scale format of
 * es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout", on the
 * grouped layouts of "Dense y Grouped GEMM"): the same operations, layouts,
 * preconditions and errors as fp8_grouped_gemm_nt_contiguous and
 * fp8_grouped_gemm_nt_masked, with every scale an exact power of two held as FP32
 * (see fp8_gemm_nt_ue8m0): the block-scaled MFMA applies them.
 */
int fp8_grouped_gemm_nt_contiguous_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                         const void* B, int64_t ldb, const float* sb,
                                         void* D, int64_t ldd, const int32_t* m_indices,
                                         int M_total, int N, int K, int G,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_grouped_gemm_nt_masked_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                     const void* B, int64_t ldb, const float* sb,
                                     void* D, int64_t ldd, const int32_t* masked_m,
                                     int G, int M_max, int N, int K, int expected_m,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense GEMM in the TN layout: D = A^T B with A stored [K][M] and B stored [K][N]
 * (the pages list the NT, TN, NN and TT layouts of the dense call, fp8_gemm_{nt,nn,
 * tn,tt}: es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout").
 * The scales keep their meaning and layouts from fp8_gemm_nt: sa [K/128][ld_sa] (one
 * per m per 128-K block), sb [ceil(N/128)][K/128] (one per 128x128 block); BF16 D [M][N]
 * rounded to nearest even once.
 *   A   e4m3 [K][lda], lda >= M, lda % 16 == 0, lda <= 2^24, 16-byte aligned.
 *   B   e4m3 [K][ldb], ldb >= N, same rules.
 *   sa  ld_sa >= M, ld_sa % 4 == 0; sb contiguous; both 4-byte aligned.
 *   D   BF16 [M][ldd], ldd >= N, 2-byte aligned (8-byte stores when ldd % 4 == 0 and D
 *       is 8-byte aligned).
 * M >= 0 (0: nothing to do), N > 0, K > 0 and a multiple of 128. Errors as for
 * fp8_gemm_nt. workspace / workspace_bytes: the optional split-K workspace of the
 * conventions above, sized by fp8_gemm_workspace_size(FP8GEMM_KIND_LAYOUT, M, N, K, 1,
 * 0); the TN, NN and TT calls split K when their tiles would leave most CUs idle (the
 * few-row shapes).
 */
int fp8_gemm_tn(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                const void* B, int64_t ldb, const float* sb,
                void* D, int64_t ldd, int M, int N, int K,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The dense call in the NN and TT layouts (es.news.hada.io/topic?id=19459, "Interfaz
 * GEMM y restricciones de layout" and "Dense y Grouped GEMM": fp8_gemm_{nt, nn, tn,
 * tt}): D = A B with A stored [M][K]
 * (K contiguous, as in fp8_gemm_nt: lda >= K) and B stored [K][N] (ldb >= N); and
 * D = A^T B^T with A stored [K][M] (lda >= M) and B stored [N][K] (as in fp8_gemm_nt:
 * ldb >= K). Scales, output, alignment (leading dimensions multiples of 16, at most
 * 2^24), shape rules and errors as for fp8_gemm_tn.
 */
int fp8_gemm_nn(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                const void* B, int64_t ldb, const float* sb,
                void* D, int64_t ldd, int M, int N, int K,
                void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_gemm_tt(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                const void* B, int64_t ldb, const float* sb,
                void* D, int64_t ldd, int M, int N, int K,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The TN, NN and TT calls in the accumulate form D = C + A B (the pages' naming of every
 * GEMM, es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout"; see
 * fp8_gemm_nt_c): C is BF16 with D's shape, row stride ldc >= N, 2-byte
 * aligned (8-byte loads when ldc % 4 == 0 and C is 8-byte aligned), added in FP32 to the
 * accumulator before the one rounding; C may be D itself (in-place accumulation), any
 * other overlap with D is not allowed. Otherwise as fp8_gemm_tn / _nn / _tt;
 * FP8GEMM_ERR_NULL for a NULL C, FP8GEMM_ERR_LAYOUT for ldc < N or a misaligned C.
 */
int fp8_gemm_tn_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                  const void* B, int64_t ldb, const float* sb, const void* C, int64_t ldc,
                  void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_gemm_nn_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                  const void* B, int64_t ldb, const float* sb, const void* C, int64_t ldc,
                  void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_gemm_tt_c(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                  const void* B, int64_t ldb, const float* sb, const void* C, int64_t ldc,
                  void* D, int64_t ldd, int M, int N, int K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The TN, NN and TT calls with UE8M0 scale factors (both from es.news.hada.io/topic?
 * id=19459, "Interfaz GEMM y restricciones de layout"): the same operations, layouts and
 * errors, with every sa and sb value an exact power of two 2^(e-127), 1 <= e <= 254,
 * held as FP32 (see fp8_gemm_nt_ue8m0); the block-scaled MFMA applies them.
 */
int fp8_gemm_tn_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const void* B, int64_t ldb, const float* sb,
                      void* D, int64_t ldd, int M, int N, int K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_gemm_nn_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const void* B, int64_t ldb, const float* sb,
                      void* D, int64_t ldd, int M, int N, int K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);
int fp8_gemm_tt_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const void* B, int64_t ldb, const float* sb,
                      void* D, int64_t ldd, int M, int N, int K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * K-grouped TN GEMM, the MoE weight-gradient form: grouping along K with M and N
 * fixed (es.news.hada.io/topic?id=19459, "Dense y Grouped GEMM",
 * k_grouped_fp8_gemm_tn_contiguous; "TN" is the layout pair of D = A^T B, "Interfaz
 * GEMM y restricciones de layout"). Group g owns the K rows [k_g, k_g + ks[g]),
 * k_g = ks[0] + ... + ks[g-1], of both operands, and
 *   D[g][m][n] = (accumulate ? D[g][m][n] : 0)
 *                + sum over the 128-row blocks kb of group g of
 *                  P_kb[m][n] * sa[kb][m] * sb[kb][n],   P_kb = sum_k A[k][m] B[k][n],
 * accumulated in FP32 (the scaled block partials added one by one). The pages give no
 * scale granularity or output type for this call; the reading implemented: both
 * operands are token-axis activations quantised per column per 128 K rows, and the
 * output is FP32 (weight gradients), optionally accumulated.
 *   A   e4m3 [K][M] (K = sum of ks), row stride lda bytes: lda >= M, lda % 16 == 0,
 *       16-byte aligned, lda <= 2^24. Bytes in columns M..lda-1 are read but unused.
 *   sa  fp32 [K/128][ld_sa]: sa[kb * ld_sa + m], ld_sa >= M, 4-byte aligned.
 *   B   e4m3 [K][N], row stride ldb: as A with N.
 *   sb  fp32 [K/128][ld_sb]: sb[kb * ld_sb + n], ld_sb >= N.
 *   D   fp32 [G][M][N]: D[g * d_gstride + m * ldd + n], ldd >= N, 4-byte aligned;
 *       d_gstride >= (M - 1) * ldd + N when G > 1. Elements outside the G x M x N
 *       box are not touched.
 *   ks  HOST array of G group lengths in K rows, each >= 0 and a multiple of 128
 *       (fp8_gemm_get_mk_alignment_for_contiguous_layout); a group with ks[g] == 0
 *       writes D[g] = 0 (or leaves it unchanged when accumulating).
 *   G   1 .. 256 groups; M, N >= 1; K <= 2^31 - 1.
 * Device pointers are owned by the caller; ks is read before the call returns; the
 * work is enqueued on `stream`. Errors: FP8GEMM_ERR_NULL, _SHAPE (G, M, N out of
 * range, a group length that is negative or not a multiple of 128), _LAYOUT (strides,
 * alignment), _DEVICE, _LAUNCH; nothing is launched on an argument error.
 */
int fp8_k_grouped_gemm_tn_contiguous(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                     const void* B, int64_t ldb, const float* sb, int64_t ld_sb,
                                     float* D, int64_t ldd, int64_t d_gstride,
                                     const int32_t* ks, int G, int M, int N, int accumulate,
                                     hipStream_t stream);

/*
 * The K-grouped TN GEMM with UE8M0 scale factors (the call of es.news.hada.io/topic?
 * id=19459, "Dense y Grouped GEMM", with the UE8M0 scale format of "Interfaz GEMM y
 * restricciones de layout"): the same operation, layouts,
 * preconditions and errors as fp8_k_grouped_gemm_tn_contiguous, with every sa and sb
 * value an exact power of two 2^(e-127), 1 <= e <= 254, held as FP32 (see
 * fp8_gemm_nt_ue8m0). gfx950's block-scaled MFMA applies them: each lane passes the
 * exponent of its A row and of its B row, which is the per-column scaling of both
 * operands, and accumulates the scaled block products itself.
 */
int fp8_k_grouped_gemm_tn_contiguous_ue8m0(const void* A, int64_t lda, const float* sa, int64_t ld_sa,
                                           const void* B, int64_t ldb, const float* sb, int64_t ld_sb,
                                           float* D, int64_t ldd, int64_t d_gstride,
                                           const int32_t* ks, int G, int M, int N, int accumulate,
                                           hipStream_t stream);

/*
 * 1x128 activation quantisation: the step upstream of every call above, producing
 * the A operand and its scales (one FP32 scale per row per 128-wide K block:
 * GeekNews topic 19444, intro). The pages leave FP8 conversion to the user
 * (es.news.hada.io/topic?id=19459, "Interfaz GEMM y restricciones de layout"); the
 * reading implemented here, per row and block, in FP32 with IEEE round-to-nearest-
 * even operations:  s = amax(|x|) / 448 (s = 1 when that is 0),  q = e4m3_rne(x / s)
 * (correctly rounded division; ties to the even code; at most 448 in magnitude).
 *   X  [M, K] row-major, row stride ldx (elements), FP32 or BF16 (x_dtype below);
 *      16-byte aligned, ldx a multiple of 4 (FP32) or 8 (BF16). NaN inputs are
 *      outside the contract.
 *   Q  e4m3 [M, K] row-major, row stride ldq; 8-byte aligned, ldq % 8 == 0.
 *   sa fp32 [K/128][ld_sa]: sa[kb * ld_sa + m], ld_sa >= M and a multiple of 4
 *      (the GEMMs' activation-scale layout); columns ld_sa > m >= M are untouched.
 * All pointers are device pointers owned by the caller; the work is enqueued on
 * `stream`. Errors: FP8GEMM_ERR_NULL, _SHAPE (M < 0, K <= 0 or K % 128), _LAYOUT
 * (strides, alignment, unknown x_dtype), _DEVICE, _LAUNCH; nothing is launched on an
 * argument error. M == 0 is a no-op.
 */
enum { FP8GEMM_QUANT_BF16 = 0, FP8GEMM_QUANT_FP32 = 1 };
int fp8_quantize_1x128(const void* X, int64_t ldx, int x_dtype, void* Q, int64_t ldq,
                       float* sa, int64_t ld_sa, int M, int K, hipStream_t stream);

/*
 * The same quantisation fused with the SwiGLU of the MoE FFN, producing the down
 * projection's A operand from the gate+up projection's output: the MoE pipeline the
 * pages list runs linear 1, then SwiGLU, then linear 2 (es.news.hada.io/topic?id=19459,
 * "Mega MoE"), and the grouped calls compute the two linears. The SwiGLU reading (gate
 * half first, silu(x) = x * sigmoid(x)) is the standard one; the pages give no formula.
 * Per row r and column k < F:
 *     y = silu(g) * u,  silu(g) = g / (1 + exp(-g)),  g = H[r][k], u = H[r][F + k]
 * evaluated in FP64 and rounded once to FP32 (the FP32 value nearest the exact y, but
 * when that lies within ~2^-28 of an FP32 ulp of a rounding midpoint), then quantised
 * exactly as by fp8_quantize_1x128 (s = amax / 448 per 128-column block, q =
 * e4m3_rne(y / s)).
 *   H  [M, 2F] row-major (gate in columns 0..F-1, up in F..2F-1), row stride ldh
 *      (elements) >= 2F, BF16 or FP32 (h_dtype); 16-byte aligned, ldh a multiple
 *      of 8 (BF16) or 4 (FP32); F a positive multiple of 128.
 *   m_indices  optional int32 [M] (NULL: every row live): rows with -1 (padding of
 *      the contiguous layout) quantise as zeros (codes 0, scale 1).
 *   Q, sa  as for fp8_quantize_1x128 with K = F.
 * Errors as for fp8_quantize_1x128 (_SHAPE for F <= 0 or F % 128).
 */
int fp8_swiglu_quantize_1x128(const void* H, int64_t ldh, int h_dtype, const int32_t* m_indices, void* Q,
                              int64_t ldq, float* sa, int64_t ld_sa, int M, int F, hipStream_t stream);

/* Bytes of split-K workspace the call with these sizes may use (0 = never splits).
 * Splitting K is this library's choice for MI355X (the pages' Hopper kernels do not
 * split K), so this utility has no counterpart on the pages.
 * kind: FP8GEMM_KIND_*. M is M (dense, layout), M_total (contiguous) or M_max
 * (masked). expected_m is the masked call's tiling hint, taken here so that the answer
 * is computed by the same planner with the same arguments as the call itself (the
 * masked workspace holds the live tiles of up to twice expected_m rows per group); it
 * is ignored for the other kinds. The size includes the 16 KiB counter block
 * described in the conventions above. */
size_t fp8_gemm_workspace_size(int kind, int M, int N, int K, int G, int expected_m);

/* Configuration the library would use for a call (no launch, no device access
 * when fp8_gemm_set_num_cus() has been given a value). Returns FP8GEMM_OK. The
 * pages' configuration printout (es.news.hada.io/topic?id=19459, "Utilidades y
 * variables de entorno": DG_PRINT_CONFIGS prints the configuration chosen per shape)
 * as a query; FP8GEMM_PRINT_CONFIGS=1 prints it at every call. */
int fp8_gemm_query_config(int kind, int M, int N, int K, int G, int expected_m,
                          size_t workspace_bytes, fp8gemm_config_t* out);

/* Force the tile configuration of later calls (tuning and tests; a utility of this
 * library with no counterpart on the pages): block_m,
 * block_n, split_k and full_tiles (clamped to the tile count; 0 splits every
 * tile) are used, grid and num_units are ignored. NULL restores
 * automatic selection. Not thread-safe; process-wide.
 * Returns FP8GEMM_ERR_CONFIG for a tile shape that no call has a kernel for; a later
 * call returns FP8GEMM_ERR_CONFIG if it has no kernel for the forced tile (the NT and
 * M-grouped calls: 64x64, 128x64, 64x128, 128x128, 256x128, 128x256, 64x96, 128x96; the TN / NN / TT
 * calls: 128x128, 256x256, 64x128, 128x64, which ignore full_tiles and do not split K
 * with 256x256) or if the forced plan splits more than 4096 tiles. */
int fp8_gemm_force_config(const fp8gemm_config_t* cfg);

/* Cap on the compute units the persistent grid is sized for: the analog of
 * DeepGEMM's set_num_sms / get_num_sms (es.news.hada.io/topic?id=19459, "Utilidades
 * y variables de entorno": set and query the maximum number of SMs to use). n <= 0
 * restores the device's own count. get returns the value in effect (0 if none is
 * known yet). */
int fp8_gemm_set_num_cus(int n);
int fp8_gemm_get_num_cus(void);

/* Row alignment of each expert segment in the contiguous layout, and of each group's
 * K length in the K-grouped call: 128. The pages require every expert segment of the
 * contiguous layout to be aligned to the GEMM's M block size and expose that
 * alignment through get_mk_alignment_for_contiguous_layout (es.news.hada.io/topic?
 * id=19459, "Dense y Grouped GEMM"; the same getter, group-level M/K alignment, in
 * "Utilidades y variables de entorno"). Here it is fixed at one scale block (128
 * rows), which every tile height used by the contiguous call divides, so a tile
 * never spans two experts. No setter: the value cannot change. */
int fp8_gemm_get_mk_alignment_for_contiguous_layout(void);

/* Smallest valid ld_sa for `rows` rows: rows rounded up to a multiple of 4. The
 * analog of DeepGEMM's get_tma_aligned_size (es.news.hada.io/topic?id=19459,
 * "Utilidades y variables de entorno": the alignment size the LHS scale layout
 * needs; "Interfaz GEMM y restricciones de layout": the LHS scales must be aligned
 * and transposed). Here the activation scales are [K/128][ld_sa] FP32 and the
 * kernels read them in 16-byte groups, so ld_sa must be a multiple of 4. rows <= 0
 * gives 0. */
int64_t fp8_gemm_scale_ld(int64_t rows);

/* Number of output tiles of an M x N output cut into block_m x block_n tiles: the
 * count behind the pages' unaligned-block argument (deepep.org/zh/deepgemm, 核心优化技术,
 * 非对齐块大小: the number of tiles decides how many SMs get work). */
int64_t fp8_gemm_num_tiles(int64_t M, int64_t N, int block_m, int block_n);

/* Static description of a status code (a utility of this library with no counterpart
 * on the pages). */
const char* fp8_gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H_ */
