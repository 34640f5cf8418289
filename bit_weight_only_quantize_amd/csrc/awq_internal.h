// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the caller and
// returns the hipError_t of the launch.  A null `zeros` pointer selects the
// symmetric grid (zero_point = 0): no zero point is read or written, and
// every group's zero is 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

enum class XType : int { F16 = 0, BF16 = 1 };
enum class YType : int { F16 = 0, BF16 = 1, F32 = 2 };

// ---- quantize_pack.hip -----------------------------------------------------
hipError_t launch_quantize_pack(const uint16_t *W, int64_t N, int64_t K, int gs,
                                const float *s, uint32_t *qweight,
                                uint16_t *scales, uint8_t *zeros,
                                int32_t *nonfinite, hipStream_t st);

// W'[n][k] = (q - z) * s as fp32 (f32) or fp16 [N][K] (quantize_pack.hip).
hipError_t launch_dequantize(const uint32_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, int gs, void *out, bool f32, hipStream_t st);

// One weight set of a fused launch: packed [N][K] weights and its output [M][N].
struct LinearPart {
  const uint32_t *qweight;
  const uint16_t *scales;
  const uint8_t *zeros;
  int64_t N;
  void *Y;
};

// ---- linear_gemv.hip (M <= 16) -------------------------------------------------
// Whether the GEMV kernel can serve this shape (M <= 16, its LDS fits) with
// np weight sets per workgroup (1, or 2 for the gate/up pair).
bool gemv_supported(int64_t M, int64_t N, int64_t K, int gs, int np = 1);
// Whether the GEMV stages the M activation rows in LDS (its fast path).
bool gemv_stages_activations(int64_t M, int64_t N, int64_t K);
// Groups of K each GEMV wave walks in sequence.
int64_t gemv_groups_per_wave(int64_t N, int64_t K, int gs);
hipError_t launch_gemv(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M,
                       int64_t N, int64_t K, int gs, void *Y, YType yt,
                       hipStream_t st);
// Up to 4 weight sets sharing X in one launch (each writes its own Y); with
// silu_mul, exactly 2 of equal N and Y of part 0 receives silu(X W0^T) *
// (X W1^T).  The zero-point mode of part 0 holds for all parts.
hipError_t launch_gemv_parts(const void *X, XType xt, const LinearPart *parts, int count,
                             bool silu_mul, int64_t M, int64_t K, int gs, YType yt,
                             hipStream_t st);

// ---- split K (gemm_f16.hip) ---------------------------------------------------------
// Split-K bookkeeping of one launch: `splits` workgroups per output tile, each
// storing its fp32 partial tile for the reduction kernel that follows.
struct SplitK {
  int splits;
  float *partials;   // [tile][split] fp32 partial tiles, summed by a second kernel
};

// ---- the quantized GEMM (any M) -------------------------------------------------
// What scratch memory a GEMM plan may use.
enum class Scratch : int {
  Full = 0,     // K split when the tiles cannot fill the CUs; bf16: row factors, and a
                // converted fp16 copy of X (M * K * 2 bytes) for the 256-row tile
  Bounded = 1,  // as Full, but bf16 input never takes the 256-row tile (no copy of X):
                // at most kBoundedPartialBytes of partials plus M * 4 bytes of factors
  None = 2,     // nothing: K is never split; bf16 input still needs its row factors
};
// Upper bound of a plan's split-K partials: tiles * splits <= 256 slots of at
// most 128 x 256 fp32.
constexpr size_t kBoundedPartialBytes = (size_t)256 * 128 * 256 * 4;

// Row tile (16 * mt rows), K split and workspace of a quantized GEMM
// (gemm_f16.hip; gemm_plan and the wrappers below are in linear_gemm.hip).
struct GemmPlan {
  int mt, splits;
  int64_t tiles;
  size_t rowf_offset;      // bf16 input: per-row activation factors (fp32 [M])
  size_t xh_offset;        // bf16 input, 256-row tile: X scaled to fp16 ([M][K]), else 0
  size_t workspace_bytes;  // 0 when splits == 1 and the input is fp16; partials first
};
// The plan of the kernel that serves activations of type xt.
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, XType xt, Scratch sc);
// Runs `plan` (from gemm_plan with the same M, N, K and xt).  `workspace`
// (plan.workspace_bytes, 256-byte aligned; its contents on entry are ignored)
// is needed only when plan.workspace_bytes > 0.
hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M,
                       int64_t N, int64_t K, int gs, void *Y, YType yt,
                       const GemmPlan &plan, void *workspace, hipStream_t st);

// ---- gemm_f16.hip (the quantized GEMM: fp16, or bf16 converted to fp16) ---------------
// Row tile (16 * mt rows), K split and workspace of the GEMM.
GemmPlan gemm_f16_plan(int64_t M, int64_t N, int64_t K, bool bf16, Scratch sc);
hipError_t launch_gemm_f16(const uint16_t *X, bool bf16, const uint32_t *qweight,
                           const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                           int64_t K, int gs, void *Y, YType yt, const GemmPlan &plan,
                           void *workspace, hipStream_t st);

// ---- linear_batched.hip (batched decode, M <= 64) ---------------------------------
// Workgroups of 256 columns over a range of gps groups of K (a split); with
// splits > 1 each writes fp32 partials ([split][M][N], partial_bytes of
// workspace) that a second kernel sums in split order.
struct BatchedPlan {
  int splits, gps;
  size_t partial_bytes;    // 0 when splits == 1
};
bool batched_gemv_supported(int64_t M, int64_t N, int64_t K, int gs);
BatchedPlan batched_gemv_plan(int64_t M, int64_t N, int64_t K, int gs, Scratch sc);
hipError_t launch_batched_gemv(const void *X, XType xt, const uint32_t *qweight,
                               const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                               int64_t K, int gs, void *Y, YType yt, const BatchedPlan &plan,
                               void *workspace, hipStream_t st);

// linear_gemm.hip: H = silu(A) * B elementwise over n fp32 values, rounded to yt.
hipError_t launch_silu_mul(const float *A, const float *B, int64_t n, void *H, YType yt,
                           hipStream_t st);

// linear_gemm.hip: the search's reference GEMM, X * W^T with W fp16 [N][K],
// fp32 output.
hipError_t launch_gemm_dense_f32(const uint16_t *X, const uint16_t *W, int64_t M,
                                 int64_t N, int64_t K, float *Y, hipStream_t st);

// gemm_f16.hip: the search's loss GEMM, exact q - z operand and fp32 group
// scaling, whose epilogue accumulates sum (Yref - Y)^2: one fp64 partial per
// workgroup tile into `partials` (gemm_tile_count entries).
hipError_t launch_gemm_loss(const uint16_t *A, const uint32_t *qweight,
                            const uint16_t *scales, const uint8_t *zeros,
                            int64_t M, int64_t N, int64_t K, int gs,
                            const float *Yref, double *partials, hipStream_t st);
int64_t gemm_tile_count(int64_t M, int64_t N);
// Whether a layer fits the kernels' 32-bit buffer offsets (packed weights, or
// the dense fp16 weights of the search, below 2 GiB).
bool gemm_supported(int64_t N, int64_t K, bool dense);

// ---- search.hip ----------------------------------------------------------------
// xbar[k] = sum_m |X[m][k]| / M in fp64 (exact sum; `units` is K u64 scratch).
hipError_t launch_mean_abs(const uint16_t *X, int64_t M, int64_t K, uint64_t *units,
                           double *xbar, hipStream_t st);
// s_table[j][k] for n_alpha alphas (host fp64 array); wbar (device, or NULL)
// enables duo scaling.
hipError_t launch_scale_table(const double *xbar, const double *wbar, int64_t K,
                              const double *alphas, int n_alpha, float *s_table, hipStream_t st);
// Weight clipping: points of the shrink grid, Gram partials per group
// (gram_parts(M) of GS*GS fp64 each), then per (row, group) the factor of
// least output error; writes the packed result for it (zeros NULL: symmetric)
// and, if clip_index is given, the chosen index (u8 [N][K/gs]).
constexpr int kClipPoints = 20;
int64_t gram_parts(int64_t M);
// fp64 entries of one group's Gram matrix as the clip selection reads it
// (the 16 x 16 blocks on and above the diagonal, in MFMA operand order).
constexpr int64_t clip_gram_doubles(int gs) { return (gs / 16) * (gs / 16 + 1) / 2 * 256; }
hipError_t launch_clip_search(const uint16_t *W, const float *s, const uint16_t *A, int64_t M,
                              int64_t N, int64_t K, int gs, double *gram_partial, double *gram,
                              uint32_t *qweight, uint16_t *scales, uint8_t *zeros,
                              uint8_t *clip_index, hipStream_t st);
// A = fp16(fp32(X) / s).
hipError_t launch_scale_activation(const uint16_t *X, const float *s, int64_t M,
                                   int64_t K, uint16_t *A, hipStream_t st);
// losses[j] = sum of partials[j][0..n) in index order; then best index.
hipError_t launch_reduce_losses(const double *partials, int64_t n_per_alpha,
                                int n_alpha, double *losses, int32_t *best,
                                hipStream_t st);

}  // namespace awq
