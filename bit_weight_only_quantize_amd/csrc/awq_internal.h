// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the caller and
// returns the hipError_t of the launch.
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

// ---- linear_gemv.hip (M <= 16) -------------------------------------------------
// Whether the GEMV kernel can serve this shape (M <= 16, its LDS fits).
bool gemv_supported(int64_t M, int64_t N, int64_t K, int gs);
// Whether the GEMV stages the M activation rows in LDS (its fast path).
bool gemv_stages_activations(int64_t M, int64_t N, int64_t K);
// Groups of K each GEMV wave walks in sequence.
int64_t gemv_groups_per_wave(int64_t N, int64_t K, int gs);
hipError_t launch_gemv(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M,
                       int64_t N, int64_t K, int gs, void *Y, YType yt,
                       hipStream_t st);

// ---- split K (gemm_f16.hip) ---------------------------------------------------------
// Split-K bookkeeping of one launch: `splits` workgroups per output tile, each
// storing its fp32 partial tile for the reduction kernel that follows.
struct SplitK {
  int splits;
  float *partials;   // [tile][split] fp32 partial tiles, summed by a second kernel
};

// ---- the quantized GEMM (any M) -------------------------------------------------
// Row tile (16 * mt rows), K split and workspace of a quantized GEMM
// (gemm_f16.hip; gemm_plan and the wrappers below are in linear_gemm.hip).
struct GemmPlan {
  int mt, splits;
  int64_t tiles;
  size_t rowf_offset;      // bf16 input: per-row activation factors (fp32 [M])
  size_t xh_offset;        // bf16 input, 256-row tile: X scaled to fp16 ([M][K]), else 0
  size_t workspace_bytes;  // 0 when splits == 1 and the input is fp16; partials first
};
// The plan of the kernel that serves activations of type xt (fp16: the
// kernel of gemm_f16.hip).
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, XType xt);
// Workspace that serves either activation type.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
// `workspace` (gemm_plan(...).workspace_bytes, 256-byte aligned; its contents
// on entry are ignored) is needed only when the plan's workspace_bytes > 0.
hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M,
                       int64_t N, int64_t K, int gs, void *Y, YType yt,
                       void *workspace, hipStream_t st);

// ---- gemm_f16.hip (the quantized GEMM: fp16, or bf16 converted to fp16) ---------------
// Row tile (16 * mt rows), K split and workspace of the GEMM.
GemmPlan gemm_f16_plan(int64_t M, int64_t N, int64_t K, bool bf16);
hipError_t launch_gemm_f16(const uint16_t *X, bool bf16, const uint32_t *qweight,
                           const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                           int64_t K, int gs, void *Y, YType yt, void *workspace, hipStream_t st);

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
// s_table[j][k] for n_alpha alphas (device fp64 array).
hipError_t launch_scale_table(const double *xbar, int64_t K, const double *alphas,
                              int n_alpha, float *s_table, hipStream_t st);
// A = fp16(fp32(X) / s).
hipError_t launch_scale_activation(const uint16_t *X, const float *s, int64_t M,
                                   int64_t K, uint16_t *A, hipStream_t st);
// losses[j] = sum of partials[j][0..n) in index order; then best index.
hipError_t launch_reduce_losses(const double *partials, int64_t n_per_alpha,
                                int n_alpha, double *losses, int32_t *best,
                                hipStream_t st);

}  // namespace awq
