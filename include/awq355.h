/*
 * awq355.h - C ABI of libawq355.so: the W4A16 group-quantized linear layer of
 * activation-aware weight quantization (AWQ), and the offline alpha-grid scale
 * search that produces its weights, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  - "AWQ Advanced Usage Guide" (skillselion.com awq-quantization skill):
 *    "How AWQ Works" (objective L(s) = ||Q(W*s)(s^-1*X) - W*X||),
 *    "WQLinear Kernel Variants" (GEMM for batches, GEMV for single tokens),
 *    "Group Size Configuration" and "Zero-Point Quantization"
 *    (w_bit = 4, q_group_size = 128, zero_point = True).
 *  - ai.lansai.wang AWQ explainer, section "AWQ 的四步链路" (Y = XW =
 *    (X/s)(sW), s positive per input channel; statistics -> scale search ->
 *    pack) and its checkpoint-field table (group = consecutive weights
 *    sharing quantization parameters; zero_point = asymmetric mapping).
 *
 * Conventions for every entry point
 *  - Pointers marked "device" point to memory of the current HIP device; the
 *    caller owns every buffer.  The library keeps no state and allocates no
 *    memory except where an entry point says otherwise.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns without waiting, unless the
 *    entry point says it synchronizes.
 *  - Arguments are validated before anything is enqueued; on any error no
 *    output is written and a status code is returned.  awq_last_error()
 *    returns a message describing the most recent error of the calling
 *    thread.
 *  - Matrices are dense, row-major, with no padding between rows.
 *
 * Quantized weight layout (fixed by this library; the pages fix none):
 *  - qweight  u32 [N][K/8]: nibble p (bits 4p..4p+3) of word c of row n holds
 *             the 4-bit code of input channel 8c + ORDER[p],
 *             ORDER = {0, 2, 4, 6, 1, 3, 5, 7}.
 *  - scales   fp16 bits [N][K/g]: step of group k/g of row n.
 *  - zeros    u8   [N][K/g]: zero point (0..15) of that group.
 *  - weight(n, k) = (code - zero) * scale.
 */
#ifndef AWQ355_H
#define AWQ355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Mirror of the pages' quant_config fields (w_bit, q_group_size,
 * zero_point).  Supported: w_bit = 4, group_size in {64, 128},
 * zero_point = 1. */
typedef struct awq_config {
    int32_t w_bit;
    int32_t group_size;
    int32_t zero_point;
} awq_config;

typedef enum awq_status {
    AWQ_OK = 0,
    AWQ_ERR_INVALID_ARG = 1, /* bad shape, NULL pointer, misalignment, bad enum */
    AWQ_ERR_UNSUPPORTED = 2, /* a config this build does not implement */
    AWQ_ERR_WORKSPACE = 3,   /* workspace smaller than required */
    AWQ_ERR_HIP = 4,         /* the HIP runtime reported an error (incl. no device) */
    AWQ_ERR_NONFINITE = 5    /* reserved: non-finite input detected */
} awq_status;

/* Element types (int32_t in signatures). */
enum { AWQ_F16 = 0, AWQ_BF16 = 1, AWQ_F32 = 2 };

/* Kernel selection for awq_linear_ex (int32_t in signatures).  The pages'
 * `version` knob (GEMM / GEMV) becomes a dispatch on M in awq_linear. */
enum { AWQ_KERNEL_AUTO = 0, AWQ_KERNEL_GEMV = 1, AWQ_KERNEL_GEMM = 2 };

typedef void *awq_stream_t;

/* Upper bound on M for the GEMV kernel (awq_linear dispatches M <= this to
 * it; awq_linear_ex(AWQ_KERNEL_GEMV) rejects larger M). */
#define AWQ_GEMV_MAX_M 16

/*
 * awq_quantize_pack - scale, group-quantize and pack a weight matrix.
 * Cites: "AWQ Advanced Usage Guide", "Group Size Configuration" and
 * "Zero-Point Quantization"; ai.lansai.wang explainer, checkpoint-field
 * table ("group" and "zero_point" rows) and section "AWQ 的四步链路" (the sW
 * of Y = (X/s)(sW); "真实量化/打包" row).
 *
 *   W        device, fp16 [N][K], 16-byte aligned.
 *   s        device, fp32 [K] per-input-channel scale, or NULL for s = 1.
 *   qweight  device, u32 [N][K/8], 16-byte aligned (layout above).
 *   scales   device, fp16 bits [N][K/g].
 *   zeros    device, u8 [N][K/g].
 *   nonfinite_count  device int32 or NULL.  When given, the number of
 *            non-finite values among s_k * W_nk is ADDED to it (the caller
 *            clears it); outputs of groups holding such values are unspecified.
 *
 * Per group of g consecutive k of one row, with v = fp32(s_k * W_nk):
 *   lo = min(min v, 0), hi = max(max v, 0), scale = fp16(max((hi-lo)/15, 2^-14)),
 *   zero = clamp(rint(-lo/scale), 0, 15), code = clamp(rint(v/scale) + zero, 0, 15),
 * fp32 correctly-rounded division, rint = round half to even.
 * Requirements: N >= 0, K > 0, K % g == 0.  N == 0 is a no-op.
 */
awq_status awq_quantize_pack(const void *W, int64_t N, int64_t K, awq_config cfg,
                             const float *s, uint32_t *qweight, uint16_t *scales,
                             uint8_t *zeros, int32_t *nonfinite_count,
                             awq_stream_t stream);

/*
 * awq_linear - Y = X * deq(W)^T, the W4A16 linear layer.
 * Cites: "AWQ Advanced Usage Guide", "WQLinear Kernel Variants" (GEMM for
 * batch > 1, GEMV for single-token decode); ai.lansai.wang explainer, table
 * of common claims (weight-only: activations stay 16-bit, W4A16).
 *
 *   X        device, [M][K] of x_dtype (AWQ_F16 or AWQ_BF16), 16-byte aligned.
 *   qweight, scales, zeros: as produced by awq_quantize_pack for [N][K].
 *   Y        device, [M][N] of y_dtype (AWQ_F16, AWQ_BF16 or AWQ_F32).
 *
 * Dispatch (where each measured faster): the GEMV kernel for M <=
 * AWQ_GEMV_MAX_M when its activation rows fit in LDS (M * K * 2 <= 128 KiB
 * for N <= 4096, else 64 KiB);
 * otherwise, unless K / group_size exceeds 8 times its waves per workgroup
 * (16 when N <= 4096, else 8), for M <= 8, and for M <= 12 when
 * N * K <= 5e7; else the MFMA GEMM.
 * GEMV: products of the exact integer (code - zero) and the 16-bit
 * activation, accumulated in fp32 within a group, multiplied by the group's
 * scale and accumulated in fp32 across groups.  GEMM: the dequantized weight
 * (code - zero) * scale is rounded once to fp16 (relative error <= 2^-11),
 * as the pages' GEMM kernels dequantize to fp16, and the products are
 * accumulated in fp32; bf16 activations are scaled per row by a power of two
 * into fp16's range (exact) and the row's output divided by it.  Y is rounded
 * once to y_dtype.  When its tiles alone cannot fill the GPU, the GEMM splits K
 * across workgroups and needs a scratch buffer (see awq_linear_ws); bf16
 * activations need one too (a factor per row, and for shapes large enough
 * for the 256-row tile an fp16 copy of X, M * K * 2 bytes): awq_linear
 * and awq_linear_ex take it from a per-device buffer the library allocates the
 * first time a shape needs it (or needs more) and keeps until the process
 * ends.  Consequently (a) inside a HIP-graph capture, first call the same
 * shape once outside the capture; (b) calls on one device that need the
 * scratch and may overlap in time (different streams) share that buffer and
 * must instead use awq_linear_ws with a workspace each.
 * Requirements: M, N >= 0, K > 0, K % g == 0.  M == 0 or N == 0 is a no-op.
 */
awq_status awq_linear(const void *X, int32_t x_dtype, const uint32_t *qweight,
                      const uint16_t *scales, const uint8_t *zeros, int64_t M,
                      int64_t N, int64_t K, awq_config cfg, void *Y,
                      int32_t y_dtype, awq_stream_t stream);

/*
 * awq_linear_ex - awq_linear with an explicit kernel choice (AWQ_KERNEL_*),
 * so the GEMV and GEMM paths can be compared on the same call (the pages
 * quote GEMV as faster than GEMM at batch size 1: "WQLinear Kernel Variants").
 * AWQ_KERNEL_GEMV requires M <= AWQ_GEMV_MAX_M (else AWQ_ERR_INVALID_ARG).
 */
awq_status awq_linear_ex(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M,
                         int64_t N, int64_t K, awq_config cfg, void *Y,
                         int32_t y_dtype, int32_t kernel, awq_stream_t stream);

/*
 * awq_linear_workspace_size - bytes of device workspace awq_linear_ws needs
 * for this shape, for either activation type (0: none; also 0 on invalid
 * arguments).
 */
size_t awq_linear_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg);

/*
 * awq_linear_ws - awq_linear (automatic kernel choice) with a caller-owned
 * workspace instead of the library's scratch; allocates nothing.
 * Cites: as awq_linear.
 *
 *   workspace  device, at least awq_linear_workspace_size() bytes, 256-byte
 *            aligned.  Scratch only: its contents on entry are ignored and
 *            on return are unspecified, so it needs no clearing and can be
 *            reused by later calls of any shape.  May be NULL when the size
 *            is 0.
 *   Calls that share a workspace must not overlap in time.
 * Errors: AWQ_ERR_WORKSPACE when workspace_bytes is too small; otherwise as
 * awq_linear.
 */
awq_status awq_linear_ws(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, void *workspace,
                         size_t workspace_bytes, awq_stream_t stream);

/*
 * awq_scale_search_workspace_size - bytes of device workspace that
 * awq_scale_search needs for these sizes (0 on invalid arguments).
 */
size_t awq_scale_search_workspace_size(int64_t M, int64_t N, int64_t K,
                                       awq_config cfg, int32_t n_alpha);

/*
 * awq_scale_search - activation-aware equivalent-scaling search for one layer.
 * Cites: "AWQ Advanced Usage Guide", "How AWQ Works" (salient channels from
 * activation distributions; L(s) = ||Q(W*s)(s^-1*X) - W*X||); ai.lansai.wang
 * explainer, section "AWQ 的四步链路" (Y = (X/s)(sW); the "采集激活" and
 * "搜索缩放" rows: record input magnitudes, evaluate candidate scalings by
 * their reconstruction error).
 *
 *   X        device, fp16 [M][K] calibration activations, 16-byte aligned.
 *   W        device, fp16 [N][K] weights, 16-byte aligned.
 *   alphas   host, fp64 [n_alpha], each in [0, 1]; NULL selects the grid
 *            alpha_j = j/20, j = 0..19 (then n_alpha must be 20).
 *   workspace  device, at least awq_scale_search_workspace_size() bytes,
 *            256-byte aligned.  Its contents are clobbered.
 *   best_index host int32: the chosen j (the smallest j attaining the minimum).
 *   losses   host fp64 [n_alpha] or NULL: L_j for every candidate.
 *   best_s   device fp32 [K]: s of the chosen candidate.
 *   qweight, scales, zeros: device, awq_quantize_pack(W, best_s) outputs.
 *
 * For candidate j: xbar_k = mean_m |X_mk| (fp64, exact), t = max(xbar,
 * 2^-24)^alpha_j, s = fp32(t / sqrt(max t * min t)); A = fp16(X / s);
 * L_j = sum over (m, n) of (X W^T - A deq(Q(s W))^T)^2, with X W^T in fp32 and
 * L accumulated in fp64.
 * Synchronization: the call waits on `stream` once, after the losses are
 * known, to fill best_index and losses; the final quantize/pack of the chosen
 * candidate is enqueued after that and is complete when `stream` is.
 * Requirements: M >= 1, N >= 1, 1 <= n_alpha <= 64, K % g == 0.
 */
awq_status awq_scale_search(const void *X, const void *W, int64_t M, int64_t N,
                            int64_t K, awq_config cfg, const double *alphas,
                            int32_t n_alpha, void *workspace,
                            size_t workspace_bytes, int32_t *best_index,
                            double *losses, float *best_s, uint32_t *qweight,
                            uint16_t *scales, uint8_t *zeros,
                            awq_stream_t stream);

/* Static description of a status code. */
const char *awq_status_string(awq_status status);

/* Message for the calling thread's most recent error ("" if none). */
const char *awq_last_error(void);

/* Library version string. */
const char *awq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AWQ355_H */
