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
 *    memory: scratch comes from workspaces the caller passes in.
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
 *  - zeros    u8   [N][K/g]: zero point (0..15) of that group; absent for
 *             the symmetric grid (zero_point = 0), whose zero is 8.
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
 * zero_point).  Supported: w_bit = 4, group_size in {64, 128}, zero_point =
 * 1 (asymmetric, a zero point per group) or 0 (symmetric: "Zero-Point
 * Quantization", no zero points; every entry point then ignores `zeros`,
 * which may be NULL, and the code of 0.0 is 8). */
typedef struct awq_config {
    int32_t w_bit;
    int32_t group_size;
    int32_t zero_point;
} awq_config;

typedef enum awq_status {
    AWQ_OK = 0,
    AWQ_ERR_INVALID_ARG = 1, /* bad shape, NULL pointer, misalignment, bad enum */
    AWQ_ERR_UNSUPPORTED = 2, /* a config the library does not implement */
    AWQ_ERR_WORKSPACE = 3,   /* workspace smaller than required */
    AWQ_ERR_HIP = 4,         /* the HIP runtime reported an error (incl. no device) */
    AWQ_ERR_NONFINITE = 5    /* reserved: non-finite input detected */
} awq_status;

/* Element types (int32_t in signatures). */
enum { AWQ_F16 = 0, AWQ_BF16 = 1, AWQ_F32 = 2 };

/* Kernel selection for awq_linear_ex (int32_t in signatures).  The pages'
 * `version` knob (GEMM / GEMV) becomes a dispatch on M in awq_linear.
 * AWQ_KERNEL_BATCHED is the batched-decode kernel between the two (M <=
 * AWQ_BATCHED_MAX_M): the GEMV's exact arithmetic with 256 output columns
 * per workgroup sharing each staged chunk of activations. */
enum { AWQ_KERNEL_AUTO = 0, AWQ_KERNEL_GEMV = 1, AWQ_KERNEL_GEMM = 2, AWQ_KERNEL_BATCHED = 3 };

typedef void *awq_stream_t;

/* Upper bound on M for the GEMV kernel (awq_linear dispatches M <= this to
 * it; awq_linear_ex(AWQ_KERNEL_GEMV) rejects larger M). */
#define AWQ_GEMV_MAX_M 16
/* Upper bound on M for AWQ_KERNEL_BATCHED. */
#define AWQ_BATCHED_MAX_M 64

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
 *   zeros    device, u8 [N][K/g] (zero_point = 1; ignored when 0).
 *   nonfinite_count  device int32 or NULL.  When given, the number of
 *            non-finite values among s_k * W_nk is ADDED to it (the caller
 *            clears it); outputs of groups holding such values are unspecified.
 *
 * Per group of g consecutive k of one row, with v = fp32(s_k * W_nk):
 *   lo = min(min v, 0), hi = max(max v, 0), scale = fp16(max((hi-lo)/15, 2^-14)),
 *   zero = clamp(rint(-lo/scale), 0, 15), code = clamp(rint(v/scale) + zero, 0, 15),
 * and with zero_point = 0 (no zeros written):
 *   scale = fp16(max(max |v| / 7, 2^-14)), code = clamp(rint(v/scale), -8, 7) + 8,
 * fp32 correctly-rounded division, rint = round half to even.
 * Requirements: N >= 0, K > 0, K % g == 0.  N == 0 is a no-op.
 */
awq_status awq_quantize_pack(const void *W, int64_t N, int64_t K, awq_config cfg,
                             const float *s, uint32_t *qweight, uint16_t *scales,
                             uint8_t *zeros, int32_t *nonfinite_count,
                             awq_stream_t stream);

/*
 * awq_dequantize - the packed weights back as floating-point weights: the
 * pseudo-quantized layer.
 * Cites: ai.lansai.wang explainer, four-stage table, "伪量化评测" row
 * (pseudo-quantized evaluation: simulate the low-bit weights without
 * depending on the target kernel).
 *
 *   qweight, scales, zeros: as produced by awq_quantize_pack for [N][K]
 *            (zeros ignored when cfg.zero_point = 0).
 *   out      device, [N][K] of out_dtype, 16-byte aligned: AWQ_F32 gives
 *            (code - zero) * scale exactly; AWQ_F16 rounds it once (nearest
 *            even).
 * awq_quantize_pack followed by awq_dequantize is the pseudo-quantization
 * of W (with s: of s * W).  Requirements: N >= 0, K > 0, K % g == 0.
 */
awq_status awq_dequantize(const uint32_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, awq_config cfg, void *out, int32_t out_dtype,
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
 * Arithmetic.  The GEMV and the GEMM's 32-row tile (M <= 32) multiply the
 * activations by the exact integers (code - zero), so every product is exact
 * in fp32; each group's fp32 sum is multiplied by the group's scale and
 * accumulated in fp32.  The GEMM's larger tiles (M > 32) multiply by the
 * dequantized weight (code - zero) * scale rounded once to fp16 (relative
 * error <= 2^-11 per weight; chosen for throughput, within the 1e-3
 * relative Frobenius tolerance) and accumulate in fp32; an output's extra
 * error is then at most 2^-11 * sum_k |x_k * w_k|.  bf16 activations on the
 * GEMM are scaled per row by a power of two into fp16's range (exact) and
 * the row's output divided by it.  Y is rounded once to y_dtype.
 * Allocation: none.  awq_linear uses no scratch memory: the GEMM runs without
 * splitting K (slower for small M than awq_linear_ws), and bf16 activations
 * on the GEMM path, which need a per-row factor in scratch memory, return
 * AWQ_ERR_WORKSPACE (use awq_linear_ws or awq_linear_ex with a workspace).
 * Requirements: M, N >= 0, K > 0, K % g == 0.  M == 0 or N == 0 is a no-op.
 */
awq_status awq_linear(const void *X, int32_t x_dtype, const uint32_t *qweight,
                      const uint16_t *scales, const uint8_t *zeros, int64_t M,
                      int64_t N, int64_t K, awq_config cfg, void *Y,
                      int32_t y_dtype, awq_stream_t stream);

/*
 * awq_linear_ex - awq_linear with an explicit kernel choice (AWQ_KERNEL_*)
 * and an optional workspace, so the GEMV and GEMM paths can be compared on
 * the same call (the pages quote GEMV as faster than GEMM at batch size 1:
 * "WQLinear Kernel Variants").
 *
 *   kernel     AWQ_KERNEL_AUTO (awq_linear's choice), AWQ_KERNEL_GEMV
 *            (requires M <= AWQ_GEMV_MAX_M, else AWQ_ERR_INVALID_ARG),
 *            AWQ_KERNEL_BATCHED (requires M <= AWQ_BATCHED_MAX_M, else
 *            AWQ_ERR_INVALID_ARG; it splits K into ranges of at most
 *            2048 / (g * ceil(M / 16)) groups, more when that leaves CUs
 *            idle, and its fp32 partials need the workspace: without one,
 *            a layer of more than one range returns AWQ_ERR_WORKSPACE) or
 *            AWQ_KERNEL_GEMM.
 *   workspace  device, 256-byte aligned, at least
 *            awq_linear_workspace_size(M, N, K, cfg, x_dtype, kernel) bytes,
 *            or NULL for awq_linear's scratch-free behaviour.  Scratch only:
 *            its contents on entry are ignored and on return unspecified.
 *            Calls that share a workspace must not overlap in time.
 * Allocation: none.  Errors: AWQ_ERR_WORKSPACE when workspace_bytes is too
 * small; otherwise as awq_linear.
 */
awq_status awq_linear_ex(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M,
                         int64_t N, int64_t K, awq_config cfg, void *Y,
                         int32_t y_dtype, int32_t kernel, void *workspace,
                         size_t workspace_bytes, awq_stream_t stream);

/*
 * awq_linear_workspace_size - bytes of device workspace the GEMM path needs
 * for this shape, activation type and kernel choice: fp32 partial tiles when
 * the output tiles alone cannot fill the GPU (K is then split across
 * workgroups and a second kernel sums the parts in a fixed order), and for
 * bf16 activations a factor per row (and, for shapes large enough for the
 * 256-row tile, an fp16 copy of X, M * K * 2 bytes).  The batched-decode
 * kernel needs splits * M * N * 4 bytes of fp32 partials when it splits K.
 * 0 when the call needs none (the GEMV, or an fp16 GEMM that fills the GPU
 * unsplit), and 0 on invalid arguments.
 */
size_t awq_linear_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                 int32_t x_dtype, int32_t kernel);

/*
 * awq_linear_ws - awq_linear (automatic kernel choice) with a caller-owned
 * workspace: awq_linear_ex(..., AWQ_KERNEL_AUTO, workspace, workspace_bytes,
 * stream).  Allocates nothing.
 * Cites: as awq_linear.
 *   workspace  device, at least awq_linear_workspace_size(M, N, K, cfg,
 *            x_dtype, AWQ_KERNEL_AUTO) bytes, 256-byte aligned; may be NULL
 *            when that size is 0.  Scratch as for awq_linear_ex.
 */
awq_status awq_linear_ws(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, void *workspace,
                         size_t workspace_bytes, awq_stream_t stream);

/* One projection of awq_linear_fused: packed weights for [N][K] (as from
 * awq_quantize_pack) and its output Y [M][N]. */
typedef struct awq_linear_part {
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint8_t *zeros;
    int64_t N;
    void *Y;
} awq_linear_part;

#define AWQ_MAX_PARTS 4

/* Epilogues of awq_linear_fused (int32_t in signatures). */
enum { AWQ_EPILOGUE_NONE = 0, AWQ_EPILOGUE_SILU_MUL = 1 };

/*
 * awq_linear_fused_workspace_size - bytes of device workspace awq_linear_fused
 * needs for these parts (their qweight/scales/zeros/Y may be NULL here), M,
 * K, activation type, epilogue and kernel choice; 0 when none is needed
 * (the GEMV path) and on invalid arguments.
 */
size_t awq_linear_fused_workspace_size(const awq_linear_part *parts, int32_t n_parts, int64_t M,
                                       int64_t K, awq_config cfg, int32_t x_dtype,
                                       int32_t epilogue, int32_t kernel);

/*
 * awq_linear_fused - several W4A16 projections of one input X.
 * Cites: "AWQ Advanced Usage Guide", "Layer Fusion", "What Gets Fused"
 * (attention: Q, K and V projections combined; MLP: gate and up projections
 * fused).
 *
 *   X        device, [M][K] of x_dtype, 16-byte aligned; shared by all parts.
 *   parts    host array of n_parts (1..AWQ_MAX_PARTS) projections of the
 *            same K, group size and zero-point mode.
 *   epilogue AWQ_EPILOGUE_NONE: parts[i].Y = X * deq(W_i)^T for every part.
 *            AWQ_EPILOGUE_SILU_MUL: two parts of equal N (gate, up) and
 *            H = silu(X * deq(W_0)^T) * (X * deq(W_1)^T), silu(x) = x / (1 +
 *            e^-x), computed in fp32 and rounded once; parts[i].Y are ignored.
 *   H        device [M][N] of y_dtype (SILU_MUL only; else ignored).
 *   kernel   AWQ_KERNEL_AUTO, _GEMV or _GEMM, as in awq_linear_ex; the
 *            choice uses the parts' total N.
 *   workspace  device, 256-byte aligned, at least
 *            awq_linear_fused_workspace_size() bytes (NULL when that is 0).
 * The GEMV path serves every part in one launch: each workgroup serves 16
 * columns of one part (with SILU_MUL, the same 16 columns of gate and up,
 * combined in its epilogue), so X is staged once per workgroup and no
 * intermediate reaches memory.  The GEMM path (large M, where each
 * projection fills the GPU by itself) runs the layer kernel once per part; with
 * SILU_MUL gate and up go to fp32 in the workspace and an elementwise kernel
 * writes H.  Arithmetic, requirements and errors per part as awq_linear_ex.
 */
awq_status awq_linear_fused(const void *X, int32_t x_dtype, const awq_linear_part *parts,
                            int32_t n_parts, int64_t M, int64_t K, awq_config cfg,
                            int32_t epilogue, void *H, int32_t y_dtype, int32_t kernel,
                            void *workspace, size_t workspace_bytes, awq_stream_t stream);

/* Bytes of device scratch behind awq_linear_noalloc, per GPU: the largest
 * split-K partials of a plan (256 tiles of 128 x 256 fp32, 32 MiB) plus 1 MiB
 * of per-row factors for bf16 activations. */
#define AWQ_NOALLOC_SCRATCH_BYTES ((size_t)33 << 20)

/*
 * awq_linear_noalloc - awq_linear_ws without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP-graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The GEMM's scratch is a static device array of
 * AWQ_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends.  Same kernel choice and results as awq_linear_ws (bf16
 * activations never take the 256-row tile here, which needs an fp16 copy
 * of X; the 128-row tile computes the same values).
 * Errors: AWQ_ERR_WORKSPACE when the call needs more scratch than the
 * static array holds (only bf16 activations on the GEMM path with more than
 * about 8.6 million rows, 4 bytes each); otherwise as awq_linear.
 * Concurrency: every call on a GPU shares that GPU's array.  Calls on one
 * GPU that may overlap in time (different streams, or concurrent graph
 * replays) race on it and must not be made; calls ordered on one stream are
 * safe.  The array carries nothing from one call to the next (each call
 * writes every scratch element it reads), so it needs no clearing.
 */
awq_status awq_linear_noalloc(const void *X, int32_t x_dtype, const uint32_t *qweight,
                              const uint16_t *scales, const uint8_t *zeros, int64_t M,
                              int64_t N, int64_t K, awq_config cfg, void *Y,
                              int32_t y_dtype, awq_stream_t stream);

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

/* Options of awq_scale_search_ex, mirroring the pages' calibration
 * parameters ("AWQ Advanced Usage Guide", "Calibration Parameters"):
 *  duo_scaling  1: candidate t_k = xbar_k^alpha / wbar_k^(1 - alpha), wbar_k
 *               the mean |W_nk| over the N rows (exact sum, rounded once;
 *               N < 2^24), both floored at 2^-24 ("Scale weights and
 *               activations"); 0: t_k = xbar_k^alpha.
 *  apply_clip   1: after the alpha search, each (row, group) of the chosen
 *               scaling takes the range shrink factor c_i = 1 - i/40, i =
 *               0..19 (rounded to fp32: the group's [lo, hi], or +-max|v|,
 *               times c) that minimizes the group's output error
 *               ||A_g (v - deq_c(v))||^2, A = fp16(X / s), v = fp32(s * W),
 *               evaluated in fp64 through A_g^T A_g; the first minimum wins
 *               ("Apply weight clipping").  The packed result is that of the
 *               chosen factors; the losses stay those of the unclipped
 *               candidates.  K/g must not exceed 65535 (else
 *               AWQ_ERR_UNSUPPORTED). */
typedef struct awq_search_options {
    int32_t duo_scaling;
    int32_t apply_clip;
} awq_search_options;

/* awq_scale_search_workspace_size for awq_scale_search_ex with `opts` (NULL:
 * both options off). */
size_t awq_scale_search_workspace_size_ex(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                          int32_t n_alpha, const awq_search_options *opts);

/*
 * awq_scale_search_ex - awq_scale_search with the calibration options above.
 * Cites: as awq_scale_search, and "Calibration Parameters" (duo_scaling,
 * apply_clip).
 *   opts        host, or NULL (both off: exactly awq_scale_search).
 *   clip_index  device u8 [N][K/g] or NULL: with apply_clip, the chosen
 *               shrink index of every (row, group).
 * Everything else as awq_scale_search.
 */
awq_status awq_scale_search_ex(const void *X, const void *W, int64_t M, int64_t N, int64_t K,
                               awq_config cfg, const double *alphas, int32_t n_alpha,
                               const awq_search_options *opts, void *workspace,
                               size_t workspace_bytes, int32_t *best_index, double *losses,
                               float *best_s, uint32_t *qweight, uint16_t *scales,
                               uint8_t *zeros, uint8_t *clip_index, awq_stream_t stream);

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
