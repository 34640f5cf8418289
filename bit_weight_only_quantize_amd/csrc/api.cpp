// C ABI of libawq355.so: argument validation, kernel dispatch and the
// orchestration of the alpha-grid scale search.  Every check runs before any
// HIP call, so invalid arguments are reported on machines without a GPU too.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <mutex>

#include "../../include/awq355.h"
#include "awq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

awq_status fail(awq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

awq_status ok() {
  g_last_error[0] = '\0';
  return AWQ_OK;
}

awq_status hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return ok();
  return fail(AWQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Automatic kernel choice, from measured times (fp16, graph replays) on 7B-
// and 13B-class layers: the GEMV wins wherever it stages the activation rows
// in LDS; unstaged, its activation reads grow with M, and it loses to the
// split-K GEMM where each wave walks a long chain of groups (> 8), beyond
// M = 8, or beyond M = 12 on layers of at most 5e7 weights (at M = 16: 28.7
// vs 22.0 us for 13824 x 5120).
bool auto_gemv(int64_t M, int64_t N, int64_t K, int g) {
  if (M > AWQ_GEMV_MAX_M || !awq::gemv_supported(M, N, K, g)) return false;
  if (awq::gemv_stages_activations(M, N, K)) return true;
  if (awq::gemv_groups_per_wave(N, K, g) > 8) return false;
  return M <= 8 || (M <= 12 && N * K <= 50000000);
}

// Automatic choice of the batched-decode kernel (with scratch for its
// partials), for 2 <= M <= 32 on layers of at least 1.6e7 weights and 4096
// columns, except where the GEMV stages the activation rows and either
// M < 8 or the layer has under 2e7 weights (4096 x 4096, whose GEMV stages
// up to 16 rows in 16-wave workgroups).  Same-box graph replays (us; GEMV /
// batched / GEMM, g = 128 unless noted, N x K):
//   11008 x 4096   M = 6: 10.0 / 10.8 / 16.1   M = 8: 12.7 / 11.1 / 16.0
//                  M = 16: 17.7 / 11.5 / 16.5  M = 32: - / 15.3 / 17.9
//   4096 x 11008   M = 4: 9.2 / 10.8 / 17.3    M = 6: 12.1 / 11.0 / 17.4
//                  M = 16: 17.9 / 11.6 / 18.2  M = 32: - / 16.1 / 18.7
//   13824 x 5120   M = 6: 15.7 / 15.5 / 20.3   M = 8: 20.9 / 15.7 / 20.4
//                  M = 32: - / 19.6 / 21.7; g = 64, M = 32: - / 23.5 / 29.0
//   5120 x 13824   M = 4: 22.0 / 15.3 / 21.0   M = 16: 34.3 / 16.1 / 21.5
//   4096 x 4096    M = 16: 7.9 / 8.8 / 12.7    M = 24: - / 9.5 / 13.3
// At M = 64 the GEMM is faster (its splits need fewer workgroups).
bool auto_batched(int64_t M, int64_t N, int64_t K, int g) {
  if (M < 2 || M > 32 || N < 4096 || N * K < 16000000) return false;
  if (!awq::batched_gemv_supported(M, N, K, g)) return false;
  const bool staged = M <= AWQ_GEMV_MAX_M && awq::gemv_supported(M, N, K, g) &&
                      awq::gemv_stages_activations(M, N, K);
  return !(staged && (M < 8 || N * K < 20000000));
}

awq_status check_config(awq_config cfg, int64_t K) {
  if (cfg.w_bit != 4) return fail(AWQ_ERR_UNSUPPORTED, "w_bit=%d: only 4 is supported", cfg.w_bit);
  if (cfg.zero_point != 0 && cfg.zero_point != 1)
    return fail(AWQ_ERR_INVALID_ARG, "zero_point=%d: must be 1 (asymmetric) or 0 (symmetric)",
                cfg.zero_point);
  if (cfg.group_size != 64 && cfg.group_size != 128)
    return fail(AWQ_ERR_UNSUPPORTED, "group_size=%d: supported values are 64 and 128",
                cfg.group_size);
  if (K <= 0) return fail(AWQ_ERR_INVALID_ARG, "K=%lld must be positive", (long long)K);
  if (K % cfg.group_size != 0)
    return fail(AWQ_ERR_INVALID_ARG, "K=%lld is not a multiple of group_size=%d", (long long)K,
                cfg.group_size);
  if (K > (int64_t)1 << 30) return fail(AWQ_ERR_INVALID_ARG, "K=%lld is too large", (long long)K);
  return AWQ_OK;
}

hipStream_t as_stream(awq_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

awq_status check_linear(const void *X, int32_t x_dtype, const uint32_t *qweight,
                        const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                        int64_t K, awq_config cfg, const void *Y, int32_t y_dtype,
                        int32_t kernel) {
  awq_status st = check_config(cfg, K);
  if (st != AWQ_OK) return st;
  if (M < 0 || N < 0) return fail(AWQ_ERR_INVALID_ARG, "negative M or N");
  if (M > ((int64_t)1 << 31) || N > ((int64_t)1 << 31))
    return fail(AWQ_ERR_INVALID_ARG, "M or N too large");
  if (x_dtype != AWQ_F16 && x_dtype != AWQ_BF16)
    return fail(AWQ_ERR_INVALID_ARG, "x_dtype=%d: must be AWQ_F16 or AWQ_BF16", x_dtype);
  if (y_dtype != AWQ_F16 && y_dtype != AWQ_BF16 && y_dtype != AWQ_F32)
    return fail(AWQ_ERR_INVALID_ARG, "y_dtype=%d: must be AWQ_F16, AWQ_BF16 or AWQ_F32",
                y_dtype);
  if (kernel != AWQ_KERNEL_AUTO && kernel != AWQ_KERNEL_GEMV && kernel != AWQ_KERNEL_GEMM &&
      kernel != AWQ_KERNEL_BATCHED)
    return fail(AWQ_ERR_INVALID_ARG, "kernel=%d: unknown kernel selector", kernel);
  if (kernel == AWQ_KERNEL_GEMV && M > AWQ_GEMV_MAX_M)
    return fail(AWQ_ERR_INVALID_ARG, "GEMV kernel serves M <= %d, got M=%lld", AWQ_GEMV_MAX_M,
                (long long)M);
  if (kernel == AWQ_KERNEL_BATCHED && M > AWQ_BATCHED_MAX_M)
    return fail(AWQ_ERR_INVALID_ARG, "batched kernel serves M <= %d, got M=%lld",
                AWQ_BATCHED_MAX_M, (long long)M);
  if (M == 0 || N == 0) return AWQ_OK;
  if (!awq::gemm_supported(N, K, false))
    return fail(AWQ_ERR_UNSUPPORTED, "layer of %lld x %lld exceeds 2 GiB of packed weights",
                (long long)N, (long long)K);
  if (!X || !qweight || !scales || (cfg.zero_point && !zeros) || !Y)
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(X, 16) || !aligned(qweight, 16))
    return fail(AWQ_ERR_INVALID_ARG, "X and qweight must be 16-byte aligned");
  if (!aligned(Y, y_dtype == AWQ_F32 ? 4 : 2))
    return fail(AWQ_ERR_INVALID_ARG, "Y is not aligned to its element size");
  if (!aligned(scales, 2)) return fail(AWQ_ERR_INVALID_ARG, "scales must be 2-byte aligned");
  return AWQ_OK;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layout of the scale search (each region 256-byte aligned; the
// duo-scaling and clipping regions only when those options are on).
struct SearchLayout {
  size_t units, xbar, table, act, qw, sc, zr, yref, partials, losses, best;
  size_t wunits, wbar, gram_partial, gram, total;
  int64_t tiles;
};

SearchLayout search_layout(int64_t M, int64_t N, int64_t K, int gs, int n_alpha, bool duo,
                           bool clip) {
  SearchLayout L{};
  const int64_t G = K / gs;
  L.tiles = awq::gemm_tile_count(M, N);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes);
    return at;
  };
  L.units = take(sizeof(uint64_t) * K);
  L.xbar = take(sizeof(double) * K);
  L.table = take(sizeof(float) * (size_t)n_alpha * K);
  L.act = take(sizeof(uint16_t) * (size_t)M * K);
  L.qw = take(sizeof(uint32_t) * (size_t)N * (K / 8));
  L.sc = take(sizeof(uint16_t) * (size_t)N * G);
  L.zr = take(sizeof(uint8_t) * (size_t)N * G);
  L.yref = take(sizeof(float) * (size_t)M * N);
  L.partials = take(sizeof(double) * (size_t)n_alpha * L.tiles);
  L.losses = take(sizeof(double) * 64);
  L.best = take(sizeof(int32_t));
  if (duo) {
    L.wunits = take(sizeof(uint64_t) * K);
    L.wbar = take(sizeof(double) * K);
  }
  if (clip) {
    L.gram_partial = take(sizeof(double) * (size_t)G * awq::gram_parts(M) * gs * gs);
    L.gram = take(sizeof(double) * (size_t)G * awq::clip_gram_doubles(gs));
  }
  L.total = off;
  return L;
}

awq_status check_search(int64_t M, int64_t N, int64_t K, awq_config cfg, int32_t n_alpha,
                        const awq_search_options *opts = nullptr) {
  awq_status st = check_config(cfg, K);
  if (st != AWQ_OK) return st;
  if (M < 1 || N < 1) return fail(AWQ_ERR_INVALID_ARG, "M and N must be >= 1");
  if (M > ((int64_t)1 << 24) - 1)
    return fail(AWQ_ERR_INVALID_ARG, "M=%lld exceeds 2^24-1 calibration rows", (long long)M);
  if (opts && (opts->duo_scaling != 0 && opts->duo_scaling != 1))
    return fail(AWQ_ERR_INVALID_ARG, "duo_scaling=%d: must be 0 or 1", opts->duo_scaling);
  if (opts && (opts->apply_clip != 0 && opts->apply_clip != 1))
    return fail(AWQ_ERR_INVALID_ARG, "apply_clip=%d: must be 0 or 1", opts->apply_clip);
  if (opts && opts->duo_scaling && N > ((int64_t)1 << 24) - 1)
    return fail(AWQ_ERR_INVALID_ARG, "duo scaling: N=%lld exceeds 2^24-1 rows", (long long)N);
  if (N > ((int64_t)1 << 31)) return fail(AWQ_ERR_INVALID_ARG, "N too large");
  if (opts && opts->apply_clip && K / cfg.group_size > 65535)
    return fail(AWQ_ERR_UNSUPPORTED, "weight clipping: K/g=%lld exceeds 65535 groups",
                (long long)(K / cfg.group_size));
  if (n_alpha < 1 || n_alpha > 64)
    return fail(AWQ_ERR_INVALID_ARG, "n_alpha=%d must be in [1, 64]", n_alpha);
  if (!awq::gemm_supported(N, K, true))
    return fail(AWQ_ERR_UNSUPPORTED, "search layer of %lld x %lld exceeds 2 GiB of fp16 weights",
                (long long)N, (long long)K);
  return AWQ_OK;
}

}  // namespace

extern "C" {

const char *awq_status_string(awq_status status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_INVALID_ARG: return "AWQ_ERR_INVALID_ARG: invalid argument";
    case AWQ_ERR_UNSUPPORTED: return "AWQ_ERR_UNSUPPORTED: configuration not supported";
    case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE: workspace too small";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP: HIP runtime error";
    case AWQ_ERR_NONFINITE: return "AWQ_ERR_NONFINITE: non-finite input";
  }
  return "unknown awq_status";
}

const char *awq_last_error(void) { return g_last_error; }

const char *awq_version(void) { return "awq355 0.1 (gfx950)"; }

awq_status awq_quantize_pack(const void *W, int64_t N, int64_t K, awq_config cfg, const float *s,
                             uint32_t *qweight, uint16_t *scales, uint8_t *zeros,
                             int32_t *nonfinite_count, awq_stream_t stream) {
  awq_status st = check_config(cfg, K);
  if (st != AWQ_OK) return st;
  if (N < 0) return fail(AWQ_ERR_INVALID_ARG, "N=%lld is negative", (long long)N);
  if (N > ((int64_t)1 << 31)) return fail(AWQ_ERR_INVALID_ARG, "N too large");
  if (N == 0) return ok();
  if (!W || !qweight || !scales || (cfg.zero_point && !zeros))
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(W, 16) || !aligned(qweight, 16))
    return fail(AWQ_ERR_INVALID_ARG, "W and qweight must be 16-byte aligned");
  if (s && !aligned(s, 16)) return fail(AWQ_ERR_INVALID_ARG, "s must be 16-byte aligned");
  if (!aligned(scales, 2)) return fail(AWQ_ERR_INVALID_ARG, "scales must be 2-byte aligned");
  if (nonfinite_count && !aligned(nonfinite_count, 4))
    return fail(AWQ_ERR_INVALID_ARG, "nonfinite_count must be 4-byte aligned");
  return hip_status(awq::launch_quantize_pack(reinterpret_cast<const uint16_t *>(W), N, K,
                                              cfg.group_size, s, qweight, scales,
                                              cfg.zero_point ? zeros : nullptr,
                                              nonfinite_count, as_stream(stream)),
                    "awq_quantize_pack");
}

awq_status awq_dequantize(const uint32_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, awq_config cfg, void *out, int32_t out_dtype,
                          awq_stream_t stream) {
  awq_status st = check_config(cfg, K);
  if (st != AWQ_OK) return st;
  if (N < 0) return fail(AWQ_ERR_INVALID_ARG, "N=%lld is negative", (long long)N);
  if (N > ((int64_t)1 << 31)) return fail(AWQ_ERR_INVALID_ARG, "N too large");
  if (out_dtype != AWQ_F16 && out_dtype != AWQ_F32)
    return fail(AWQ_ERR_INVALID_ARG, "out_dtype=%d: must be AWQ_F16 or AWQ_F32", out_dtype);
  if (N == 0) return ok();
  if (!qweight || !scales || (cfg.zero_point && !zeros) || !out)
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(out, 16) || !aligned(qweight, 4) || !aligned(scales, 2))
    return fail(AWQ_ERR_INVALID_ARG, "out must be 16-byte aligned, qweight 4, scales 2");
  return hip_status(awq::launch_dequantize(qweight, scales, cfg.zero_point ? zeros : nullptr, N, K,
                                           cfg.group_size, out, out_dtype == AWQ_F32,
                                           as_stream(stream)),
                    "awq_dequantize");
}

namespace {

// Whether the automatic choice (or the explicit `kernel`) runs the batched-
// decode kernel.  The automatic choice takes it only with scratch for its
// split-K partials (awq_linear, which has none, never splits K).
bool runs_batched(int64_t M, int64_t N, int64_t K, int gs, int32_t kernel, bool has_scratch) {
  if (kernel == AWQ_KERNEL_BATCHED) return true;
  return kernel == AWQ_KERNEL_AUTO && has_scratch && auto_batched(M, N, K, gs);
}

// Whether it runs the GEMV (the batched kernel, when chosen, comes first).
bool runs_gemv(int64_t M, int64_t N, int64_t K, int gs, int32_t kernel, bool has_scratch) {
  if (kernel == AWQ_KERNEL_GEMV) return true;
  return kernel == AWQ_KERNEL_AUTO && !runs_batched(M, N, K, gs, kernel, has_scratch) &&
         auto_gemv(M, N, K, gs);
}

// The linear layer with the GEMM's scratch from the caller's workspace, or
// (workspace == NULL) with a scratch-free plan.
awq_status linear_impl(const char *who, const void *X, int32_t x_dtype, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, awq_config cfg, void *Y, int32_t y_dtype, int32_t kernel,
                       void *workspace, size_t workspace_bytes, awq_stream_t stream) {
  awq_status st =
      check_linear(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype, kernel);
  if (st != AWQ_OK) return st;
  if (kernel == AWQ_KERNEL_GEMV && !awq::gemv_supported(M, N > 0 ? N : 1, K, cfg.group_size))
    return fail(AWQ_ERR_UNSUPPORTED, "%s: the GEMV kernel cannot serve K=%lld", who,
                (long long)K);
  if (workspace && !aligned(workspace, kAlign))
    return fail(AWQ_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", who);
  if (M == 0 || N == 0) return ok();
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  const awq::YType yt = y_dtype == AWQ_F16    ? awq::YType::F16
                        : y_dtype == AWQ_BF16 ? awq::YType::BF16
                                              : awq::YType::F32;
  const hipStream_t hs = as_stream(stream);
  if (runs_gemv(M, N, K, cfg.group_size, kernel, workspace != nullptr))
    return hip_status(awq::launch_gemv(X, xt, qweight, scales, cfg.zero_point ? zeros : nullptr, M, N, K, cfg.group_size, Y,
                                       yt, hs),
                      who);
  if (runs_batched(M, N, K, cfg.group_size, kernel, workspace != nullptr)) {
    const awq::BatchedPlan bp = awq::batched_gemv_plan(
        M, N, K, cfg.group_size, workspace ? awq::Scratch::Full : awq::Scratch::None);
    if (bp.partial_bytes > 0 && !workspace)
      return fail(AWQ_ERR_WORKSPACE,
                  "%s: the batched kernel splits this K and needs a workspace of %zu bytes "
                  "(awq_linear_workspace_size)",
                  who, bp.partial_bytes);
    if (bp.partial_bytes > workspace_bytes)
      return fail(AWQ_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                  workspace_bytes, bp.partial_bytes);
    return hip_status(awq::launch_batched_gemv(X, xt, qweight, scales,
                                               cfg.zero_point ? zeros : nullptr, M, N, K,
                                               cfg.group_size, Y, yt, bp, workspace, hs),
                      who);
  }
  const awq::GemmPlan plan =
      awq::gemm_plan(M, N, K, xt, workspace ? awq::Scratch::Full : awq::Scratch::None);
  if (plan.workspace_bytes > 0) {
    if (!workspace)
      return fail(AWQ_ERR_WORKSPACE,
                  "%s: bf16 activations on the GEMM path need a workspace of %zu bytes "
                  "(awq_linear_workspace_size)",
                  who, plan.workspace_bytes);
    if (workspace_bytes < plan.workspace_bytes)
      return fail(AWQ_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                  workspace_bytes, plan.workspace_bytes);
  }
  return hip_status(awq::launch_gemm(X, xt, qweight, scales, cfg.zero_point ? zeros : nullptr, M, N, K, cfg.group_size, Y,
                                     yt, plan, workspace, hs),
                    who);
}

}  // namespace

awq_status awq_linear_ex(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, int32_t kernel,
                         void *workspace, size_t workspace_bytes, awq_stream_t stream) {
  return linear_impl("awq_linear_ex", X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y,
                     y_dtype, kernel, workspace, workspace_bytes, stream);
}

size_t awq_linear_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                 int32_t x_dtype, int32_t kernel) {
  if (check_config(cfg, K) != AWQ_OK || M < 0 || N < 0) return 0;
  if (M > ((int64_t)1 << 31) || N > ((int64_t)1 << 31)) return 0;
  if (x_dtype != AWQ_F16 && x_dtype != AWQ_BF16) return 0;
  if (kernel != AWQ_KERNEL_AUTO && kernel != AWQ_KERNEL_GEMV && kernel != AWQ_KERNEL_GEMM &&
      kernel != AWQ_KERNEL_BATCHED)
    return 0;
  if (kernel == AWQ_KERNEL_BATCHED && M > AWQ_BATCHED_MAX_M) return 0;
  if (M == 0 || N == 0 || runs_gemv(M, N, K, cfg.group_size, kernel, true)) return 0;
  if (!awq::gemm_supported(N, K, false)) return 0;
  if (runs_batched(M, N, K, cfg.group_size, kernel, true))
    return awq::batched_gemv_plan(M, N, K, cfg.group_size, awq::Scratch::Full).partial_bytes;
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  return awq::gemm_plan(M, N, K, xt, awq::Scratch::Full).workspace_bytes;
}

awq_status awq_linear_ws(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, void *workspace,
                         size_t workspace_bytes, awq_stream_t stream) {
  return linear_impl("awq_linear_ws", X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y,
                     y_dtype, AWQ_KERNEL_AUTO, workspace, workspace_bytes, stream);
}

awq_status awq_linear(const void *X, int32_t x_dtype, const uint32_t *qweight,
                      const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                      int64_t K, awq_config cfg, void *Y, int32_t y_dtype, awq_stream_t stream) {
  return linear_impl("awq_linear", X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype,
                     AWQ_KERNEL_AUTO, nullptr, 0, stream);
}

}  // extern "C"

// ---- awq_linear_fused: projections that share one input ------------------------
namespace {

// Workspace layout of a fused call on the GEMM path.
struct FusedLayout {
  bool gemv;
  size_t gemm_ws, gate_off, up_off, scratch_off, total;
};

awq_status check_fused(const void *X, int32_t x_dtype, const awq_linear_part *parts,
                       int32_t n_parts, int64_t M, int64_t K, awq_config cfg, int32_t epilogue,
                       const void *H, int32_t y_dtype, int32_t kernel, bool need_ptrs) {
  if (n_parts < 1 || n_parts > AWQ_MAX_PARTS || !parts)
    return fail(AWQ_ERR_INVALID_ARG, "n_parts=%d: must be in [1, %d]", n_parts, AWQ_MAX_PARTS);
  if (epilogue != AWQ_EPILOGUE_NONE && epilogue != AWQ_EPILOGUE_SILU_MUL)
    return fail(AWQ_ERR_INVALID_ARG, "epilogue=%d: unknown", epilogue);
  if (epilogue == AWQ_EPILOGUE_SILU_MUL && (n_parts != 2 || parts[0].N != parts[1].N))
    return fail(AWQ_ERR_INVALID_ARG, "the SiLU-mul epilogue takes 2 parts of equal N");
  if (kernel == AWQ_KERNEL_BATCHED)
    return fail(AWQ_ERR_INVALID_ARG, "fused projections take AWQ_KERNEL_AUTO, _GEMV or _GEMM");
  for (int i = 0; i < n_parts; ++i) {
    // each part is checked as a linear call of its own (the output pointer
    // is H for the SiLU-mul epilogue)
    const void *y = epilogue == AWQ_EPILOGUE_SILU_MUL ? H : parts[i].Y;
    awq_status st = check_linear(need_ptrs ? X : (const void *)16, x_dtype,
                                 need_ptrs ? parts[i].qweight : (const uint32_t *)16,
                                 need_ptrs ? parts[i].scales : (const uint16_t *)16,
                                 need_ptrs ? parts[i].zeros : (const uint8_t *)16, M, parts[i].N, K,
                                 cfg, need_ptrs ? y : (const void *)16, y_dtype, kernel);
    if (st != AWQ_OK) return st;
  }
  return AWQ_OK;
}

// Whether a part of a fused call that does not run the GEMV runs the
// batched-decode kernel (the automatic choice with scratch) or the GEMM.
bool fused_part_batched(int64_t M, int64_t N, int64_t K, int gs, int32_t kernel) {
  return kernel == AWQ_KERNEL_AUTO && auto_batched(M, N, K, gs);
}

FusedLayout fused_layout(const awq_linear_part *parts, int32_t n_parts, int64_t M, int64_t K,
                         awq_config cfg, awq::XType xt, int32_t epilogue, int32_t kernel) {
  FusedLayout L{};
  const bool pair = epilogue == AWQ_EPILOGUE_SILU_MUL;
  int64_t ntot = 0, nmax = 0, tiles = 0;
  for (int i = 0; i < n_parts; ++i) {
    ntot += parts[i].N;
    nmax = parts[i].N > nmax ? parts[i].N : nmax;
    if (!pair || i == 0) tiles += (parts[i].N + 15) / 16;   // the GEMV's workgroups
  }
  L.gemv = M > 0 && ntot > 0 && kernel != AWQ_KERNEL_GEMM &&
           awq::gemv_supported(M, 16 * tiles, K, cfg.group_size, pair ? 2 : 1) &&
           (kernel == AWQ_KERNEL_GEMV || auto_gemv(M, ntot, K, cfg.group_size));
  if (L.gemv || M == 0 || ntot == 0) return L;
  for (int i = 0; i < n_parts; ++i) {
    if (parts[i].N == 0) continue;
    // each part on its own: the batched-decode kernel where the automatic
    // choice takes it, else the GEMM; the parts run in turn and share scratch
    const size_t b =
        fused_part_batched(M, parts[i].N, K, cfg.group_size, kernel)
            ? awq::batched_gemv_plan(M, parts[i].N, K, cfg.group_size, awq::Scratch::Full).partial_bytes
            : awq::gemm_plan(M, parts[i].N, K, xt, awq::Scratch::Full).workspace_bytes;
    L.gemm_ws = b > L.gemm_ws ? b : L.gemm_ws;
  }
  if (pair) {
    L.gate_off = 0;
    L.up_off = round_up(sizeof(float) * (size_t)M * nmax);
    L.scratch_off = L.up_off + round_up(sizeof(float) * (size_t)M * nmax);
  }
  L.total = L.scratch_off + L.gemm_ws;
  return L;
}

}  // namespace

extern "C" {

size_t awq_linear_fused_workspace_size(const awq_linear_part *parts, int32_t n_parts, int64_t M,
                                       int64_t K, awq_config cfg, int32_t x_dtype,
                                       int32_t epilogue, int32_t kernel) {
  if (check_fused(nullptr, x_dtype, parts, n_parts, M, K, cfg, epilogue, nullptr, AWQ_F32, kernel,
                  false) != AWQ_OK)
    return 0;
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  return fused_layout(parts, n_parts, M, K, cfg, xt, epilogue, kernel).total;
}

awq_status awq_linear_fused(const void *X, int32_t x_dtype, const awq_linear_part *parts,
                            int32_t n_parts, int64_t M, int64_t K, awq_config cfg,
                            int32_t epilogue, void *H, int32_t y_dtype, int32_t kernel,
                            void *workspace, size_t workspace_bytes, awq_stream_t stream) {
  const char *who = "awq_linear_fused";
  awq_status st =
      check_fused(X, x_dtype, parts, n_parts, M, K, cfg, epilogue, H, y_dtype, kernel, true);
  if (st != AWQ_OK) return st;
  if (workspace && !aligned(workspace, kAlign))
    return fail(AWQ_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", who);
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  const awq::YType yt = y_dtype == AWQ_F16    ? awq::YType::F16
                        : y_dtype == AWQ_BF16 ? awq::YType::BF16
                                              : awq::YType::F32;
  const FusedLayout L = fused_layout(parts, n_parts, M, K, cfg, xt, epilogue, kernel);
  if (kernel == AWQ_KERNEL_GEMV && M > 0 && !L.gemv)
    return fail(AWQ_ERR_UNSUPPORTED, "%s: the GEMV kernel cannot serve these parts", who);
  if (L.total > 0 && (!workspace || workspace_bytes < L.total))
    return fail(AWQ_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed "
                "(awq_linear_fused_workspace_size)", who, workspace ? workspace_bytes : 0, L.total);
  if (M == 0) return ok();
  const bool pair = epilogue == AWQ_EPILOGUE_SILU_MUL;
  awq::LinearPart lp[AWQ_MAX_PARTS];
  for (int i = 0; i < n_parts; ++i)
    lp[i] = awq::LinearPart{parts[i].qweight, parts[i].scales,
                            cfg.zero_point ? parts[i].zeros : nullptr, parts[i].N,
                            pair ? H : parts[i].Y};
  const hipStream_t hs = as_stream(stream);
  if (L.gemv)
    return hip_status(awq::launch_gemv_parts(X, xt, lp, n_parts, pair, M, K, cfg.group_size, yt, hs),
                      who);
  char *ws = reinterpret_cast<char *>(workspace);
  void *scratch = L.gemm_ws ? ws + L.scratch_off : nullptr;
  hipError_t e = hipSuccess;
  for (int i = 0; i < n_parts && e == hipSuccess; ++i) {
    if (lp[i].N == 0) continue;
    void *y = pair ? (void *)(ws + (i == 0 ? L.gate_off : L.up_off)) : lp[i].Y;
    const awq::YType pyt = pair ? awq::YType::F32 : yt;
    if (fused_part_batched(M, lp[i].N, K, cfg.group_size, kernel)) {
      const awq::BatchedPlan bp =
          awq::batched_gemv_plan(M, lp[i].N, K, cfg.group_size, awq::Scratch::Full);
      e = awq::launch_batched_gemv(X, xt, lp[i].qweight, lp[i].scales, lp[i].zeros, M, lp[i].N,
                                   K, cfg.group_size, y, pyt, bp, scratch, hs);
      continue;
    }
    const awq::GemmPlan plan = awq::gemm_plan(M, lp[i].N, K, xt, awq::Scratch::Full);
    e = awq::launch_gemm(X, xt, lp[i].qweight, lp[i].scales, lp[i].zeros, M, lp[i].N, K,
                         cfg.group_size, y, pyt, plan, scratch, hs);
  }
  if (e == hipSuccess && pair)
    e = awq::launch_silu_mul(reinterpret_cast<const float *>(ws + L.gate_off),
                             reinterpret_cast<const float *>(ws + L.up_off), M * parts[0].N, H,
                             yt, hs);
  return hip_status(e, who);
}

}  // extern "C"

// ---- awq_linear_noalloc: the GEMM's scratch in a static device array -----------
namespace {

// The GEMM scratch of awq_linear_noalloc: split-K partials (at most
// kBoundedPartialBytes) and, for bf16 activations, one fp32 factor per row.
// One copy per GPU, in the library's code object; it lives until the process
// ends.  Host code must never pass `scratch` itself to a kernel (in host code
// the name is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = AWQ_NOALLOC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes >= awq::kBoundedPartialBytes + 256, "scratch too small");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
awq_status static_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "awq_linear_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(AWQ_ERR_UNSUPPORTED, "awq_linear_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "awq_linear_noalloc (hipGetSymbolAddress)");
    if (!p) return fail(AWQ_ERR_HIP, "awq_linear_noalloc: no device address for the scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}

}  // namespace

extern "C" {

awq_status awq_linear_noalloc(const void *X, int32_t x_dtype, const uint32_t *qweight,
                              const uint16_t *scales, const uint8_t *zeros, int64_t M,
                              int64_t N, int64_t K, awq_config cfg, void *Y, int32_t y_dtype,
                              awq_stream_t stream) {
  const char *who = "awq_linear_noalloc";
  awq_status st = check_linear(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype,
                               AWQ_KERNEL_AUTO);
  if (st != AWQ_OK) return st;
  if (M == 0 || N == 0) return ok();
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  const awq::YType yt = y_dtype == AWQ_F16    ? awq::YType::F16
                        : y_dtype == AWQ_BF16 ? awq::YType::BF16
                                              : awq::YType::F32;
  const hipStream_t hs = as_stream(stream);
  if (runs_gemv(M, N, K, cfg.group_size, AWQ_KERNEL_AUTO, true))
    return hip_status(awq::launch_gemv(X, xt, qweight, scales, cfg.zero_point ? zeros : nullptr, M, N, K, cfg.group_size, Y,
                                       yt, hs),
                      who);
  if (runs_batched(M, N, K, cfg.group_size, AWQ_KERNEL_AUTO, true)) {
    const awq::BatchedPlan bp =
        awq::batched_gemv_plan(M, N, K, cfg.group_size, awq::Scratch::Bounded);
    void *ws = nullptr;
    if (bp.partial_bytes > 0) {
      st = static_scratch(&ws);
      if (st != AWQ_OK) return st;
    }
    return hip_status(awq::launch_batched_gemv(X, xt, qweight, scales,
                                               cfg.zero_point ? zeros : nullptr, M, N, K,
                                               cfg.group_size, Y, yt, bp, ws, hs),
                      who);
  }
  const awq::GemmPlan plan = awq::gemm_plan(M, N, K, xt, awq::Scratch::Bounded);
  if (plan.workspace_bytes > kStaticScratchBytes)
    return fail(AWQ_ERR_WORKSPACE,
                "%s: this call needs %zu bytes of scratch, beyond the static %zu (bf16 "
                "activations need one fp32 factor per row)",
                who, plan.workspace_bytes, kStaticScratchBytes);
  void *ws = nullptr;
  if (plan.workspace_bytes > 0) {
    st = static_scratch(&ws);
    if (st != AWQ_OK) return st;
  }
  return hip_status(awq::launch_gemm(X, xt, qweight, scales, cfg.zero_point ? zeros : nullptr, M, N, K, cfg.group_size, Y,
                                     yt, plan, ws, hs),
                    who);
}

size_t awq_scale_search_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                       int32_t n_alpha) {
  return awq_scale_search_workspace_size_ex(M, N, K, cfg, n_alpha, nullptr);
}

size_t awq_scale_search_workspace_size_ex(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                          int32_t n_alpha, const awq_search_options *opts) {
  if (check_search(M, N, K, cfg, n_alpha, opts) != AWQ_OK) return 0;
  return search_layout(M, N, K, cfg.group_size, n_alpha, opts && opts->duo_scaling,
                       opts && opts->apply_clip)
      .total;
}

awq_status awq_scale_search(const void *X, const void *W, int64_t M, int64_t N, int64_t K,
                            awq_config cfg, const double *alphas, int32_t n_alpha,
                            void *workspace, size_t workspace_bytes, int32_t *best_index,
                            double *losses, float *best_s, uint32_t *qweight,
                            uint16_t *scales, uint8_t *zeros, awq_stream_t stream) {
  return awq_scale_search_ex(X, W, M, N, K, cfg, alphas, n_alpha, nullptr, workspace,
                             workspace_bytes, best_index, losses, best_s, qweight, scales, zeros,
                             nullptr, stream);
}

awq_status awq_scale_search_ex(const void *X, const void *W, int64_t M, int64_t N, int64_t K,
                               awq_config cfg, const double *alphas, int32_t n_alpha,
                               const awq_search_options *opts, void *workspace,
                               size_t workspace_bytes, int32_t *best_index, double *losses,
                               float *best_s, uint32_t *qweight, uint16_t *scales,
                               uint8_t *zeros, uint8_t *clip_index, awq_stream_t stream) {
  awq_status st = check_search(M, N, K, cfg, n_alpha, opts);
  if (st != AWQ_OK) return st;
  const bool duo = opts && opts->duo_scaling, clip = opts && opts->apply_clip;
  double grid[64];
  if (alphas == nullptr) {
    if (n_alpha != 20)
      return fail(AWQ_ERR_INVALID_ARG, "alphas=NULL selects the 20-point grid; n_alpha=%d",
                  n_alpha);
    for (int j = 0; j < 20; ++j) grid[j] = (double)j / 20.0;
  } else {
    for (int j = 0; j < n_alpha; ++j) {
      if (!(alphas[j] >= 0.0 && alphas[j] <= 1.0))
        return fail(AWQ_ERR_INVALID_ARG, "alphas[%d] is not in [0, 1]", j);
      grid[j] = alphas[j];
    }
  }
  if (!X || !W || !workspace || !best_index || !best_s || !qweight || !scales ||
      (cfg.zero_point && !zeros))
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(qweight, 16) || !aligned(best_s, 16))
    return fail(AWQ_ERR_INVALID_ARG, "X, W, qweight and best_s must be 16-byte aligned");
  if (!aligned(workspace, kAlign))
    return fail(AWQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!aligned(scales, 2)) return fail(AWQ_ERR_INVALID_ARG, "scales must be 2-byte aligned");
  const SearchLayout L = search_layout(M, N, K, cfg.group_size, n_alpha, duo, clip);
  if (workspace_bytes < L.total)
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes,
                L.total);

  const hipStream_t s = as_stream(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  auto *units = reinterpret_cast<uint64_t *>(ws + L.units);
  auto *xbar = reinterpret_cast<double *>(ws + L.xbar);
  auto *table = reinterpret_cast<float *>(ws + L.table);
  auto *act = reinterpret_cast<uint16_t *>(ws + L.act);
  auto *qw = reinterpret_cast<uint32_t *>(ws + L.qw);
  auto *sc = reinterpret_cast<uint16_t *>(ws + L.sc);
  auto *zr = cfg.zero_point ? reinterpret_cast<uint8_t *>(ws + L.zr) : nullptr;
  auto *yref = reinterpret_cast<float *>(ws + L.yref);
  auto *partials = reinterpret_cast<double *>(ws + L.partials);
  auto *dlosses = reinterpret_cast<double *>(ws + L.losses);
  auto *dbest = reinterpret_cast<int32_t *>(ws + L.best);
  const auto *x = reinterpret_cast<const uint16_t *>(X);
  const auto *w = reinterpret_cast<const uint16_t *>(W);
  const int gs = cfg.group_size;

  auto *wbar = duo ? reinterpret_cast<double *>(ws + L.wbar) : nullptr;
  hipError_t e = awq::launch_mean_abs(x, M, K, units, xbar, s);
  if (e == hipSuccess && duo)   // the weights' statistic: the same kernel over the N rows of W
    e = awq::launch_mean_abs(w, N, K, reinterpret_cast<uint64_t *>(ws + L.wunits), wbar, s);
  if (e == hipSuccess) e = awq::launch_scale_table(xbar, wbar, K, grid, n_alpha, table, s);
  if (e == hipSuccess) e = awq::launch_gemm_dense_f32(x, w, M, N, K, yref, s);
  for (int j = 0; j < n_alpha && e == hipSuccess; ++j) {
    const float *sj = table + (size_t)j * K;
    e = awq::launch_quantize_pack(w, N, K, gs, sj, qw, sc, zr, nullptr, s);
    if (e == hipSuccess) e = awq::launch_scale_activation(x, sj, M, K, act, s);
    if (e == hipSuccess)
      e = awq::launch_gemm_loss(act, qw, sc, zr, M, N, K, gs, yref, partials + j * L.tiles, s);
  }
  if (e == hipSuccess) e = awq::launch_reduce_losses(partials, L.tiles, n_alpha, dlosses, dbest, s);
  double hlosses[64];
  int32_t hbest = 0;
  if (e == hipSuccess)
    e = hipMemcpyAsync(hlosses, dlosses, sizeof(double) * n_alpha, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&hbest, dbest, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "awq_scale_search");
  if (hbest < 0 || hbest >= n_alpha)
    return fail(AWQ_ERR_HIP, "awq_scale_search: device returned index %d", hbest);

  const float *sbest = table + (size_t)hbest * K;
  e = hipMemcpyAsync(best_s, sbest, sizeof(float) * K, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && !clip)
    e = awq::launch_quantize_pack(w, N, K, gs, sbest, qweight, scales,
                                  cfg.zero_point ? zeros : nullptr, nullptr, s);
  if (e == hipSuccess && clip) {
    // the clipping search on the chosen scaling, with A = fp16(X / s)
    e = awq::launch_scale_activation(x, sbest, M, K, act, s);
    if (e == hipSuccess)
      e = awq::launch_clip_search(w, sbest, act, M, N, K, gs,
                                  reinterpret_cast<double *>(ws + L.gram_partial),
                                  reinterpret_cast<double *>(ws + L.gram), qweight, scales,
                                  cfg.zero_point ? zeros : nullptr, clip_index, s);
  }
  if (e != hipSuccess) return hip_status(e, "awq_scale_search (final pack)");
  *best_index = hbest;
  if (losses) std::memcpy(losses, hlosses, sizeof(double) * n_alpha);
  return ok();
}

}  // extern "C"
