// C ABI of libawq355.so: argument validation, kernel dispatch and the
// orchestration of the alpha-grid scale search.  Every check runs before any
// HIP call, so invalid arguments are reported on machines without a GPU too.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

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

// GEMM scratch of awq_linear / awq_linear_ex (split-K partials, bf16 row
// factors and converted rows), one per device, allocated the first time a
// call needs it (or needs more).  A buffer is never freed: a larger one
// replaces it for later calls, and HIP graphs captured with the old one stay
// valid.  Its contents between calls do not matter.
struct Scratch {
  void *ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_scratch_mu;
std::map<int, Scratch> g_scratch;

hipError_t linear_scratch(size_t bytes, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  Scratch &s = g_scratch[dev];
  if (s.bytes < bytes) {
    const size_t want = bytes > 2 * s.bytes ? bytes : 2 * s.bytes;
    void *p = nullptr;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) return e;
    s.ptr = p;
    s.bytes = want;
  }
  *out = s.ptr;
  return hipSuccess;
}

// Automatic kernel choice (measured on MI355X, fp16, graph replays): the GEMV
// up to M = 8; from 9 to AWQ_GEMV_MAX_M rows only for layers of at most 5e7
// weights.  Above that the GEMV, whose activation reads grow with M once the
// rows no longer fit its LDS staging, is slower than the split-K GEMM (at
// M = 16: 28.7 vs 22.0 us for 13824 x 5120; the GEMV stays ahead on the
// 4096 x 4096 and 4096 x 11008 layers).
// GEMV or GEMM, from measured times on 7B- and 13B-class layers: the GEMV
// wins wherever it stages the activation rows in LDS; unstaged, its
// activation reads grow with M, and it loses where each wave walks a long
// chain of groups (> 8), beyond M = 8, or beyond M = 12 on layers of at most
// 5e7 weights.
bool auto_gemv(int64_t M, int64_t N, int64_t K, int g) {
  if (M > AWQ_GEMV_MAX_M || !awq::gemv_supported(M, N, K, g)) return false;
  if (awq::gemv_stages_activations(M, N, K)) return true;
  if (awq::gemv_groups_per_wave(N, K, g) > 8) return false;
  return M <= 8 || (M <= 12 && N * K <= 50000000);
}

awq_status check_config(awq_config cfg, int64_t K) {
  if (cfg.w_bit != 4) return fail(AWQ_ERR_UNSUPPORTED, "w_bit=%d: only 4 is supported", cfg.w_bit);
  if (cfg.zero_point != 1)
    return fail(AWQ_ERR_UNSUPPORTED, "zero_point=%d: only 1 (asymmetric) is supported",
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
  if (kernel != AWQ_KERNEL_AUTO && kernel != AWQ_KERNEL_GEMV && kernel != AWQ_KERNEL_GEMM)
    return fail(AWQ_ERR_INVALID_ARG, "kernel=%d: unknown kernel selector", kernel);
  if (kernel == AWQ_KERNEL_GEMV && M > AWQ_GEMV_MAX_M)
    return fail(AWQ_ERR_INVALID_ARG, "GEMV kernel serves M <= %d, got M=%lld", AWQ_GEMV_MAX_M,
                (long long)M);
  if (M == 0 || N == 0) return AWQ_OK;
  if (!awq::gemm_supported(N, K, false))
    return fail(AWQ_ERR_UNSUPPORTED, "layer of %lld x %lld exceeds 2 GiB of packed weights",
                (long long)N, (long long)K);
  if (!X || !qweight || !scales || !zeros || !Y)
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

// Workspace layout of the scale search (each region 256-byte aligned).
struct SearchLayout {
  size_t units, xbar, table, act, qw, sc, zr, yref, partials, losses, best, total;
  int64_t tiles;
};

SearchLayout search_layout(int64_t M, int64_t N, int64_t K, int gs, int n_alpha) {
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
  L.total = off;
  return L;
}

awq_status check_search(int64_t M, int64_t N, int64_t K, awq_config cfg, int32_t n_alpha) {
  awq_status st = check_config(cfg, K);
  if (st != AWQ_OK) return st;
  if (M < 1 || N < 1) return fail(AWQ_ERR_INVALID_ARG, "M and N must be >= 1");
  if (M > ((int64_t)1 << 24) - 1)
    return fail(AWQ_ERR_INVALID_ARG, "M=%lld exceeds 2^24-1 calibration rows", (long long)M);
  if (N > ((int64_t)1 << 31)) return fail(AWQ_ERR_INVALID_ARG, "N too large");
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
  if (!W || !qweight || !scales || !zeros)
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(W, 16) || !aligned(qweight, 16))
    return fail(AWQ_ERR_INVALID_ARG, "W and qweight must be 16-byte aligned");
  if (s && !aligned(s, 16)) return fail(AWQ_ERR_INVALID_ARG, "s must be 16-byte aligned");
  if (!aligned(scales, 2)) return fail(AWQ_ERR_INVALID_ARG, "scales must be 2-byte aligned");
  if (nonfinite_count && !aligned(nonfinite_count, 4))
    return fail(AWQ_ERR_INVALID_ARG, "nonfinite_count must be 4-byte aligned");
  return hip_status(awq::launch_quantize_pack(reinterpret_cast<const uint16_t *>(W), N, K,
                                              cfg.group_size, s, qweight, scales, zeros,
                                              nonfinite_count, as_stream(stream)),
                    "awq_quantize_pack");
}

namespace {

// awq_linear_ex with an optional caller workspace (NULL: the library scratch).
awq_status linear_impl(const void *X, int32_t x_dtype, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, awq_config cfg, void *Y, int32_t y_dtype, int32_t kernel,
                       void *workspace, size_t workspace_bytes, bool caller_ws,
                       awq_stream_t stream) {
  awq_status st =
      check_linear(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype, kernel);
  if (st != AWQ_OK) return st;
  const awq::XType xt = x_dtype == AWQ_F16 ? awq::XType::F16 : awq::XType::BF16;
  const awq::GemmPlan plan = awq::gemm_plan(M > 0 ? M : 1, N > 0 ? N : 1, K, xt);
  const bool gemv_ok = awq::gemv_supported(M, N > 0 ? N : 1, K, cfg.group_size);
  if (kernel == AWQ_KERNEL_GEMV && !gemv_ok)
    return fail(AWQ_ERR_UNSUPPORTED, "GEMV kernel cannot serve K=%lld", (long long)K);
  const bool gemv = kernel == AWQ_KERNEL_GEMV ||
                    (kernel == AWQ_KERNEL_AUTO && auto_gemv(M, N, K, cfg.group_size));
  if (caller_ws && !gemv && plan.workspace_bytes > 0) {
    if (!workspace) return fail(AWQ_ERR_INVALID_ARG, "this shape needs a workspace");
    if (!aligned(workspace, 256)) return fail(AWQ_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    // The documented minimum (awq_linear_workspace_size) covers both
    // activation types.
    const size_t need = awq::gemm_workspace_bytes(M, N, K);
    if (workspace_bytes < need)
      return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  if (M == 0 || N == 0) return ok();
  const awq::YType yt = y_dtype == AWQ_F16    ? awq::YType::F16
                        : y_dtype == AWQ_BF16 ? awq::YType::BF16
                                              : awq::YType::F32;
  const hipStream_t hs = as_stream(stream);
  if (gemv)
    return hip_status(awq::launch_gemv(X, xt, qweight, scales, zeros, M, N, K, cfg.group_size, Y,
                                       yt, hs),
                      "awq_linear (gemv)");
  void *scratch = caller_ws ? workspace : nullptr;
  if (!caller_ws && plan.workspace_bytes > 0) {
    const hipError_t e = linear_scratch(plan.workspace_bytes, &scratch);
    if (e != hipSuccess) return hip_status(e, "awq_linear (split-K scratch)");
  }
  return hip_status(awq::launch_gemm(X, xt, qweight, scales, zeros, M, N, K, cfg.group_size, Y,
                                     yt, scratch, hs),
                    "awq_linear (gemm)");
}

}  // namespace

awq_status awq_linear_ex(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, int32_t kernel,
                         awq_stream_t stream) {
  return linear_impl(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype, kernel,
                     nullptr, 0, false, stream);
}

size_t awq_linear_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg) {
  if (check_config(cfg, K) != AWQ_OK || M < 0 || N < 0) return 0;
  if (M == 0 || N == 0) return 0;
  if (auto_gemv(M, N, K, cfg.group_size)) return 0;
  return awq::gemm_workspace_bytes(M, N, K);
}

awq_status awq_linear_ws(const void *X, int32_t x_dtype, const uint32_t *qweight,
                         const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                         int64_t K, awq_config cfg, void *Y, int32_t y_dtype, void *workspace,
                         size_t workspace_bytes, awq_stream_t stream) {
  return linear_impl(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype,
                     AWQ_KERNEL_AUTO, workspace, workspace_bytes, true, stream);
}

awq_status awq_linear(const void *X, int32_t x_dtype, const uint32_t *qweight,
                      const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                      int64_t K, awq_config cfg, void *Y, int32_t y_dtype, awq_stream_t stream) {
  return awq_linear_ex(X, x_dtype, qweight, scales, zeros, M, N, K, cfg, Y, y_dtype,
                       AWQ_KERNEL_AUTO, stream);
}

size_t awq_scale_search_workspace_size(int64_t M, int64_t N, int64_t K, awq_config cfg,
                                       int32_t n_alpha) {
  if (check_search(M, N, K, cfg, n_alpha) != AWQ_OK) return 0;
  return search_layout(M, N, K, cfg.group_size, n_alpha).total;
}

awq_status awq_scale_search(const void *X, const void *W, int64_t M, int64_t N, int64_t K,
                            awq_config cfg, const double *alphas, int32_t n_alpha,
                            void *workspace, size_t workspace_bytes, int32_t *best_index,
                            double *losses, float *best_s, uint32_t *qweight,
                            uint16_t *scales, uint8_t *zeros, awq_stream_t stream) {
  awq_status st = check_search(M, N, K, cfg, n_alpha);
  if (st != AWQ_OK) return st;
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
  if (!X || !W || !workspace || !best_index || !best_s || !qweight || !scales || !zeros)
    return fail(AWQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(qweight, 16) || !aligned(best_s, 16))
    return fail(AWQ_ERR_INVALID_ARG, "X, W, qweight and best_s must be 16-byte aligned");
  if (!aligned(workspace, kAlign))
    return fail(AWQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!aligned(scales, 2)) return fail(AWQ_ERR_INVALID_ARG, "scales must be 2-byte aligned");
  const SearchLayout L = search_layout(M, N, K, cfg.group_size, n_alpha);
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
  auto *zr = reinterpret_cast<uint8_t *>(ws + L.zr);
  auto *yref = reinterpret_cast<float *>(ws + L.yref);
  auto *partials = reinterpret_cast<double *>(ws + L.partials);
  auto *dlosses = reinterpret_cast<double *>(ws + L.losses);
  auto *dbest = reinterpret_cast<int32_t *>(ws + L.best);
  const auto *x = reinterpret_cast<const uint16_t *>(X);
  const auto *w = reinterpret_cast<const uint16_t *>(W);
  const int gs = cfg.group_size;

  hipError_t e = awq::launch_mean_abs(x, M, K, units, xbar, s);
  if (e == hipSuccess) e = awq::launch_scale_table(xbar, K, grid, n_alpha, table, s);
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
  if (e == hipSuccess)
    e = awq::launch_quantize_pack(w, N, K, gs, sbest, qweight, scales, zeros, nullptr, s);
  if (e != hipSuccess) return hip_status(e, "awq_scale_search (final pack)");
  *best_index = hbest;
  if (losses) std::memcpy(losses, hlosses, sizeof(double) * n_alpha);
  return ok();
}

}  // extern "C"
