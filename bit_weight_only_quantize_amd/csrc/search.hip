// Scale-search kernels for gfx950: activation statistic, candidate scale
// vectors, scaled activations and the deterministic loss reduction.
//
// Follows "AWQ Advanced Usage Guide", "How AWQ Works" (salient channels from
// activation distributions; objective L(s) = ||Q(W*s)(s^-1*X) - W*X||) and the
// ai.lansai.wang explainer, section "AWQ 的四步链路" (Y = (X/s)(sW); collect
// input magnitudes, then evaluate candidate scalings by reconstruction error).
// The statistic is xbar_k = mean_m |X_mk|; candidate j uses
// s = fp32(t / sqrt(max t * min t)), t = max(xbar, 2^-24)^alpha_j.

#include "awq_internal.h"
#include "device_common.h"
#include "exact_quotient.h"

namespace awq {

// ---- xbar: column sums of |X|, exact ---------------------------------------------
// An fp16 magnitude is an integer number of units of 2^-24 (below 2^40), so the
// column sums are accumulated as 64-bit integers: exact for any M < 2^24 and
// independent of the order in which the atomics land.  The mean is then the
// correctly rounded quotient of the exact sum by M (rn_quotient_u64, exact
// also for sums beyond 2^53, where a conversion to fp64 first would round
// twice), times 2^-24.
// A workgroup of 16 waves sums a block of 512 columns by 128 rows: each wave
// takes every 16th row of the block (8 rows, all loads in flight at once),
// the waves' sums meet in LDS, and one 64-bit atomic per column and block
// adds the block's sum.  (Per-thread atomics over 16- or 64-row strips were
// atomic- or latency-bound at a tenth of HBM bandwidth.)
constexpr int kAbsWaves = 16;
constexpr int kAbsRowsPerWave = 8;
constexpr int kAbsRows = kAbsWaves * kAbsRowsPerWave;
constexpr int kAbsCols = 64 * 8;

__device__ __forceinline__ uint64_t half_magnitude_units(uint32_t h) {
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t f = h & 0x3FFu;
  return e == 0 ? (uint64_t)f : ((uint64_t)(1024u + f) << (e - 1));
}

__global__ __launch_bounds__(256) void zero_u64_kernel(uint64_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(64 * kAbsWaves) void abs_colsum_kernel(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, unsigned long long *__restrict__ sums) {
  __shared__ uint64_t part[kAbsWaves][kAbsCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * kAbsCols + lane * 8;   // this lane's 8 columns
  uint64_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // row blocks blockIdx.y, + gridDim.y, ... (the grid's y extent is capped)
  for (int64_t b = blockIdx.y; k0 < K && b * kAbsRows < M; b += gridDim.y) {
    const int64_t m0 = b * kAbsRows + wave;                       // rows m0 + 16 r
    u32x4 v[kAbsRowsPerWave];
    if ((b + 1) * kAbsRows <= M) {                      // uniform: a full block
#pragma unroll
      for (int r = 0; r < kAbsRowsPerWave; ++r)
        v[r] = *reinterpret_cast<const u32x4 *>(X + (m0 + kAbsWaves * r) * K + k0);
    } else {                                            // rows past M count as zero
#pragma unroll
      for (int r = 0; r < kAbsRowsPerWave; ++r) {
        const int64_t m = m0 + kAbsWaves * r;
        v[r] = m < M ? *reinterpret_cast<const u32x4 *>(X + m * K + k0) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int r = 0; r < kAbsRowsPerWave; ++r) {
      const u32x4 w = v[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[i];
        acc[2 * i] += half_magnitude_units(x & 0xFFFFu);
        acc[2 * i + 1] += half_magnitude_units(x >> 16);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[wave][lane * 8 + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < kAbsCols) {
    uint64_t t = 0;
#pragma unroll
    for (int w = 0; w < kAbsWaves; ++w) t += part[w][threadIdx.x];
    const int64_t k = (int64_t)blockIdx.x * kAbsCols + threadIdx.x;
    if (k < K) atomicAdd(&sums[k], (unsigned long long)t);
  }
}

__global__ __launch_bounds__(256) void mean_from_units_kernel(const uint64_t *__restrict__ units,
                                                              int64_t n, uint32_t m,
                                                              double *__restrict__ xbar) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) xbar[i] = rn_quotient_u64(units[i], m) * 0x1p-24;
}

hipError_t launch_mean_abs(const uint16_t *X, int64_t M, int64_t K, uint64_t *units,
                           double *xbar, hipStream_t st) {
  const unsigned gk = (unsigned)((K + 255) / 256);
  zero_u64_kernel<<<gk, 256, 0, st>>>(units, K);
  const int64_t blocks = (M + kAbsRows - 1) / kAbsRows;
  const dim3 grid((unsigned)((K + kAbsCols - 1) / kAbsCols), (unsigned)(blocks < 4096 ? blocks : 4096));
  abs_colsum_kernel<<<grid, 64 * kAbsWaves, 0, st>>>(X, M, K,
                                                     reinterpret_cast<unsigned long long *>(units));
  mean_from_units_kernel<<<gk, 256, 0, st>>>(units, K, (uint32_t)M, xbar);
  return hipGetLastError();
}

// ---- s-table: one workgroup per alpha ------------------------------------------
struct Alphas {
  double a[64];
};

constexpr int kTableThreads = 1024;

__device__ __forceinline__ double stat_pow(double xbar, double alpha) {
  return pow(fmax(xbar, 0x1p-24), alpha);
}

__global__ __launch_bounds__(kTableThreads) void scale_table_kernel(
    const double *__restrict__ xbar, int64_t K, Alphas alphas, float *__restrict__ table) {
  const int j = blockIdx.x;
  const double alpha = alphas.a[j];
  double tmax = 0.0, tmin = __builtin_huge_val();
  for (int64_t k = threadIdx.x; k < K; k += kTableThreads) {
    const double t = stat_pow(xbar[k], alpha);
    tmax = fmax(tmax, t);
    tmin = fmin(tmin, t);
  }
  // max / min are exact, so the reduction order does not matter.
  for (int off = 32; off > 0; off >>= 1) {
    tmax = fmax(tmax, __shfl_xor(tmax, off, 64));
    tmin = fmin(tmin, __shfl_xor(tmin, off, 64));
  }
  __shared__ double smax[kTableThreads / 64], smin[kTableThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    smax[w] = tmax;
    smin[w] = tmin;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = smax[0], b = smin[0];
    for (int i = 1; i < kTableThreads / 64; ++i) {
      a = fmax(a, smax[i]);
      b = fmin(b, smin[i]);
    }
    smax[0] = a;
    smin[0] = b;
  }
  __syncthreads();
  const double norm = sqrt(smax[0] * smin[0]);
  for (int64_t k = threadIdx.x; k < K; k += kTableThreads)
    table[j * K + k] = (float)(stat_pow(xbar[k], alpha) / norm);
}

hipError_t launch_scale_table(const double *xbar, int64_t K, const double *alphas, int n_alpha,
                              float *s_table, hipStream_t st) {
  Alphas a;
  for (int j = 0; j < 64; ++j) a.a[j] = j < n_alpha ? alphas[j] : 0.0;
  scale_table_kernel<<<n_alpha, kTableThreads, 0, st>>>(xbar, K, a, s_table);
  return hipGetLastError();
}

// ---- A = fp16(fp32(X) / s) --------------------------------------------------------
__global__ __launch_bounds__(256) void scale_activation_kernel(const uint16_t *__restrict__ X,
                                                               const float *__restrict__ s,
                                                               int64_t M, int64_t K,
                                                               uint16_t *__restrict__ A) {
  const int64_t words = M * K / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= words) return;
  const int64_t k0 = (t * 8) % K;
  const u32x4 v = *reinterpret_cast<const u32x4 *>(X + t * 8);
  const float4 s0 = *reinterpret_cast<const float4 *>(s + k0);
  const float4 s1 = *reinterpret_cast<const float4 *>(s + k0 + 4);
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = half_bits_to_float((uint16_t)(v[i] & 0xFFFFu)) / sv[2 * i];
    const float hi = half_bits_to_float((uint16_t)(v[i] >> 16)) / sv[2 * i + 1];
    o[i] = (uint32_t)float_to_half_bits(lo) | ((uint32_t)float_to_half_bits(hi) << 16);
  }
  *reinterpret_cast<u32x4 *>(A + t * 8) = o;
}

hipError_t launch_scale_activation(const uint16_t *X, const float *s, int64_t M, int64_t K,
                                   uint16_t *A, hipStream_t st) {
  const int64_t words = M * K / 8;
  if (words == 0) return hipSuccess;
  scale_activation_kernel<<<(unsigned)((words + 255) / 256), 256, 0, st>>>(X, s, M, K, A);
  return hipGetLastError();
}

// ---- losses and argmin --------------------------------------------------------------
// Each alpha's tile partials are summed sequentially in index order, so the
// result does not depend on scheduling.  The workgroup streams the partials
// through LDS in chunks of kLossChunk per alpha (cooperative, coalesced
// loads), and thread j continues alpha j's running sum over each chunk: the
// order of additions is the plain sequential one.  Thread 0 then takes the
// first minimum.
constexpr int kLossChunk = 128;

__global__ __launch_bounds__(1024) void reduce_losses_kernel(const double *__restrict__ partials,
                                                             int64_t n, int n_alpha,
                                                             double *__restrict__ losses,
                                                             int32_t *__restrict__ best) {
  __shared__ double chunk[64 * kLossChunk];
  __shared__ double sl[64];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t c0 = 0; c0 < n; c0 += kLossChunk) {
    const int len = n - c0 < kLossChunk ? (int)(n - c0) : kLossChunk;
    for (int i = tid; i < n_alpha * len; i += 1024) {
      const int j = i / len, t = i - j * len;
      chunk[j * kLossChunk + t] = partials[(int64_t)j * n + c0 + t];
    }
    __syncthreads();
    if (tid < n_alpha)
      for (int t = 0; t < len; ++t) s += chunk[tid * kLossChunk + t];
    __syncthreads();
  }
  if (tid < n_alpha) {
    sl[tid] = s;
    losses[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int b = 0;
    for (int i = 1; i < n_alpha; ++i)
      if (sl[i] < sl[b]) b = i;
    *best = b;
  }
}

hipError_t launch_reduce_losses(const double *partials, int64_t n_per_alpha, int n_alpha,
                                double *losses, int32_t *best, hipStream_t st) {
  reduce_losses_kernel<<<1, 1024, 0, st>>>(partials, n_per_alpha, n_alpha, losses, best);
  return hipGetLastError();
}

}  // namespace awq
