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

// t = max(xbar, 2^-24)^alpha, and with duo scaling ("Calibration Parameters":
// duo_scaling scales by weights and activations) divided by
// max(wbar, 2^-24)^(1 - alpha), wbar the mean |W| of the input channel.
__device__ __forceinline__ double stat_pow(const double *xbar, const double *wbar, int64_t k,
                                           double alpha) {
  double t = pow(fmax(xbar[k], 0x1p-24), alpha);
  if (wbar) t = t / pow(fmax(wbar[k], 0x1p-24), 1.0 - alpha);
  return t;
}

__global__ __launch_bounds__(kTableThreads) void scale_table_kernel(
    const double *__restrict__ xbar, const double *__restrict__ wbar, int64_t K, Alphas alphas,
    float *__restrict__ table) {
  const int j = blockIdx.x;
  const double alpha = alphas.a[j];
  double tmax = 0.0, tmin = __builtin_huge_val();
  for (int64_t k = threadIdx.x; k < K; k += kTableThreads) {
    const double t = stat_pow(xbar, wbar, k, alpha);
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
    table[j * K + k] = (float)(stat_pow(xbar, wbar, k, alpha) / norm);
}

hipError_t launch_scale_table(const double *xbar, const double *wbar, int64_t K,
                              const double *alphas, int n_alpha, float *s_table, hipStream_t st) {
  Alphas a;
  for (int j = 0; j < 64; ++j) a.a[j] = j < n_alpha ? alphas[j] : 0.0;
  scale_table_kernel<<<n_alpha, kTableThreads, 0, st>>>(xbar, wbar, K, a, s_table);
  return hipGetLastError();
}

// ---- weight clipping ------------------------------------------------------------------
// "Calibration Parameters": apply_clip, "Apply weight clipping".  Per output
// row n and group g of the chosen scaling, the shrink factor c of a 20-point
// grid whose quantization minimizes the group's output error on the
// calibration inputs, E_c = ||A_g d||^2 = d^T C_g d with A = fp16(X / s), d =
// v - deq_c(v), v = fp32(s * W) and C_g = A_g^T A_g.  C is accumulated in fp64
// (products of fp16 values are exact), d is exact in fp32 (deq is 0 or within
// a factor 2 of v, and has at most 15 significant bits), E is fp64: the
// choice differs from an exact evaluation only at fp64 near-ties.

constexpr int kGramRows = 512;     // calibration rows per partial Gram matrix
constexpr int kGramTile = 32;      // rows staged in LDS at a time

// Partial Gram matrices: grid (G, P); workgroup (g, p) sums rows
// [p * kGramRows, (p + 1) * kGramRows) of group g.  Thread t owns the 8 x 8
// block (t / 16, t % 16) of a 128 x 128 matrix (g = 64: 4 x 4 blocks of the
// 64 x 64 one, threads 0..255 as 16 x 16 blocks).
template <int GS>
__global__ __launch_bounds__(256) void gram_partial_kernel(const uint16_t *__restrict__ A,
                                                           int64_t M, int64_t K,
                                                           double *__restrict__ partial) {
  constexpr int kB = GS / 16;                       // block edge: 8 (g128) or 4 (g64)
  __shared__ __attribute__((aligned(16))) uint16_t tile[kGramTile][GS];
  const int g = blockIdx.x, p = blockIdx.y, P = gridDim.y;
  const int t = threadIdx.x, bi = t / 16, bj = t % 16;
  double acc[kB][kB];
#pragma unroll
  for (int i = 0; i < kB; ++i)
#pragma unroll
    for (int j = 0; j < kB; ++j) acc[i][j] = 0.0;
  const int64_t m0 = (int64_t)p * kGramRows, m1 = m0 + kGramRows < M ? m0 + kGramRows : M;
  for (int64_t mt = m0; mt < m1; mt += kGramTile) {
    __syncthreads();
    // stage kGramTile rows x GS columns (16 bytes per thread and round)
    for (int e = t; e < kGramTile * GS / 8; e += 256) {
      const int r = e / (GS / 8), ch = e % (GS / 8);
      const int64_t m = mt + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < m1) v = *reinterpret_cast<const u32x4 *>(A + m * K + (int64_t)g * GS + ch * 8);
      *reinterpret_cast<u32x4 *>(&tile[r][ch * 8]) = v;
    }
    __syncthreads();
    const int rows = m1 - mt < kGramTile ? (int)(m1 - mt) : kGramTile;
    for (int r = 0; r < rows; ++r) {
      double a[kB], b[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        a[i] = (double)half_bits_to_float(tile[r][bi * kB + i]);
        b[i] = (double)half_bits_to_float(tile[r][bj * kB + i]);
      }
#pragma unroll
      for (int i = 0; i < kB; ++i)
#pragma unroll
        for (int j = 0; j < kB; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
    }
  }
  double *out = partial + ((int64_t)g * P + p) * GS * GS;
#pragma unroll
  for (int i = 0; i < kB; ++i)
#pragma unroll
    for (int j = 0; j < kB; ++j) out[(bi * kB + i) * GS + bj * kB + j] = acc[i][j];
}

// The clip selection multiplies 16 x 16 blocks of C on the matrix cores
// (mfma_f64_16x16x4: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// and holds D[4 r + l / 16][l % 16] in its r-th result, r = 0..3; measured
// on gfx950 with single-entry operands).  Block pair (I, J), I <= J,
// is pair index I*NB - I(I-1)/2 + (J - I); its operand for k-step s is
//   frag[pair][s][l] = C'[16 I + l % 16][16 J + 4 s + l / 16],
// C' = C on the diagonal blocks and 2C above them (exact), so that
//   d^T C d = sum_I d_I^T (sum_{J >= I} C'_IJ d_J).
// gram_frag_kernel sums the P partials of each element in index order and
// writes it there.  Grid (G, pairs), 256 threads: thread s * 64 + l.
template <int GS>
__global__ __launch_bounds__(256) void gram_frag_kernel(const double *__restrict__ partial,
                                                        int P, double *__restrict__ frag) {
  constexpr int NB = GS / 16;
  const int g = blockIdx.x, pair = blockIdx.y;
  int I = 0, rem = pair;
  while (rem >= NB - I) {
    rem -= NB - I;
    ++I;
  }
  const int J = I + rem;
  const int st = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int i = 16 * I + (l & 15), j = 16 * J + 4 * st + (l >> 4);
  const double *src = partial + (int64_t)g * P * GS * GS + i * GS + j;
  double v = 0.0;
  for (int p = 0; p < P; ++p) v += src[(int64_t)p * GS * GS];
  if (I < J) v *= 2.0;
  frag[(int64_t)g * clip_gram_doubles(GS) + (int64_t)pair * 256 + threadIdx.x] = v;
}

struct ClipGrid {
  float c[kClipPoints];
};

// Quantization of value v with shrink factor c: the step (fp16 bits) and the
// zero point of the group (lo, hi, amax over the group), then code(v).  The
// arithmetic of quantize_pack_kernel with the range scaled by c, written
// with IEEE divisions (this kernel is not bound by them).
template <bool SYM>
__device__ __forceinline__ void clip_params(float lo, float hi, float amax, float c, float &sf,
                                            float &zf, uint16_t &sbits) {
  float step;
  if constexpr (SYM) {
    step = (amax * c) / 7.0f;
  } else {
    step = (hi * c - lo * c) / 15.0f;
  }
  const _Float16 sh = (_Float16)fmaxf(step, 0x1p-14f);
  sbits = __builtin_bit_cast(uint16_t, sh);
  sf = (float)sh;
  zf = SYM ? 8.0f : fminf(fmaxf(__builtin_rintf(-(lo * c) / sf), 0.0f), 15.0f);
}
template <bool SYM>
__device__ __forceinline__ float clip_code(float v, float sf, float zf) {
  const float q = __builtin_rintf(v / sf);
  return SYM ? fminf(fmaxf(q, -8.0f), 7.0f) + 8.0f : fminf(fmaxf(q + zf, 0.0f), 15.0f);
}

// Grid point ci (lane-varying) without a dynamic index into the argument block.
__device__ __forceinline__ float clip_factor(const ClipGrid &grid, int ci) {
  float c = grid.c[0];
#pragma unroll
  for (int i = 1; i < kClipPoints; ++i) c = ci == i ? grid.c[i] : c;
  return c;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Per group g and 32 rows of W: E[r][c] = d^T C_g d for each row r and grid
// point c, d = v - deq_c(v) (exact in fp32), in fp64 on the matrix cores.
// The 640 columns (row, c) form 40 blocks of 16 (block b: rows 16 (b / 20)
// .. + 15, point b % 20); wave w takes blocks 10 w .. 10 w + 9, two at a
// time.  Per pair of blocks it builds the B operands d_J (every j, in
// registers) and, for each row block I, U_I = sum_{J >= I} C'_IJ d_J and
// E += d_I . U_I (lane-wise, then over the four lanes of a column in a fixed
// order).  Then each row takes the first minimum over c (strict <, in grid
// order) and packs its codes, scale and zero point for it.
constexpr int kClipRowsPerBlock = 32;
template <int GS, bool SYM>
__global__ __launch_bounds__(256) void clip_select_kernel(
    const uint16_t *__restrict__ W, const float *__restrict__ s, int64_t N, int64_t K,
    const double *__restrict__ frag, ClipGrid grid, uint32_t *__restrict__ qweight,
    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros, uint8_t *__restrict__ clip_index) {
  constexpr int NB = GS / 16;
  constexpr int kPairs = NB * (NB + 1) / 2;
  constexpr int R = kClipRowsPerBlock;
  __shared__ __attribute__((aligned(16))) double sC[kPairs * 256];
  // rows padded by 4 floats: a column's 16 lanes (16 rows) hit distinct banks
  __shared__ __attribute__((aligned(16))) float sV[R][GS + 4];
  __shared__ float sStat[R][3];
  __shared__ double sE[R][kClipPoints];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.y;
  const int G = (int)(K / GS);
  const int64_t row0 = (int64_t)blockIdx.x * R;

  // this group's operand blocks, and v = fp32(s * W) of the block's rows
  // (rows past N repeat row N - 1; nothing of theirs is stored)
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(frag + (int64_t)g * (kPairs * 256));
    u32x4 *dst = reinterpret_cast<u32x4 *>(sC);
    for (int e = tid; e < kPairs * 128; e += 256) dst[e] = src[e];
  }
  for (int e = tid; e < R * GS / 8; e += 256) {
    const int r = e / (GS / 8), k8 = e % (GS / 8);
    const int64_t n = row0 + r < N ? row0 + r : N - 1;
    const u32x4 wv = *reinterpret_cast<const u32x4 *>(W + n * K + (int64_t)g * GS + k8 * 8);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint16_t h = (uint16_t)(wv[q >> 1] >> (16 * (q & 1)));
      sV[r][k8 * 8 + q] = s[(int64_t)g * GS + k8 * 8 + q] * half_bits_to_float(h);
    }
  }
  __syncthreads();
  // row statistics: 8 threads per row
  {
    const int r = tid >> 3, part = tid & 7;
    float lo = 0.0f, hi = 0.0f, amax = 0.0f;
    for (int k = part; k < GS; k += 8) {
      const float v = sV[r][k];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
      amax = fmaxf(amax, __builtin_fabsf(v));
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, off, 64));
      hi = fmaxf(hi, __shfl_xor(hi, off, 64));
      amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    }
    if (part == 0) {
      sStat[r][0] = lo;
      sStat[r][1] = hi;
      sStat[r][2] = amax;
    }
  }
  __syncthreads();

  const int q = lane & 15, kq = lane >> 4;
  const int half = wave >> 1;                         // rows 16 half .. 16 half + 15
  const int rl = 16 * half + q;                        // this lane's row within the block
  const float lo = sStat[rl][0], hi = sStat[rl][1], amax = sStat[rl][2];
  for (int t = 0; t < 5; ++t) {
    const int ca = (wave & 1) * 10 + 2 * t, cb = ca + 1;
    float sfa, zfa, sfb, zfb;
    uint16_t sbits;
    clip_params<SYM>(lo, hi, amax, grid.c[ca], sfa, zfa, sbits);
    clip_params<SYM>(lo, hi, amax, grid.c[cb], sfb, zfb, sbits);
    auto dd = [&](int j, float sf, float zf) {
      const float v = sV[rl][j];
      return (double)(v - (clip_code<SYM>(v, sf, zf) - zf) * sf);
    };
    double bA[NB][4], bB[NB][4];
#pragma unroll
    for (int J = 0; J < NB; ++J)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bA[J][st] = dd(16 * J + 4 * st + kq, sfa, zfa);
        bB[J][st] = dd(16 * J + 4 * st + kq, sfb, zfb);
      }
    double eA = 0.0, eB = 0.0;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      // one row block at a time: keeps the compiler from hoisting every
      // block's operand reads and error terms at once (register spills)
      __builtin_amdgcn_sched_barrier(0);
      f64x4 uA = {0.0, 0.0, 0.0, 0.0}, uB = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int J = I; J < NB; ++J) {
        const int pair = I * NB - I * (I - 1) / 2 + (J - I);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const double a = sC[(pair * 4 + st) * 64 + lane];
          uA = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bA[J][st], uA, 0, 0, 0);
          uB = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bB[J][st], uB, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * r + kq;
        eA = __builtin_fma(dd(i, sfa, zfa), uA[r], eA);
        eB = __builtin_fma(dd(i, sfb, zfb), uB[r], eB);
      }
    }
    eA += __shfl_xor(eA, 16, 64);
    eB += __shfl_xor(eB, 16, 64);
    eA += __shfl_xor(eA, 32, 64);
    eB += __shfl_xor(eB, 32, 64);
    if (kq == 0) {
      sE[rl][ca] = eA;
      sE[rl][cb] = eB;
    }
  }
  __syncthreads();

  // per row (8 threads each): first minimum over the grid, then the row's
  // codes for it, GS/64 packed words per thread
  constexpr int kWordsPerRow = GS / 8;
  constexpr int kThreadsPerRow = 256 / R;              // 8
  constexpr int kWordsPerThread = kWordsPerRow / kThreadsPerRow;
  const int r = tid / kThreadsPerRow, part = tid % kThreadsPerRow;
  const int64_t n = row0 + r;
  if (n >= N) return;
  int best = 0;
  double ebest = sE[r][0];
#pragma unroll
  for (int ci = 1; ci < kClipPoints; ++ci) {
    const double e = sE[r][ci];
    if (e < ebest) {                                   // strict: the first minimum wins
      ebest = e;
      best = ci;
    }
  }
  float sf, zf;
  uint16_t sb;
  clip_params<SYM>(sStat[r][0], sStat[r][1], sStat[r][2], clip_factor(grid, best), sf, zf, sb);
#pragma unroll
  for (int u = 0; u < kWordsPerThread; ++u) {
    const int wi = part * kWordsPerThread + u;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      word |= ((uint32_t)clip_code<SYM>(sV[r][wi * 8 + e], sf, zf)) << (4 * nibble_of_channel(e));
    qweight[n * (K / 8) + (int64_t)g * (GS / 8) + wi] = word;
  }
  if (part == 0) {
    scales[n * G + g] = sb;
    if constexpr (!SYM) zeros[n * G + g] = (uint8_t)zf;
    if (clip_index) clip_index[n * G + g] = (uint8_t)best;
  }
}

int64_t gram_parts(int64_t M) { return (M + kGramRows - 1) / kGramRows; }

hipError_t launch_clip_search(const uint16_t *W, const float *s, const uint16_t *A, int64_t M,
                              int64_t N, int64_t K, int gs, double *gram_partial, double *gram,
                              uint32_t *qweight, uint16_t *scales, uint8_t *zeros,
                              uint8_t *clip_index, hipStream_t st) {
  const int64_t G = K / gs, P = gram_parts(M);
  ClipGrid grid;
  for (int i = 0; i < kClipPoints; ++i) grid.c[i] = (float)(1.0 - (double)i / 40.0);
  const dim3 cgrid((unsigned)((N + kClipRowsPerBlock - 1) / kClipRowsPerBlock), (unsigned)G);
  const unsigned pairs = (unsigned)(clip_gram_doubles(gs) / 256);
  if (gs == 128) {
    gram_partial_kernel<128><<<dim3((unsigned)G, (unsigned)P), 256, 0, st>>>(A, M, K, gram_partial);
    gram_frag_kernel<128><<<dim3((unsigned)G, pairs), 256, 0, st>>>(gram_partial, (int)P, gram);
    if (zeros)
      clip_select_kernel<128, false><<<cgrid, 256, 0, st>>>(W, s, N, K, gram, grid, qweight, scales, zeros, clip_index);
    else
      clip_select_kernel<128, true><<<cgrid, 256, 0, st>>>(W, s, N, K, gram, grid, qweight, scales, zeros, clip_index);
  } else {
    gram_partial_kernel<64><<<dim3((unsigned)G, (unsigned)P), 256, 0, st>>>(A, M, K, gram_partial);
    gram_frag_kernel<64><<<dim3((unsigned)G, pairs), 256, 0, st>>>(gram_partial, (int)P, gram);
    if (zeros)
      clip_select_kernel<64, false><<<cgrid, 256, 0, st>>>(W, s, N, K, gram, grid, qweight, scales, zeros, clip_index);
    else
      clip_select_kernel<64, true><<<cgrid, 256, 0, st>>>(W, s, N, K, gram, grid, qweight, scales, zeros, clip_index);
  }
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
