// Batched / prefill W4A16 GEMM on gfx950 MFMA.
//
// The GEMM variant of the quantized linear layer ("AWQ Advanced Usage Guide",
// "WQLinear Kernel Variants": batch sizes > 1).  Y = X * deq(W)^T with
// deq = (q - z) * s per group of g input channels.
//
// Exactness: the B operand is the exact integer q - z (fp16) or 128 + q
// (bf16, zero removed through the row sums of A), MFMA accumulates one group
// in fp32, and the group's scale multiplies that fp32 partial.  No dequantized
// weight is ever rounded to 16 bits.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of Y; its four
// waves each own a 64 x 64 quarter (4 x 4 MFMA tiles of 16 x 16).  K advances
// in blocks of 128 (one g128 group or two g64 groups).  The activation block
// (128 rows x 128 channels, 32 KiB fp16) is staged in LDS with a 16-byte row
// pad (conflict-free 128-bit reads) and prefetched into registers one block
// ahead.  Packed weights bypass LDS: each lane loads the 16 bytes it needs
// (32 codes of one column) one block ahead and dequantizes them in registers;
// each dequantized fragment feeds 4 MFMA tiles.  Block ids are remapped so
// each XCD works on a contiguous run of tiles that share activation rows.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kMT = 4, kNT = 4;        // 16x16 tiles per wave along M and N
constexpr int kLDA = kBK + 8;          // fp16 elements per LDS row (16-byte pad)
constexpr int kThreads = 256;

enum Epi : int { kEpiStore = 0, kEpiLoss = 1 };

}  // namespace

template <class XT, int GS, int EPI, bool DENSE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ Wdense, const uint16_t *__restrict__ scales,
    const uint8_t *__restrict__ zeros, int64_t M, int64_t N, int64_t K,
    void *__restrict__ Y, int ytype, const float *__restrict__ Yref,
    double *__restrict__ partials) {
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  constexpr int kGS = DENSE ? 128 : GS;
  constexpr int kWpl = kGS / 32;        // 8-channel words per lane per group
  constexpr int kGPB = kBK / kGS;       // groups per K block

  __shared__ __attribute__((aligned(16))) uint16_t sA[kBM * kLDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 15, kq = lane >> 4;

  const int64_t tiles_n = (N + kBN - 1) / kBN;
  const int64_t tiles_m = (M + kBM - 1) / kBM;
  const int64_t bid = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int64_t tm = bid / tiles_n, tn = bid - (bid / tiles_n) * tiles_n;
  if (tm >= tiles_m) return;
  const int64_t row0 = tm * kBM, col0 = tn * kBN;

  const int64_t G = K / kGS;
  const int64_t wrow = K / 8;
  const int64_t nkb = (K + kBK - 1) / kBK;

  // ---- activation block: global -> registers -> LDS ------------------------
  u32x4 apre[8];
  auto load_a = [&](int64_t kb) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (tid >> 4) + 16 * r;
      const int64_t kk = kb * kBK + (tid & 15) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row0 + row < M && kk < K)
        v = *reinterpret_cast<const u32x4 *>(X + (row0 + row) * K + kk);
      apre[r] = v;
    }
  };
  auto store_a = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (tid >> 4) + 16 * r;
      *reinterpret_cast<u32x4 *>(&sA[row * kLDA + (tid & 15) * 8]) = apre[r];
    }
  };

  // ---- packed weights, scales and zeros for one K block ----------------------
  int64_t ncol[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) ncol[j] = col0 + wn * 64 + j * 16 + c;

  uint32_t braw[kNT][kGPB][kWpl];
  float bsc[kNT][kGPB];
  uint32_t bzr[kNT][kGPB];
  auto load_b = [&](int64_t kb) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        const int64_t g = kb * kGPB + gi;
        const bool ok = ncol[j] < N && g < G;
        const uint32_t *p = qweight + (ok ? ncol[j] : 0) * wrow + g * (kGS / 8) + kq * kWpl;
        if constexpr (kWpl == 4) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ok) v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
          for (int w = 0; w < kWpl; ++w) braw[j][gi][w] = v[w];
        } else {
          u32x2 v = {0u, 0u};
          if (ok) v = *reinterpret_cast<const u32x2 *>(p);
#pragma unroll
          for (int w = 0; w < kWpl; ++w) braw[j][gi][w] = v[w];
        }
        bsc[j][gi] = ok ? half_bits_to_float(scales[ncol[j] * G + g]) : 0.0f;
        bzr[j][gi] = ok ? (uint32_t)zeros[ncol[j] * G + g] : 0u;
      }
    }
  };

  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  if constexpr (!DENSE) load_b(0);
  store_a();
  __syncthreads();

  for (int64_t kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) load_a(kb + 1);

    if constexpr (DENSE) {
      // B straight from the fp16 weight rows (used for X * W^T only).
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        u32x4 b[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int64_t kk = kb * kBK + kq * 32 + 8 * st;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ncol[j] < N && kk < K)
            v = *reinterpret_cast<const u32x4 *>(Wdense + ncol[j] * K + kk);
          b[st] = v;
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
          const uint16_t *ap = &sA[(wm * 64 + i * 16 + c) * kLDA + kq * 32];
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc[i][j] = mfma32<XT>(*reinterpret_cast<const u32x4 *>(ap + 8 * st), b[st], acc[i][j]);
        }
      }
    } else {
      uint32_t craw[kNT][kGPB][kWpl];
      float csc[kNT][kGPB];
      uint32_t czr[kNT][kGPB];
#pragma unroll
      for (int j = 0; j < kNT; ++j)
#pragma unroll
        for (int gi = 0; gi < kGPB; ++gi) {
          csc[j][gi] = bsc[j][gi];
          czr[j][gi] = bzr[j][gi];
#pragma unroll
          for (int w = 0; w < kWpl; ++w) craw[j][gi][w] = braw[j][gi][w];
        }
      if (more) load_b(kb + 1);

#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        if (kb * kGPB + gi >= G) break;
        u32x4 bq[kNT][kWpl];
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          if constexpr (!kBF16) {
            const DeqF16 deq(czr[j][gi]);
#pragma unroll
            for (int w = 0; w < kWpl; ++w) bq[j][w] = deq(craw[j][gi][w]);
          } else {
            const DeqBF16 deq;
#pragma unroll
            for (int w = 0; w < kWpl; ++w) bq[j][w] = deq(craw[j][gi][w]);
          }
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
          const uint16_t *ap = &sA[(wm * 64 + i * 16 + c) * kLDA + gi * kGS + kq * 8 * kWpl];
          u32x4 a[kWpl];
#pragma unroll
          for (int w = 0; w < kWpl; ++w) a[w] = *reinterpret_cast<const u32x4 *>(ap + 8 * w);
          f32x4 rs = {0.f, 0.f, 0.f, 0.f};
          if constexpr (kBF16) {
#pragma unroll
            for (int w = 0; w < kWpl; ++w) rs = mfma32<TagBF16>(a[w], bf16_ones(), rs);
          }
#pragma unroll
          for (int j = 0; j < kNT; ++j) {
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWpl; ++w) t = mfma32<XT>(a[w], bq[j][w], t);
            if constexpr (kBF16) {
              const float cz = -(float)(128u + czr[j][gi]);
#pragma unroll
              for (int e = 0; e < 4; ++e) t[e] = __builtin_fmaf(cz, rs[e], t[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(t[e], csc[j][gi], acc[i][j][e]);
          }
        }
      }
    }

    __syncthreads();
    if (more) {
      store_a();
      __syncthreads();
    }
  }

  // ---- epilogue -------------------------------------------------------------
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = row0 + wm * 64 + i * 16 + 4 * kq + e;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const int64_t n = ncol[j];
          if (n >= N) continue;
          const float v = acc[i][j][e];
          const int64_t o = m * N + n;
          if (ytype == (int)YType::F16)
            reinterpret_cast<uint16_t *>(Y)[o] = float_to_half_bits(v);
          else if (ytype == (int)YType::BF16)
            reinterpret_cast<uint16_t *>(Y)[o] = float_to_bf16_bits(v);
          else
            reinterpret_cast<float *>(Y)[o] = v;
        }
      }
    }
  } else {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = row0 + wm * 64 + i * 16 + 4 * kq + e;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const int64_t n = ncol[j];
          if (n >= N) continue;
          const double d = (double)Yref[m * N + n] - (double)acc[i][j][e];
          sum = __builtin_fma(d, d, sum);
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    __shared__ double wsum[4];
    if (lane == 0) wsum[wave] = sum;
    __syncthreads();
    if (tid == 0) partials[tm * tiles_n + tn] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

int64_t gemm_tile_count(int64_t M, int64_t N) {
  return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
}

template <class XT, int GS, int EPI, bool DENSE>
static void gemm_go(const uint16_t *X, const uint32_t *qw, const uint16_t *Wd,
                    const uint16_t *sc, const uint8_t *zr, int64_t M, int64_t N, int64_t K,
                    void *Y, int yt, const float *Yref, double *partials, hipStream_t st) {
  const dim3 grid((unsigned)gemm_tile_count(M, N));
  gemm_kernel<XT, GS, EPI, DENSE><<<grid, kThreads, 0, st>>>(X, qw, Wd, sc, zr, M, N, K, Y, yt,
                                                            Yref, partials);
}

hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
  const int y = (int)yt;
  if (xt == XType::F16) {
    if (gs == 128)
      gemm_go<TagF16, 128, kEpiStore, false>(x, qweight, nullptr, scales, zeros, M, N, K, Y, y,
                                             nullptr, nullptr, st);
    else
      gemm_go<TagF16, 64, kEpiStore, false>(x, qweight, nullptr, scales, zeros, M, N, K, Y, y,
                                            nullptr, nullptr, st);
  } else {
    if (gs == 128)
      gemm_go<TagBF16, 128, kEpiStore, false>(x, qweight, nullptr, scales, zeros, M, N, K, Y, y,
                                              nullptr, nullptr, st);
    else
      gemm_go<TagBF16, 64, kEpiStore, false>(x, qweight, nullptr, scales, zeros, M, N, K, Y, y,
                                             nullptr, nullptr, st);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_dense_f32(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N,
                                 int64_t K, float *Y, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  gemm_go<TagF16, 128, kEpiStore, true>(X, nullptr, W, nullptr, nullptr, M, N, K, Y,
                                        (int)YType::F32, nullptr, nullptr, st);
  return hipGetLastError();
}

hipError_t launch_gemm_loss(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales,
                            const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int gs,
                            const float *Yref, double *partials, hipStream_t st) {
  if (gs == 128)
    gemm_go<TagF16, 128, kEpiLoss, false>(A, qweight, nullptr, scales, zeros, M, N, K, nullptr, 0,
                                          Yref, partials, st);
  else
    gemm_go<TagF16, 64, kEpiLoss, false>(A, qweight, nullptr, scales, zeros, M, N, K, nullptr, 0,
                                         Yref, partials, st);
  return hipGetLastError();
}

}  // namespace awq
