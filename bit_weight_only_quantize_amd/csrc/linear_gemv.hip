// Decode GEMV / skinny GEMM for M <= 16 on gfx950.
//
// The W4A16 linear layer for single-token and small-batch decode ("AWQ
// Advanced Usage Guide", "WQLinear Kernel Variants": the GEMV variant serves
// single-token generation).  Y[m][n] = sum_g s[n][g] * sum_{k in g} X[m][k] *
// (q[n][k] - z[n][g]), fp32 accumulation.
//
// Design for MI355X: the layer is bound by streaming the packed weights from
// HBM once (0.5 byte per weight + 3 bytes per group).  Each workgroup owns 16
// output columns; its waves split the groups of K between them (wave w takes
// groups w, w + NW, ...), so neighbouring waves read neighbouring 64-byte
// halves of the same 128-byte lines.  Within a wave, lane (c = l & 15,
// kq = l >> 4) reads 16 bytes (32 codes) of column c per group and the
// contraction runs on the 16x16x32 MFMA with the activation rows padded to
// 16: the matrix core does the multiply-adds, leaving the VALU only the
// dequantization (about 9 instructions per 8 weights).  The per-group scale is
// applied to the fp32 partial of each group, so the B operand is the exact
// integer q - z and no rounding of dequantized weights ever happens.
// Partials of the NW waves are combined through LDS in a fixed order.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

template <class XT, int GS, int NW, int U>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M,
    int64_t N, int64_t K, void *__restrict__ Y, int ytype) {
  constexpr int kWpl = GS / 32;            // packed words per lane per group
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int kq = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * 16 + c;
  const bool nvalid = n < N;
  const int64_t G = K / GS;
  const int64_t wrow = K / 8;
  const bool mvalid = c < M;               // A-operand row of this lane

  const uint32_t *wp = qweight + (nvalid ? n : 0) * wrow + kq * kWpl;
  const uint16_t *sp = scales + (nvalid ? n : 0) * G;
  const uint8_t *zp = zeros + (nvalid ? n : 0) * G;
  const uint16_t *xp = X + (int64_t)(mvalid ? c : 0) * K + kq * 8 * kWpl;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int64_t g0 = wave; g0 < G; g0 += (int64_t)NW * U) {
    uint32_t raw[U][kWpl];
    u32x4 a[U][kWpl];
    float sc[U];
    uint32_t zr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + (int64_t)u * NW;
      const bool gv = g < G;
      if (kWpl == 4) {
        u32x4 r = {0u, 0u, 0u, 0u};
        if (gv && nvalid) r = *reinterpret_cast<const u32x4 *>(wp + g * (GS / 8));
#pragma unroll
        for (int j = 0; j < kWpl; ++j) raw[u][j] = r[j];
      } else {
        u32x2 r = {0u, 0u};
        if (gv && nvalid) r = *reinterpret_cast<const u32x2 *>(wp + g * (GS / 8));
#pragma unroll
        for (int j = 0; j < kWpl; ++j) raw[u][j] = r[j];
      }
      sc[u] = (gv && nvalid) ? half_bits_to_float(sp[g]) : 0.0f;
      zr[u] = (gv && nvalid) ? (uint32_t)zp[g] : 0u;
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (gv && mvalid) x = *reinterpret_cast<const u32x4 *>(xp + g * GS + 8 * j);
        a[u][j] = x;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!kBF16) {
        const DeqF16 deq(zr[u]);
#pragma unroll
        for (int j = 0; j < kWpl; ++j) t = mfma32<TagF16>(a[u][j], deq(raw[u][j]), t);
      } else {
        const DeqBF16 deq;
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kWpl; ++j) {
          t = mfma32<TagBF16>(a[u][j], deq(raw[u][j]), t);
          r = mfma32<TagBF16>(a[u][j], bf16_ones(), r);
        }
        const float cz = -(float)(128u + zr[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = __builtin_fmaf(cz, r[e], t[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(t[e], sc[u], acc[e]);
    }
  }

  __shared__ f32x4 red[NW][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const f32x4 o = red[w][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += o[e];
  }
  if (!nvalid) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * kq + e;
    if (m >= M) continue;
    const int64_t o = (int64_t)m * N + n;
    if (ytype == (int)YType::F16)
      reinterpret_cast<uint16_t *>(Y)[o] = float_to_half_bits(sum[e]);
    else if (ytype == (int)YType::BF16)
      reinterpret_cast<uint16_t *>(Y)[o] = float_to_bf16_bits(sum[e]);
    else
      reinterpret_cast<float *>(Y)[o] = sum[e];
  }
}

template <class XT, int GS>
static void gemv_dispatch(const uint16_t *X, const uint32_t *qw, const uint16_t *sc,
                          const uint8_t *zr, int M, int64_t N, int64_t K, void *Y, YType yt,
                          hipStream_t st) {
  constexpr int NW = 8, U = 4;
  const dim3 grid((unsigned)((N + 15) / 16));
  gemv_kernel<XT, GS, NW, U><<<grid, 64 * NW, 0, st>>>(X, qw, sc, zr, M, N, K, Y, (int)yt);
}

hipError_t launch_gemv(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
  if (xt == XType::F16) {
    if (gs == 128) gemv_dispatch<TagF16, 128>(x, qweight, scales, zeros, (int)M, N, K, Y, yt, st);
    else gemv_dispatch<TagF16, 64>(x, qweight, scales, zeros, (int)M, N, K, Y, yt, st);
  } else {
    if (gs == 128) gemv_dispatch<TagBF16, 128>(x, qweight, scales, zeros, (int)M, N, K, Y, yt, st);
    else gemv_dispatch<TagBF16, 64>(x, qweight, scales, zeros, (int)M, N, K, Y, yt, st);
  }
  return hipGetLastError();
}

}  // namespace awq
