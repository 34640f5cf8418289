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

namespace {
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
}  // namespace

// Largest 16*G the kernel stages (scale/zero elements of one workgroup).
constexpr int kGemvMaxSZ = 4096;
// Activations are staged in LDS when their M rows fit the budget: 64 KiB for
// 8-wave workgroups (at most 80 KiB of LDS each, two per CU), 128 KiB for
// 16-wave workgroups (grids of at most 256 workgroups, one per CU, which
// then owns the CU's 160 KiB of LDS).  Larger M*K streams them from global
// memory instead.
constexpr uint32_t kGemvStageBytes = 64u * 1024u;
constexpr uint32_t kGemvStageBytesSolo = 128u * 1024u;
// Waves per workgroup for N output columns (see gemv_dispatch).
__host__ __device__ constexpr int gemv_waves(int64_t N) { return (N + 15) / 16 <= 256 ? 16 : 8; }
__host__ __device__ constexpr uint32_t gemv_stage_budget(int nw) {
  return nw == 16 ? kGemvStageBytesSolo : kGemvStageBytes;
}

// LDS layout (dynamic shared memory, byte offsets; every region starts on a
// 1 KiB boundary):
//   [0, xbytes)              activation rows 0..M-1 (when staged)
//   [soff, ...)              scales of the 16 columns, fp16 bits, [16][G]
//   [zoff, ...)              zero points of the 16 columns, u8, [16][G]
// The cross-wave reduction reuses the start of the buffer after the loop.

struct GemvSmem {
  uint32_t xrow;     // bytes per activation row (K * 2)
  uint32_t soff, zoff, total;
};

__host__ __device__ inline uint32_t kib_up(uint32_t b) { return (b + 1023u) & ~1023u; }

__host__ __device__ inline GemvSmem gemv_smem(int M, int K, int G, bool stage_x) {
  GemvSmem L;
  L.xrow = (uint32_t)K * 2u;
  L.soff = stage_x ? kib_up(L.xrow * (uint32_t)M) : 0u;
  L.zoff = L.soff + kib_up(32u * (uint32_t)G);
  L.total = L.zoff + kib_up(16u * (uint32_t)G);
  return L;
}

// Memory instructions are the scarce resource here (each one occupies the
// CU's address unit for tens of cycles), so per group a wave issues exactly
// one: the 16-byte packed-weight load of each lane.  Activations (staged by
// the workgroup once when M*K*2 fits the LDS budget), scales and zero points
// come from LDS.  All global reads use buffer resources, so rows
// >= M, columns >= N and groups >= G read zero without branches.
template <class XT, int GS, int NW, int U, bool STAGE_X>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    void *__restrict__ Y, int ytype) {
  constexpr int kWpl = GS / 32;            // packed words per lane per group
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;
  const int kq = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + c;
  const int G = K / GS;
  const GemvSmem L = gemv_smem(M, K, G, STAGE_X);

  const rsrc_t rQ = make_rsrc(qweight, (uint32_t)N * (uint32_t)K / 2u);
  const rsrc_t rS = make_rsrc(scales, (uint32_t)N * (uint32_t)G * 2u);
  const rsrc_t rZ = make_rsrc(zeros, (uint32_t)N * (uint32_t)G);
  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);

  const uint32_t q_lane = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  const uint32_t x_lane = (uint32_t)c * (uint32_t)K * 2u + (uint32_t)(kq * kWpl * 16);
  struct Batch {
    uint32_t raw[U][kWpl];
    u32x4 a[U][kWpl];      // used only when activations are not staged
  };
  // Packed weights (and, without staging, activations) of groups
  // g0, g0 + NW, ..., g0 + (U-1)*NW.  No load is issued for a group past the
  // end (g is uniform across the wave, so this is a scalar branch): its
  // registers keep stale values, which the zero scale of such a group cancels.
  auto load_batch = [&](int g0, Batch &b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NW;
      if (g >= G) continue;
      const uint32_t qo = q_lane + (uint32_t)g * (GS / 2);
      if constexpr (kWpl == 4) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
#pragma unroll
        for (int j = 0; j < kWpl; ++j) b.raw[u][j] = v[j];
      } else {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rQ, qo, 0, 0));
#pragma unroll
        for (int j = 0; j < kWpl; ++j) b.raw[u][j] = v[j];
      }
      if constexpr (!STAGE_X) {
        const uint32_t xo = x_lane + (uint32_t)g * (GS * 2);
#pragma unroll
        for (int j = 0; j < kWpl; ++j)
          b.a[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, xo + 16u * j, 0, 0));
      }
    }
  };

  // ---- prologue ---------------------------------------------------------------
  // Staging loads are issued before the weight stream: issued after it, they
  // would queue behind every CU's weight traffic and the barrier below would
  // hold all math until the stream had drained.  They go to registers and
  // are written to LDS once the first weight batch is in flight, so the
  // barrier waits for the staging loads only (counted vmcnt), not for that
  // batch (an LDS DMA could only be waited for with vmcnt(0)):
  //  * activation rows, 16 bytes per thread and round (M*K*2 is a multiple
  //    of 128 bytes, so no chunk straddles the end of X);
  //  * scales and zero points of the 16 columns ([16][G], contiguous),
  //    element by element (a 16-byte chunk could straddle the end of those
  //    arrays, where the range check would zero it).
  constexpr int kSZ = kGemvMaxSZ / (64 * NW);   // scale/zero elements per thread
  constexpr int kXR = STAGE_X ? gemv_stage_budget(NW) / (64 * NW * 16) : 1;   // X chunks per thread
  const int nsz = (16 * G + 64 * NW - 1) / (64 * NW);   // uniform: rounds needed
  const uint32_t xbytes = STAGE_X ? (uint32_t)M * L.xrow : 0u;
  const int nxr = (int)((xbytes + 64u * NW * 16u - 1u) / (64u * NW * 16u));
  uint32_t sreg[kSZ], zreg[kSZ];
  u32x4 xreg[kXR];
  {
    const uint32_t base = (uint32_t)n0 * (uint32_t)G;
#pragma unroll
    for (int r = 0; r < kSZ; ++r) {
      if (r >= nsz) break;
      const uint32_t i = (uint32_t)(tid + r * 64 * NW);
      const uint32_t o = i < 16u * (uint32_t)G ? base + i : 0x7FFFFFF0u;
      sreg[r] = __builtin_amdgcn_raw_buffer_load_b16(rS, o * 2u, 0, 0);
      zreg[r] = __builtin_amdgcn_raw_buffer_load_b8(rZ, o, 0, 0);
    }
    if constexpr (STAGE_X) {
#pragma unroll
      for (int r = 0; r < kXR; ++r) {
        if (r >= nxr) break;
        const uint32_t o = (uint32_t)(tid + r * 64 * NW) * 16u;
        xreg[r] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, o < xbytes ? o : 0x7FFFFFF0u, 0, 0));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // First batch of packed weights, behind the staging loads.
  Batch cur, nxt;
  load_batch(wave, cur);
  __builtin_amdgcn_sched_barrier(0);
  {
    uint16_t *ss = reinterpret_cast<uint16_t *>(smem + L.soff);
    uint8_t *zs = reinterpret_cast<uint8_t *>(smem + L.zoff);
#pragma unroll
    for (int r = 0; r < kSZ; ++r) {
      if (r >= nsz) break;
      const int i = tid + r * 64 * NW;
      if (i < 16 * G) {
        ss[i] = (uint16_t)sreg[r];
        zs[i] = (uint8_t)zreg[r];
      }
    }
    if constexpr (STAGE_X) {
#pragma unroll
      for (int r = 0; r < kXR; ++r) {
        if (r >= nxr) break;
        const uint32_t o = (uint32_t)(tid + r * 64 * NW) * 16u;
        if (o < xbytes) *reinterpret_cast<u32x4 *>(smem + o) = xreg[r];
      }
    }
  }
  __syncthreads();

  // Activation row of this lane as the A operand: row c, or row 0 for the
  // padding rows c >= M.  Row m of the MFMA result depends on row m of A
  // alone, and result rows >= M are never stored, so the padding rows may
  // hold any values.
  const char *xlds = smem + (c < M ? (uint32_t)c * L.xrow : 0u) + (uint32_t)(kq * kWpl * 16);
  const uint16_t *ss = reinterpret_cast<const uint16_t *>(smem + L.soff) + c * G;
  const uint8_t *zs = reinterpret_cast<const uint8_t *>(smem + L.zoff) + c * G;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const DeqRegs dq;

  // Software pipeline: the next batch's loads are in flight while this batch
  // is dequantized and multiplied.
  for (int g0 = wave; g0 < G; g0 += NW * U) {
    load_batch(g0 + NW * U, nxt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NW;
      const int gs = g < G ? g : G - 1;
      u32x4 a[kWpl];
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        if constexpr (STAGE_X)
          a[j] = *reinterpret_cast<const u32x4 *>(xlds + (uint32_t)gs * (GS * 2) + 16u * j);
        else  // a group past the end loaded nothing: its stale registers may hold any bits
          a[j] = g < G ? cur.a[u][j] : u32x4{0u, 0u, 0u, 0u};
      }
      const uint32_t zr = zs[gs];
      const uint16_t sb = ss[gs];
      const float sc = g < G ? half_bits_to_float(sb) : 0.0f;
      // Biased codes times a, plus a times the bias-and-zero correction: two
      // independent MFMA chains, summed once per group.
      const u32x4 corr = kBF16 ? corr_bf16(zr) : corr_f16(zr);
      f32x4 t = {0.f, 0.f, 0.f, 0.f}, tc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        const u32x4 b = kBF16 ? deq_bf16_biased(cur.raw[u][j], dq) : deq_f16_biased(cur.raw[u][j], dq);
        t = mfma32<XT>(a[j], b, t);
        tc = mfma32<XT>(a[j], corr, tc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(t[e] + tc[e], sc, acc[e]);
    }
    cur = nxt;
  }

  __syncthreads();
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = red[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const f32x4 o = red[w * 64 + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += o[e];
  }
  if (n >= N) return;
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


template <class XT, int GS, int NW>
static void gemv_launch(const uint16_t *X, const uint32_t *qw, const uint16_t *sc,
                        const uint8_t *zr, int M, int64_t N, int64_t K, void *Y, YType yt,
                        hipStream_t st) {
  const dim3 grid((unsigned)((N + 15) / 16));
  const int G = (int)(K / GS);
  const bool stage = (uint64_t)M * (uint64_t)K * 2u <= gemv_stage_budget(NW);
  const GemvSmem L = gemv_smem(M, (int)K, G, stage);
  // the reduction reuses the buffer: at least NW * 64 * 16 bytes
  const uint32_t bytes = L.total > 64u * NW * 16u ? L.total : 64u * NW * 16u;
  // Two batches in flight once a wave walks more than 8 groups (measured 7%
  // faster at 13.5 groups per wave, slower at 5 and below).
  if (stage && G > 8 * NW)
    gemv_kernel<XT, GS, NW, 2, true><<<grid, 64 * NW, bytes, st>>>(X, qw, sc, zr, M, (int)N,
                                                                   (int)K, Y, (int)yt);
  else if (stage)
    gemv_kernel<XT, GS, NW, 1, true><<<grid, 64 * NW, bytes, st>>>(X, qw, sc, zr, M, (int)N,
                                                                   (int)K, Y, (int)yt);
  else
    gemv_kernel<XT, GS, NW, 2, false><<<grid, 64 * NW, bytes, st>>>(X, qw, sc, zr, M, (int)N,
                                                                    (int)K, Y, (int)yt);
}

// Waves per workgroup.  Every workgroup of a launch should be resident at
// once (a second partial round of workgroups costs a whole extra memory
// latency): with at most one workgroup per CU (N <= 16 * 256) the workgroup
// takes 16 waves, otherwise 8.  One group per wave is in flight ahead of the
// one being computed: deeper windows were measured slower on MI355X (every
// wave's staging loads then queue behind more weight traffic).
template <class XT, int GS>
static void gemv_dispatch(const uint16_t *X, const uint32_t *qw, const uint16_t *sc,
                          const uint8_t *zr, int M, int64_t N, int64_t K, void *Y, YType yt,
                          hipStream_t st) {
  if (gemv_waves(N) == 16)
    gemv_launch<XT, GS, 16>(X, qw, sc, zr, M, N, K, Y, yt, st);
  else
    gemv_launch<XT, GS, 8>(X, qw, sc, zr, M, N, K, Y, yt, st);
}

int64_t gemv_groups_per_wave(int64_t N, int64_t K, int gs) {
  return (K / gs) / gemv_waves(N);
}

bool gemv_stages_activations(int64_t M, int64_t N, int64_t K) {
  return (uint64_t)M * (uint64_t)K * 2u <= gemv_stage_budget(gemv_waves(N));
}

bool gemv_supported(int64_t M, int64_t N, int64_t K, int gs) {
  const int64_t G = K / gs;
  const bool stage = gemv_stages_activations(M, N, K);
  const GemvSmem L = gemv_smem((int)M, (int)K, (int)G, stage);
  const uint32_t lds = gemv_waves(N) == 16 ? 160u * 1024u : 80u * 1024u;
  return M <= 16 && 16 * G <= kGemvMaxSZ && L.total <= lds;
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
