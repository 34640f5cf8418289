// Batched decode, 1 < M <= 64, on gfx950.
//
// The W4A16 layer for a small batch of rows ("AWQ Advanced Usage Guide",
// "WQLinear Kernel Variants": the GEMV variant serves decode, the GEMM variant
// larger batches; between the two, a batch of a few tokens is still bound by
// streaming the packed weights once).  Same arithmetic as the GEMV:
// Y[m][n] = sum_g s[n][g] * sum_{k in g} X[m][k] * (q[n][k] - z[n][g]), with
// the exact integer q - z as the MFMA operand, fp32 sums per group, the fp16
// group scale applied once per group sum.
//
// Design for MI355X.  The GEMV gives each workgroup 16 columns, so every
// workgroup reads all of X: at M = 16 that is 4 bytes of activations per byte
// of weights.  Here a workgroup owns 128 columns (8 waves, wave w: 16 of
// them, for all M rows) and a range of at most kMaxGroups groups of K (a
// split); the range's activations, scales and zero points are staged once in
// LDS and shared by the 8 waves, so X is read once per 128 columns.  The
// staging loads are issued first, with one barrier after them (a pipeline of
// several X chunks per workgroup, with a barrier each, measured slower: every
// chunk paid a latency of its own).  Each wave streams its packed weights
// with 48-64 bytes per lane in flight at M <= 16 and 32 above (the next
// groups' loads are issued as groups are consumed): measured 5-14% faster
// than issuing the whole range at once, bit-identical; windows of 2, 3, 6
// and 8 groups at g = 128 were no faster than 4.  Two workgroups fit a
// CU (at most 80 KiB of LDS and 128 VGPRs each); the split count balances
// the most loaded CU against the partials' cost.
// Splits of K write fp32 partials that a second kernel sums in split order
// (deterministic); a single split stores Y directly.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
}  // namespace

constexpr int kBgWaves = 8;                  // waves per workgroup: 128 columns

// Most groups per split (kMaxGroups): the range's activations (at most 64 KiB)
// stay in LDS.
template <int GS, int MT>
struct BgGeom {
  static constexpr int kRows = 16 * MT;                 // padded activation rows
  static constexpr int kMaxGroups = 2048 / GS / MT;
  // Groups of packed weights in flight per wave.  M <= 16: four (64 bytes
  // per lane) at g = 128, six (48 bytes) at g = 64.  Above M = 16: 32 bytes
  // per lane.  The kernel's REFILL is how many are requested at a time (see
  // bg_refill).
  static constexpr int kWinWant = MT == 1 ? (GS == 64 ? 6 : 4) : 2 * 128 / GS;
  static constexpr int kWin = kWinWant < kMaxGroups ? kWinWant : kMaxGroups;
  static constexpr int kKR = kMaxGroups * GS;            // K values of a full range
  static constexpr int kRowBytes = kKR * 2 + 16;         // +16: rows start 4 banks apart
  static constexpr int kXBytes = kRows * kRowBytes;
  static constexpr int kCols = 16 * kBgWaves;
  static constexpr int kSBytes = kCols * kMaxGroups * 2;  // scales, [col][group]
  static constexpr int kZBytes = kCols * kMaxGroups;      // zero points, [col][group]
  static constexpr int kBytes = kXBytes + kSBytes + kZBytes;
  static constexpr int kThreads = 64 * kBgWaves;
  static constexpr int kXPieces = kRows * (kKR / 8);      // 16-byte pieces of X
  static constexpr int kXLoads = (kXPieces + kThreads - 1) / kThreads;
  static constexpr int kSZLoads = (kCols * kMaxGroups + kThreads - 1) / kThreads;
};

// (four waves per SIMD: two workgroups per CU)
template <class XT, int GS, int MT, int REFILL>
__global__ __launch_bounds__(64 * kBgWaves) __attribute__((amdgpu_waves_per_eu(4, 8)))
void batched_gemv_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int gps, void *__restrict__ Y, int ytype, uint32_t zfix, float *__restrict__ partial) {
  using Geo = BgGeom<GS, MT>;
  constexpr int kWpl = GS / 32;            // packed words per lane per group
  constexpr int kMG = Geo::kMaxGroups;
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  const int G = K / GS;
  const int col0 = blockIdx.x * Geo::kCols;            // first column of the workgroup
  const int n = col0 + 16 * wave + c;                  // this lane's column
  const int split = blockIdx.y;
  const int g_begin = split * gps;                     // gps <= kMG (the plan's bound)
  const int g_end = g_begin + gps < G ? g_begin + gps : G;
  const int k_begin = g_begin * GS, k_end = g_end * GS;

  const rsrc_t rQ = make_rsrc(qweight, (uint32_t)N * (uint32_t)K / 2u);
  const rsrc_t rS = make_rsrc(scales, (uint32_t)N * (uint32_t)G * 2u);
  const rsrc_t rZ = make_rsrc(zeros, zeros ? (uint32_t)N * (uint32_t)G : 0u);
  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);

  // ---- staging loads first, then the first weight window ---------------------
  // Staging (registers, then LDS): X rows 0..kRows-1 over [k_begin, k_end)
  // (rows >= M and values past the range read 0), scales and zero points of
  // the 128 columns, [col][group] (columns >= N and groups past the range
  // read 0).
  u32x4 xs[Geo::kXLoads];
  uint32_t ss[Geo::kSZLoads], zs[Geo::kSZLoads];
#pragma unroll
  for (int r = 0; r < Geo::kXLoads; ++r) {
    const int e = tid + r * Geo::kThreads;
    const int row = e / (Geo::kKR / 8), piece = e % (Geo::kKR / 8);
    const int k = k_begin + piece * 8;
    const uint32_t o = (e < Geo::kXPieces && row < M && k < k_end)
                           ? ((uint32_t)row * (uint32_t)K + (uint32_t)k) * 2u : 0x7FFFFFF0u;
    xs[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, o, 0, 0));
  }
#pragma unroll
  for (int r = 0; r < Geo::kSZLoads; ++r) {
    const int e = tid + r * Geo::kThreads;
    const int col = e / kMG, gl = e % kMG;
    const int g = g_begin + gl;
    const uint32_t o = (e < Geo::kCols * kMG && col0 + col < N && g < g_end)
                           ? (uint32_t)(col0 + col) * (uint32_t)G + (uint32_t)g : 0x7FFFFFF0u;
    ss[r] = __builtin_amdgcn_raw_buffer_load_b16(rS, o * 2u, 0, 0);
    zs[r] = __builtin_amdgcn_raw_buffer_load_b8(rZ, o, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // packed weights of this lane, group gl of the range (groups past it read 0
  // and are not used); the first window now, the rest as groups are consumed
  const uint32_t q_lane = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  typedef uint32_t wvec_t __attribute__((ext_vector_type(kWpl)));
  wvec_t w[kMG];
  auto load_group = [&](int gl) {
    const int g = g_begin + gl;
    const uint32_t qo = g < g_end ? q_lane + (uint32_t)g * (GS / 2) : 0x7FFFFFF0u;
    if constexpr (kWpl == 4)
      w[gl] = __builtin_bit_cast(wvec_t, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
    else
      w[gl] = __builtin_bit_cast(wvec_t, __builtin_amdgcn_raw_buffer_load_b64(rQ, qo, 0, 0));
  };
#pragma unroll
  for (int gl = 0; gl < Geo::kWin; ++gl) load_group(gl);
  __builtin_amdgcn_sched_barrier(0);
  // the staging registers to LDS (the counted wait leaves the weight loads,
  // issued after them, in flight)
  uint16_t *sS = reinterpret_cast<uint16_t *>(smem + Geo::kXBytes);
  uint8_t *sZ = reinterpret_cast<uint8_t *>(smem + Geo::kXBytes + Geo::kSBytes);
#pragma unroll
  for (int r = 0; r < Geo::kXLoads; ++r) {
    const int e = tid + r * Geo::kThreads;
    if (e >= Geo::kXPieces) break;
    const int row = e / (Geo::kKR / 8), piece = e % (Geo::kKR / 8);
    *reinterpret_cast<u32x4 *>(smem + row * Geo::kRowBytes + piece * 16) = xs[r];
  }
#pragma unroll
  for (int r = 0; r < Geo::kSZLoads; ++r) {
    const int e = tid + r * Geo::kThreads;
    if (e >= Geo::kCols * kMG) break;
    sS[e] = (uint16_t)ss[r];
    sZ[e] = (uint8_t)zs[r];
  }
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const DeqRegs dq;
#pragma unroll
  for (int gl = 0; gl < kMG; ++gl) {
    if (gl % REFILL == 0 && gl + Geo::kWin < kMG) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < REFILL; ++u)
        if (gl + Geo::kWin + u < kMG) load_group(gl + Geo::kWin + u);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (a guarded body rather than an early exit: the loop stays fully
    // unrolled and w[] in registers)
    if (g_begin + gl >= g_end) continue;                // uniform
    const int sc_i = (16 * wave + c) * kMG + gl;
    const float sc = half_bits_to_float(sS[sc_i]);
    const DeqF16 deq((uint32_t)sZ[sc_i] + zfix);
    f32x4 t[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) t[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kWpl; ++j) {
      const uint32_t wj = w[gl][j];      // (scalar copy first, see DeqF16)
      const u32x4 h = deq(wj, dq);
      const u32x4 bop = kBF16 ? f16_pairs_to_bf16(h) : h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(
            smem + (16 * mt + c) * Geo::kRowBytes + (gl * GS + kq * kWpl * 8 + 8 * j) * 2);
        t[mt] = mfma32<XT>(a, bop, t[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mt][e] = __builtin_fmaf(t[mt][e], sc, acc[mt][e]);
  }

  if (n >= N) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mt + 4 * kq + e;
      if (m >= M) continue;
      const int64_t o = (int64_t)m * N + n;
      const float v = acc[mt][e];
      if (partial) {
        partial[(int64_t)split * M * N + o] = v;
      } else if (ytype == (int)YType::F16) {
        reinterpret_cast<uint16_t *>(Y)[o] = float_to_half_bits(v);
      } else if (ytype == (int)YType::BF16) {
        reinterpret_cast<uint16_t *>(Y)[o] = float_to_bf16_bits(v);
      } else {
        reinterpret_cast<float *>(Y)[o] = v;
      }
    }
  }
}

// Y[m][n] = sum over splits (in split order) of partial[split][m][n]; one
// thread per 4 consecutive outputs (16-byte partial loads: M * N is a
// multiple of 4 here), or per output when it is not.  The loads of up to
// eight splits are issued before their adds (a loop that added each split as
// it arrived waited for them one by one: 4.4 us for 4 splits of 16 x 13824).
template <int VEC>
__global__ __launch_bounds__(256) void batched_gemv_reduce_kernel(const float *__restrict__ partial,
                                                                  int splits, int64_t MN,
                                                                  void *__restrict__ Y, int ytype) {
  constexpr int kChunk = 8;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
  if (i >= MN) return;
  float v[VEC];
  for (int s0 = 0; s0 < splits; s0 += kChunk) {
    float p[kChunk][VEC];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (s0 + u >= splits) break;                     // uniform
      const float *src = partial + (int64_t)(s0 + u) * MN + i;
      if constexpr (VEC == 4) {
        const float4 q = *reinterpret_cast<const float4 *>(src);
        p[u][0] = q.x; p[u][1] = q.y; p[u][2] = q.z; p[u][3] = q.w;
      } else {
        p[u][0] = src[0];
      }
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (s0 + u >= splits) break;
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = s0 + u == 0 ? p[u][e] : v[e] + p[u][e];
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (ytype == (int)YType::F16)
      reinterpret_cast<uint16_t *>(Y)[i + e] = float_to_half_bits(v[e]);
    else if (ytype == (int)YType::BF16)
      reinterpret_cast<uint16_t *>(Y)[i + e] = float_to_bf16_bits(v[e]);
    else
      reinterpret_cast<float *>(Y)[i + e] = v[e];
  }
}

namespace {
int bg_mt(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }
int bg_max_groups(int gs, int mt) { return 2048 / gs / mt; }
size_t bg_lds(int gs, int mt) {
  const int mg = bg_max_groups(gs, mt), cols = 16 * kBgWaves;
  return (size_t)16 * mt * (mg * gs * 2 + 16) + (size_t)cols * mg * 3;
}
}  // namespace

bool batched_gemv_supported(int64_t M, int64_t N, int64_t K, int gs) {
  return M >= 1 && M <= 64 && N * K / 2 < 0x7FFFFFF0 && M * K * 2 < 0x7FFFFFF0 &&
         bg_lds(gs, bg_mt(M)) <= 80 * 1024;
}

BatchedPlan batched_gemv_plan(int64_t M, int64_t N, int64_t K, int gs, Scratch sc) {
  BatchedPlan p{};
  const int64_t G = K / gs;
  const int64_t mg = bg_max_groups(gs, bg_mt(M));
  const int64_t colblocks = (N + 16 * kBgWaves - 1) / (16 * kBgWaves);
  // At least G / mg splits (a split stages at most mg groups).  Among the
  // counts up to four workgroups per CU, the one that minimizes the most
  // loaded CU's groups (workgroups per CU, ceil(wgs / 256), times groups per
  // split), plus 1.1 groups' time per split (each adds a partial to write
  // and sum), plus 4 when the workgroups need a second residency round (more
  // than 512); ties to fewer splits.  Fitted to same-box sweeps of every
  // split count on 13824 x 5120, 5120 x 13824 (g = 64 and 128) and
  // 11008 x 4096 at M = 4..32: the pick is the best or within 0.5 us of it
  // (11008 x 4096: 2 splits, 2 us faster than filling every slot; 13824 x
  // 5120 at g = 64: 4, 2 us faster than 7).
  const int64_t s_min = (G + mg - 1) / mg;
  int64_t best = s_min;
  if (sc != Scratch::None) {
    int64_t s_max = 1024 / colblocks;
    if (s_max > G) s_max = G;
    double best_cost = 1e30;
    for (int64_t sp = s_min; sp <= (s_max > s_min ? s_max : s_min); ++sp) {
      const int64_t gps = (G + sp - 1) / sp;
      const int64_t wgs = colblocks * ((G + gps - 1) / gps);
      const double cost = (double)((wgs + 255) / 256 * gps) + 1.1 * (double)sp +
                          (wgs > 512 ? 4.0 : 0.0);
      if (cost < best_cost) {
        best_cost = cost;
        best = sp;
      }
    }
  }
  int64_t splits = best;
  for (;;) {
    const int64_t gps = (G + splits - 1) / splits;
    const int64_t s2 = (G + gps - 1) / gps;
    const size_t bytes = s2 > 1 ? (size_t)s2 * M * N * 4 : 0;
    if (sc == Scratch::Bounded && bytes > kBoundedPartialBytes && splits > s_min) {
      --splits;
      continue;
    }
    p.splits = (int)s2;
    p.gps = (int)gps;
    p.partial_bytes = bytes;
    break;
  }
  return p;
}

// Weight groups requested at a time.  Pairs make each column's refill one
// run of two groups: at g = 64 and M <= 32 (a 64-byte run instead of two
// 32-byte ones) measured 2-7% faster at M = 8 and 16 and 1-4% at M = 24 and
// 32 on 13B-class layers (no gain at M = 48), and no slower with an odd
// number of groups per split (13 or 11 on 7B-class layers, within 1%); at
// g = 128 and M <= 16, 1.5-5%
// faster where a split holds an even number of groups (10 or 16) and 1-3%
// slower where it holds an odd number (9 or 11), hence the choice by the
// plan's groups per split.  Same box, bit-identical either way.
template <int GS, int MT>
static int bg_refill(const BatchedPlan &p) {
  if (GS == 64 && MT <= 2) return 2;
  if (GS == 128 && MT == 1 && p.gps % 2 == 0) return 2;
  return 1;
}

template <class XT, int GS, int MT>
static hipError_t bg_go(const void *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                        int64_t M, int64_t N, int64_t K, void *Y, YType yt,
                        const BatchedPlan &p, float *partial, hipStream_t st) {
  using Geo = BgGeom<GS, MT>;
  const dim3 grid((unsigned)((N + Geo::kCols - 1) / Geo::kCols), (unsigned)p.splits);
  const uint32_t zfix = zr ? 0u : 8u;
  float *part = p.splits > 1 ? partial : nullptr;
  const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
  constexpr bool kPairs = (GS == 64 && MT <= 2) || (GS == 128 && MT == 1);
  if constexpr (kPairs) {
    if (bg_refill<GS, MT>(p) == 2)
      batched_gemv_kernel<XT, GS, MT, 2><<<grid, Geo::kThreads, Geo::kBytes, st>>>(
          x, qw, sc, zr, (int)M, (int)N, (int)K, p.gps, Y, (int)yt, zfix, part);
    else
      batched_gemv_kernel<XT, GS, MT, 1><<<grid, Geo::kThreads, Geo::kBytes, st>>>(
          x, qw, sc, zr, (int)M, (int)N, (int)K, p.gps, Y, (int)yt, zfix, part);
  } else {
    batched_gemv_kernel<XT, GS, MT, 1><<<grid, Geo::kThreads, Geo::kBytes, st>>>(
        x, qw, sc, zr, (int)M, (int)N, (int)K, p.gps, Y, (int)yt, zfix, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t MN = M * N;
  if (MN % 4 == 0)
    batched_gemv_reduce_kernel<4><<<(unsigned)((MN / 4 + 255) / 256), 256, 0, st>>>(
        partial, p.splits, MN, Y, (int)yt);
  else
    batched_gemv_reduce_kernel<1><<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(
        partial, p.splits, MN, Y, (int)yt);
  return hipGetLastError();
}

template <class XT, int GS>
static hipError_t bg_mt_go(const void *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                           int64_t M, int64_t N, int64_t K, void *Y, YType yt,
                           const BatchedPlan &p, float *partial, hipStream_t st) {
  switch (bg_mt(M)) {
    case 1: return bg_go<XT, GS, 1>(X, qw, sc, zr, M, N, K, Y, yt, p, partial, st);
    case 2: return bg_go<XT, GS, 2>(X, qw, sc, zr, M, N, K, Y, yt, p, partial, st);
    default: return bg_go<XT, GS, 4>(X, qw, sc, zr, M, N, K, Y, yt, p, partial, st);
  }
}

hipError_t launch_batched_gemv(const void *X, XType xt, const uint32_t *qweight,
                               const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                               int64_t K, int gs, void *Y, YType yt, const BatchedPlan &plan,
                               void *workspace, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  float *partial = reinterpret_cast<float *>(workspace);
  if (xt == XType::F16) {
    if (gs == 128) return bg_mt_go<TagF16, 128>(X, qweight, scales, zeros, M, N, K, Y, yt, plan, partial, st);
    return bg_mt_go<TagF16, 64>(X, qweight, scales, zeros, M, N, K, Y, yt, plan, partial, st);
  }
  if (gs == 128) return bg_mt_go<TagBF16, 128>(X, qweight, scales, zeros, M, N, K, Y, yt, plan, partial, st);
  return bg_mt_go<TagBF16, 64>(X, qweight, scales, zeros, M, N, K, Y, yt, plan, partial, st);
}

}  // namespace awq
