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
// dequantization (9 instructions per 8 weights for fp16 activations, 21 for
// bf16).  The B operand is the exact integer q - z, so every product
// a * (q - z) is exact in fp32 and the only roundings are those of the fp32
// sums; the group's fp16 scale multiplies the fp32 sum of each group once.
// No dequantized weight is ever rounded.  Partials of the NW waves are
// combined through LDS in a fixed order.

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
// Waves per workgroup for a grid of column tiles (see gemv_dispatch).
__host__ __device__ constexpr int gemv_waves_for_tiles(int64_t tiles) { return tiles <= 256 ? 16 : 8; }
__host__ __device__ constexpr int gemv_waves(int64_t N) { return gemv_waves_for_tiles((N + 15) / 16); }
__host__ __device__ constexpr uint32_t gemv_stage_budget(int nw) {
  return nw == 16 ? kGemvStageBytesSolo : kGemvStageBytes;
}
// LDS a workgroup may take: the CU's 160 KiB alone, or 80 KiB two per CU.
__host__ __device__ constexpr uint32_t gemv_lds_cap(int nw) { return nw == 16 ? 160u * 1024u : 80u * 1024u; }

// LDS layout (dynamic shared memory, byte offsets; every region starts on a
// 1 KiB boundary):
//   [0, xbytes)              activation rows 0..M-1 (when staged)
//   [soff[i], ...)           scales of the 16 columns of weight set i, fp16 bits, [16][G]
//   [zoff[i], ...)           zero points of those columns, u8, [16][G]
//   [total, ...)             cross-wave partials, [NP][M][16] outputs x (NW + 4) floats,
//                            when they fit; else they reuse the start of the buffer

struct GemvSmem {
  uint32_t xrow;     // bytes per activation row (K * 2)
  uint32_t soff[2], zoff[2], total;
};

__host__ __device__ inline uint32_t kib_up(uint32_t b) { return (b + 1023u) & ~1023u; }

// np weight sets per workgroup (2: the gate/up pair of awq_linear_fused).
__host__ __device__ inline GemvSmem gemv_smem(int M, int K, int G, bool stage_x, int np) {
  GemvSmem L;
  L.xrow = (uint32_t)K * 2u;
  uint32_t off = stage_x ? kib_up(L.xrow * (uint32_t)M) : 0u;
  for (int i = 0; i < 2; ++i) {
    L.soff[i] = off;
    if (i < np) off += kib_up(32u * (uint32_t)G);
    L.zoff[i] = off;
    if (i < np) off += kib_up(16u * (uint32_t)G);
  }
  L.total = off;
  return L;
}

// The weight sets of one launch ("AWQ Advanced Usage Guide", "Layer Fusion":
// projections that share an input, such as Q, K and V, run as one launch).
// Workgroup b serves 16 columns of part p, where tile_end[p-1] <= b <
// tile_end[p] (cumulative 16-column tiles).  In the paired mode (NP = 2) the
// workgroups tile part 0 and each serves the same 16 columns of parts 0 and 1
// (gate and up), and stores silu(gate) * up.
constexpr int kGemvMaxParts = 4;
struct GemvParts {
  const uint32_t *qw[kGemvMaxParts];
  const uint16_t *sc[kGemvMaxParts];
  const uint8_t *zr[kGemvMaxParts];
  void *y[kGemvMaxParts];
  int n[kGemvMaxParts];
  int tile_end[kGemvMaxParts];
  int count;
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Memory instructions are the scarce resource here (each one occupies the
// CU's address unit for tens of cycles), so per group a wave issues exactly
// one per weight set: the 16-byte packed-weight load of each lane.
// Activations (staged by the workgroup once when M*K*2 fits the LDS budget),
// scales and zero points come from LDS.  All global reads use buffer
// resources, so rows >= M, columns >= N and groups >= G read zero without
// branches.
//
// MULTI: more than one part (a single part reads its pointers at fixed
// argument offsets, with no dependent lookup before the first load).
// SMALL: the staging needs at most two activation rounds and one scale/zero
// round; the staging loops then unroll to that, not to the LDS budget's
// maximum (8 rounds), and the kernel's code shrinks by up to a third
// (measured 0.1-0.3 us per launch on the decode layers).
template <class XT, int GS, int NW, int U, bool STAGE_X, int NP, bool MULTI, bool SMALL>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const uint16_t *__restrict__ X,
                                                       GemvParts parts, int M, int K, int ytype,
                                                       uint32_t zfix) {
  constexpr int kWpl = GS / 32;            // packed words per lane per group
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;
  const int kq = lane >> 4;
  // this workgroup's part and column tile (uniform)
  int part = 0;
  if constexpr (NP == 1 && MULTI) {
    while (part + 1 < parts.count && (int)blockIdx.x >= parts.tile_end[part]) ++part;
  }
  const int tile = (int)blockIdx.x - (part ? parts.tile_end[part - 1] : 0);
  const int N = parts.n[part];
  // read the output pointer with the other arguments: left to its use after
  // the reduction, its argument load was measured to cost 2-5% per launch
  void *const Y = parts.y[part];
  asm volatile("" : : "s"(Y));
  const int n0 = tile * 16;
  const int n = n0 + c;
  const int G = K / GS;
  const GemvSmem L = gemv_smem(M, K, G, STAGE_X, NP);

  rsrc_t rQ[NP], rS[NP], rZ[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    rQ[i] = make_rsrc(parts.qw[part + i], (uint32_t)N * (uint32_t)K / 2u);
    rS[i] = make_rsrc(parts.sc[part + i], (uint32_t)N * (uint32_t)G * 2u);
    // no zeros (the symmetric grid): every load reads 0 and zfix = 8 is added
    rZ[i] = make_rsrc(parts.zr[part + i], parts.zr[part + i] ? (uint32_t)N * (uint32_t)G : 0u);
  }
  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);

  const uint32_t q_lane = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  const uint32_t x_lane = (uint32_t)c * (uint32_t)K * 2u + (uint32_t)(kq * kWpl * 16);
  struct Batch {
    uint32_t raw[NP][U][kWpl];
    u32x4 a[U][kWpl];      // used only when activations are not staged
  };
  // Packed weights (and, without staging, activations) of groups
  // g0, g0 + NW, ..., g0 + (U-1)*NW.  Every batch issues the same number of
  // load instructions: a group past the end loads from an offset beyond every
  // buffer, which the range check turns into zeros without a memory access
  // (and the zero scale of such a group cancels whatever it computes).  A
  // fixed count lets every wait for a batch be a counted vmcnt that leaves
  // the next batch in flight; a conditional load between a load and its use
  // makes the compiler wait for all loads instead.
  // Packed weights with the non-temporal hint when the workgroup owns its CU
  // (16 waves, at most 256 column tiles): 2-4% faster on those layers at
  // M = 1 and 4, while on layers of 688 and more workgroups the hint measured
  // 4-14% slower.
  constexpr int kWAux = NW == 16 ? 2 : 0;   // buffer cache policy: nt
  auto load_batch = [&](int g0, Batch &b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NW;
      const uint32_t qo = g < G ? q_lane + (uint32_t)g * (GS / 2) : 0x7FFFFFF0u;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if constexpr (kWpl == 4) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ[i], qo, 0, kWAux));
#pragma unroll
          for (int j = 0; j < kWpl; ++j) b.raw[i][u][j] = v[j];
        } else {
          const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rQ[i], qo, 0, kWAux));
#pragma unroll
          for (int j = 0; j < kWpl; ++j) b.raw[i][u][j] = v[j];
        }
      }
      if constexpr (!STAGE_X) {
        const uint32_t xo = g < G ? x_lane + (uint32_t)g * (GS * 2) : 0x7FFFFFF0u - 16u * kWpl;
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
  //    of 128 bytes, so no chunk straddles the end of X); in a 16-wave
  //    workgroup a wave whose chunks all lie past the end issues no load (in
  //    the 8-wave kernel that skip made the compiler copy the staging
  //    registers, and wait for their loads, before the first weight load);
  //  * scales ([16][G] fp16, 32*G bytes) and zero points ([16][G] u8, 16*G
  //    bytes) of the 16 columns, both contiguous.
  // Every load instruction occupies the CU's address unit for the same ~16
  // clocks whatever its width.  A 16-wave workgroup owns its CU, and its
  // staging took 48-96 instructions element by element against 32-88 for
  // its weights; it loads scales and zero points in 16-byte chunks instead
  // (measured 0.2-0.5 us faster per layer).  8-wave workgroups share a CU
  // two or three at a time, and there the 16-byte chunks measured 0.1-0.3 us
  // slower per launch (4096 x 11008), so they keep one element per lane,
  // except the gate/up pair in the compact variant (two weight sets to
  // stage: 12.05 -> 11.59 us on 2 x 11008 x 4096 at M = 1).
  constexpr bool kVecSZ = NW == 16 || (SMALL && NP == 2);
  constexpr int kXR = !STAGE_X ? 1 : SMALL ? 2 : gemv_stage_budget(NW) / (64 * NW * 16);   // X chunks per thread
  const uint32_t xbytes = STAGE_X ? (uint32_t)M * L.xrow : 0u;
  const int nxr = (int)((xbytes + 64u * NW * 16u - 1u) / (64u * NW * 16u));
  u32x4 xreg[kXR];
  // 16-byte chunks (16-wave workgroups).  The tile starts at element
  // 16*tile*G, so both blocks are 16-byte aligned.  A chunk across the end of
  // the arrays would read as zero under the range check; that happens only
  // in a partial last tile with N*G not a multiple of 16, which stages
  // element by element after the first weight batch instead.  The chunks are
  // dealt out in wave-sized slots (slot v = wave + r * NW), each segment
  // starting on a slot boundary, so every load instruction reads one array
  // (a uniform buffer resource): per weight set, ceil(2G/64) slots of
  // scales, then ceil(G/64) of zero points.
  const int ws = (2 * G + 63) / 64, wz = (G + 63) / 64;
  const bool sz_vec = kVecSZ && (n0 + 16 <= N || ((N * G) & 15) == 0);
  constexpr int kSZV = kVecSZ && !SMALL ? (NP * (kGemvMaxSZ / 512 + kGemvMaxSZ / 1024) + NW - 1) / NW : 1;
  const int nslots = NP * (ws + wz);
  // slot v (uniform): weight set, array, and the byte offsets of this lane's
  // chunk in global memory (beyond every buffer when past the segment) and LDS
  auto sz_slot = [&](int v, int &set, bool &is_zero, uint32_t &gofs, uint32_t &lofs) {
    set = v >= ws + wz ? 1 : 0;
    const int u = v - set * (ws + wz);
    is_zero = u >= ws;
    const int j = (is_zero ? u - ws : u) * 64 + lane;
    gofs = j < (is_zero ? G : 2 * G)
               ? (uint32_t)n0 * (uint32_t)G * (is_zero ? 1u : 2u) + 16u * (uint32_t)j : 0x7FFFFFF0u;
    // arithmetic on the layout of gemv_smem, not an index into L: a runtime
    // index puts L in scratch memory, whose load waits for every load in flight
    const uint32_t sbytes = kib_up(32u * (uint32_t)G), zbytes = kib_up(16u * (uint32_t)G);
    lofs = L.soff[0] + (uint32_t)set * (sbytes + zbytes) + (is_zero ? sbytes : 0u) + 16u * (uint32_t)j;
  };
  u32x4 szreg[kSZV];
  // One element per lane (8-wave workgroups).
  constexpr int kSZ = kVecSZ || SMALL ? 1 : kGemvMaxSZ / (64 * NW);   // scale/zero elements per thread
  const int nsz = (16 * G + 64 * NW - 1) / (64 * NW);         // uniform: rounds needed
  uint32_t sreg[NP][kSZ], zreg[NP][kSZ];
  if constexpr (kVecSZ) {
    if (__builtin_expect(sz_vec, 1)) {
#pragma unroll
      for (int r = 0; r < kSZV; ++r) {
        const int v = wave + r * NW;
        if (v >= nslots) break;
        int set;
        bool z;
        uint32_t go, lo;
        sz_slot(v, set, z, go, lo);
        const rsrc_t rr = z ? (set ? rZ[NP - 1] : rZ[0]) : (set ? rS[NP - 1] : rS[0]);
        szreg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, go, 0, 0));
      }
    }
  } else {
    const uint32_t base = (uint32_t)n0 * (uint32_t)G;
#pragma unroll
    for (int r = 0; r < kSZ; ++r) {
      if (r >= nsz) break;
      const uint32_t i = (uint32_t)(tid + r * 64 * NW);
      const uint32_t o = i < 16u * (uint32_t)G ? base + i : 0x7FFFFFF0u;
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        sreg[s][r] = __builtin_amdgcn_raw_buffer_load_b16(rS[s], o * 2u, 0, 0);
        zreg[s][r] = __builtin_amdgcn_raw_buffer_load_b8(rZ[s], o, 0, 0);
      }
    }
  }
  if constexpr (STAGE_X) {
#pragma unroll
    for (int r = 0; r < kXR; ++r) {
      if (r >= nxr || (kVecSZ && (uint32_t)(wave * 64 + r * 64 * NW) * 16u >= xbytes)) break;
      const uint32_t o = (uint32_t)(tid + r * 64 * NW) * 16u;
      xreg[r] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, o < xbytes ? o : 0x7FFFFFF0u, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // First batch of packed weights, behind the staging loads.
  Batch bA, bB;
  load_batch(wave, bA);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kVecSZ) {
    if (__builtin_expect(sz_vec, 1)) {
#pragma unroll
      for (int r = 0; r < kSZV; ++r) {
        const int v = wave + r * NW;
        if (v >= nslots) break;
        int set;
        bool z;
        uint32_t go, lo;
        sz_slot(v, set, z, go, lo);
        if (go != 0x7FFFFFF0u) *reinterpret_cast<u32x4 *>(smem + lo) = szreg[r];
      }
    } else {
      // partial last tile with a chunk across the end of the arrays
      const uint32_t base = (uint32_t)n0 * (uint32_t)G;
      for (int i = tid; i < 16 * G; i += 64 * NW) {
        const uint32_t o = base + (uint32_t)i;
#pragma unroll
        for (int s = 0; s < NP; ++s) {
          reinterpret_cast<uint16_t *>(smem + L.soff[s])[i] =
              (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rS[s], o * 2u, 0, 0);
          reinterpret_cast<uint8_t *>(smem + L.zoff[s])[i] =
              (uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rZ[s], o, 0, 0);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kSZ; ++r) {
      if (r >= nsz) break;
      const int i = tid + r * 64 * NW;
      if (i < 16 * G) {
#pragma unroll
        for (int s = 0; s < NP; ++s) {
          reinterpret_cast<uint16_t *>(smem + L.soff[s])[i] = (uint16_t)sreg[s][r];
          reinterpret_cast<uint8_t *>(smem + L.zoff[s])[i] = (uint8_t)zreg[s][r];
        }
      }
    }
  }
  if constexpr (STAGE_X) {
#pragma unroll
    for (int r = 0; r < kXR; ++r) {
      if (r >= nxr || (kVecSZ && (uint32_t)(wave * 64 + r * 64 * NW) * 16u >= xbytes)) break;
      const uint32_t o = (uint32_t)(tid + r * 64 * NW) * 16u;
      if (o < xbytes) *reinterpret_cast<u32x4 *>(smem + o) = xreg[r];
    }
  }
  __syncthreads();

  // Activation row of this lane as the A operand: row c, or row 0 for the
  // padding rows c >= M.  Row m of the MFMA result depends on row m of A
  // alone, and result rows >= M are never stored, so the padding rows may
  // hold any values.
  const char *xlds = smem + (c < M ? (uint32_t)c * L.xrow : 0u) + (uint32_t)(kq * kWpl * 16);

  f32x4 acc[NP];
#pragma unroll
  for (int s = 0; s < NP; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const DeqRegs dq;

  // Batch i of this wave holds groups wave + i*NW*U + u*NW (u < U).
  auto compute = [&](const Batch &cur, int g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NW;
      const int gs = g < G ? g : G - 1;
      u32x4 a[kWpl];
#pragma unroll
      for (int j = 0; j < kWpl; ++j) {
        if constexpr (STAGE_X)
          a[j] = *reinterpret_cast<const u32x4 *>(xlds + (uint32_t)gs * (GS * 2) + 16u * j);
        else
          a[j] = g < G ? cur.a[u][j] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const uint32_t zr = reinterpret_cast<const uint8_t *>(smem + L.zoff[s])[c * G + gs] + zfix;
        const uint16_t sb = reinterpret_cast<const uint16_t *>(smem + L.soff[s])[c * G + gs];
        const float sc = g < G ? half_bits_to_float(sb) : 0.0f;
        // The exact integers q - z times a, summed in fp32 over the group
        // (every product is exact), then scaled once.
        const DeqF16 deq(zr);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kWpl; ++j) {
          const u32x4 h = deq(cur.raw[s][u][j], dq);
          t = mfma32<XT>(a[j], kBF16 ? f16_pairs_to_bf16(h) : h, t);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[s][e] = __builtin_fmaf(t[e], sc, acc[s][e]);
      }
    }
  };

  // Software pipeline over two register sets: while one batch is dequantized
  // and multiplied, the next one's loads are in flight.  The steady-state
  // loop body issues exactly one batch before each computed batch, and the
  // last one or two batches are peeled, so no load is ever conditional and
  // no register copy forces a wait.
  const int nb = wave < G ? (G - wave + NW * U - 1) / (NW * U) : 0;   // uniform
  int i = 0;
  for (; i + 2 < nb; i += 2) {
    const int g0 = wave + i * NW * U;
    load_batch(g0 + NW * U, bB);
    __builtin_amdgcn_sched_barrier(0);
    compute(bA, g0);
    load_batch(g0 + 2 * NW * U, bA);
    __builtin_amdgcn_sched_barrier(0);
    compute(bB, g0 + NW * U);
  }
  if (nb - i == 2) {
    const int g0 = wave + i * NW * U;
    load_batch(g0 + NW * U, bB);
    __builtin_amdgcn_sched_barrier(0);
    compute(bA, g0);
    compute(bB, g0 + NW * U);
  } else if (nb - i == 1) {
    compute(bA, wave + i * NW * U);
  }

  // Cross-wave sum.  Wave w's partial of output (m, c) goes to
  // red[(s*M*16 + m*16 + c) * kRS + w]: the NW partials of one output are
  // contiguous (kRS = NW + 4 floats per output keeps rows 16-byte aligned and
  // the 16 lanes of a row of outputs on distinct banks), so thread t < M*16
  // sums output t with NW/4 16-byte reads, in wave order as before.  The
  // partials have their own LDS region after the staged data when it fits
  // (one barrier); otherwise they reuse the start of the buffer, after a
  // barrier that waits for every wave to leave the loop.
  constexpr int kRS = NW + 4;
  const uint32_t red_bytes = (uint32_t)NP * (uint32_t)M * 16u * kRS * 4u;
  const bool red_alias = L.total + red_bytes > gemv_lds_cap(NW);
  if (__builtin_expect(red_alias, 0)) __syncthreads();
  float *red = reinterpret_cast<float *>(smem + (red_alias ? 0u : L.total));
#pragma unroll
  for (int s = 0; s < NP; ++s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * kq + e;
      if (m < M) red[((s * M + m) * 16 + c) * kRS + wave] = acc[s][e];
    }
  }
  __syncthreads();
  if (tid >= M * 16) return;
  const int om = tid >> 4, oc = tid & 15;
  const int on = n0 + oc;
  if (on >= N) return;
  float sum[NP];
#pragma unroll
  for (int s = 0; s < NP; ++s) {
    const f32x4 *row = reinterpret_cast<const f32x4 *>(red + ((s * M + om) * 16 + oc) * kRS);
    f32x4 part[NW / 4];
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) part[i] = row[i];
    sum[s] = part[0][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum[s] += part[w >> 2][w & 3];
  }
  const int64_t o = (int64_t)om * N + on;
  const float v = NP == 2 ? silu(sum[0]) * sum[1] : sum[0];
  if (ytype == (int)YType::F16)
    reinterpret_cast<uint16_t *>(Y)[o] = float_to_half_bits(v);
  else if (ytype == (int)YType::BF16)
    reinterpret_cast<uint16_t *>(Y)[o] = float_to_bf16_bits(v);
  else
    reinterpret_cast<float *>(Y)[o] = v;
}


template <class XT, int GS, int NW, int NP, bool MULTI>
static void gemv_launch(const uint16_t *X, const GemvParts &parts, int tiles, int M, int64_t K,
                        YType yt, uint32_t zfix, hipStream_t st) {
  const dim3 grid((unsigned)tiles);
  const int G = (int)(K / GS);
  const bool stage = (uint64_t)M * (uint64_t)K * 2u <= gemv_stage_budget(NW);
  const GemvSmem L = gemv_smem(M, (int)K, G, stage, NP);
  // the cross-wave partials: after the staged data when that fits, else
  // over its start (the kernel makes the same choice)
  const uint32_t red = (uint32_t)NP * (uint32_t)M * 16u * (NW + 4) * 4u;
  const uint32_t bytes = L.total + red <= gemv_lds_cap(NW) ? L.total + red : (L.total > red ? L.total : red);
  // Two groups per batch once a wave walks more than 8 groups (measured 7%
  // faster at 13.5 groups per wave, slower at 5 and below: 4096 x 4096 and
  // 4096 x 11008 at M = 1 and 4 took 1-10% longer with two).
  // staging rounds: activations (16 bytes per thread), and scale/zero slots
  // (16-wave: one wave-slot of 16-byte chunks per wave) or elements (8-wave)
  const uint32_t xr = (uint32_t)(((uint64_t)M * (uint64_t)K * 2u + 64u * NW * 16u - 1u) / (64u * NW * 16u));
  // (16-wave workgroups and the 8-wave gate/up pair stage them in 16-byte
  // wave slots, single 8-wave sets element by element: gemv_kernel's kVecSZ)
  const int szr = NW == 16 || NP == 2 ? (NP * ((2 * G + 63) / 64 + (G + 63) / 64) + NW - 1) / NW
                                      : (16 * G + 64 * NW - 1) / (64 * NW);
  const bool small = xr <= 2 && szr <= 1;
  if (stage && G > 8 * NW)
    gemv_kernel<XT, GS, NW, 2, true, NP, MULTI, false><<<grid, 64 * NW, bytes, st>>>(X, parts, M, (int)K, (int)yt, zfix);
  else if (stage && small)
    gemv_kernel<XT, GS, NW, 1, true, NP, MULTI, true><<<grid, 64 * NW, bytes, st>>>(X, parts, M, (int)K, (int)yt, zfix);
  else if (stage)
    gemv_kernel<XT, GS, NW, 1, true, NP, MULTI, false><<<grid, 64 * NW, bytes, st>>>(X, parts, M, (int)K, (int)yt, zfix);
  else
    gemv_kernel<XT, GS, NW, 2, false, NP, MULTI, false><<<grid, 64 * NW, bytes, st>>>(X, parts, M, (int)K, (int)yt, zfix);
}

// Waves per workgroup.  Every workgroup of a launch should be resident at
// once (a second partial round of workgroups costs a whole extra memory
// latency): with at most one workgroup per CU (at most 256 column tiles) the
// workgroup takes 16 waves, otherwise 8.  One batch per wave is in flight ahead
// of the one being computed: deeper windows were measured slower on MI355X
// (every wave's staging loads then queue behind more weight traffic).
template <class XT, int GS, int NP>
static void gemv_dispatch(const uint16_t *X, const GemvParts &parts, int tiles, int M, int64_t K,
                          YType yt, uint32_t zfix, hipStream_t st) {
  // the gate/up pair always takes 8 waves: with 16, its two sets of staging
  // registers spill under the 1024-thread register budget
  if (NP == 2)
    gemv_launch<XT, GS, 8, NP, false>(X, parts, tiles, M, K, yt, zfix, st);
  else if (parts.count > 1 && gemv_waves_for_tiles(tiles) == 16)
    gemv_launch<XT, GS, 16, NP, true>(X, parts, tiles, M, K, yt, zfix, st);
  else if (parts.count > 1)
    gemv_launch<XT, GS, 8, NP, true>(X, parts, tiles, M, K, yt, zfix, st);
  else if (gemv_waves_for_tiles(tiles) == 16)
    gemv_launch<XT, GS, 16, NP, false>(X, parts, tiles, M, K, yt, zfix, st);
  else
    gemv_launch<XT, GS, 8, NP, false>(X, parts, tiles, M, K, yt, zfix, st);
}

int64_t gemv_groups_per_wave(int64_t N, int64_t K, int gs) {
  return (K / gs) / gemv_waves(N);
}

bool gemv_stages_activations(int64_t M, int64_t N, int64_t K) {
  return (uint64_t)M * (uint64_t)K * 2u <= gemv_stage_budget(gemv_waves(N));
}

bool gemv_supported(int64_t M, int64_t N, int64_t K, int gs, int np) {
  const int64_t G = K / gs;
  const int nw = np == 2 ? 8 : gemv_waves(N);
  const bool stage = (uint64_t)M * (uint64_t)K * 2u <= gemv_stage_budget(nw);
  const GemvSmem L = gemv_smem((int)M, (int)K, (int)G, stage, np);
  return M <= 16 && 16 * G <= kGemvMaxSZ && L.total <= gemv_lds_cap(nw) && N * K / 2 < 0x7FFFFFF0;
}

namespace {
template <int NP>
hipError_t gemv_go(const void *X, XType xt, const GemvParts &parts, int tiles, int64_t M,
                   int64_t K, int gs, YType yt, uint32_t zfix, hipStream_t st) {
  const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
  if (xt == XType::F16) {
    if (gs == 128) gemv_dispatch<TagF16, 128, NP>(x, parts, tiles, (int)M, K, yt, zfix, st);
    else gemv_dispatch<TagF16, 64, NP>(x, parts, tiles, (int)M, K, yt, zfix, st);
  } else {
    if (gs == 128) gemv_dispatch<TagBF16, 128, NP>(x, parts, tiles, (int)M, K, yt, zfix, st);
    else gemv_dispatch<TagBF16, 64, NP>(x, parts, tiles, (int)M, K, yt, zfix, st);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemv(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, hipStream_t st) {
  const LinearPart one{qweight, scales, zeros, N, Y};
  return launch_gemv_parts(X, xt, &one, 1, false, M, K, gs, yt, st);
}

hipError_t launch_gemv_parts(const void *X, XType xt, const LinearPart *p, int count,
                             bool silu_mul, int64_t M, int64_t K, int gs, YType yt,
                             hipStream_t st) {
  if (M == 0 || count <= 0) return hipSuccess;
  GemvParts parts{};
  int tiles = 0;
  for (int i = 0; i < count; ++i) {
    parts.qw[i] = p[i].qweight;
    parts.sc[i] = p[i].scales;
    parts.zr[i] = p[i].zeros;
    parts.y[i] = p[i].Y;
    parts.n[i] = (int)p[i].N;
    if (!silu_mul || i == 0) tiles += (int)((p[i].N + 15) / 16);
    parts.tile_end[i] = tiles;
  }
  parts.count = count;
  if (tiles == 0) return hipSuccess;
  const uint32_t zfix = p[0].zeros ? 0u : 8u;
  if (silu_mul) return gemv_go<2>(X, xt, parts, tiles, M, K, gs, yt, zfix, st);
  return gemv_go<1>(X, xt, parts, tiles, M, K, gs, yt, zfix, st);
}

}  // namespace awq
