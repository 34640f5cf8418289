// The scale search's GEMMs on gfx950 MFMA ("AWQ Advanced Usage Guide", "How
// AWQ Works": the per-alpha reconstruction loss of the scaled, quantized
// layer; ai.lansai.wang explainer, section "AWQ 的四步链路", the scale search).
//  * Dense B: Y_ref = X * W^T with fp16 W, fp32 output.
//  * Loss: A * deq(Q(sW))^T against Y_ref; the epilogue reduces the squared
//    error of its tile to one fp64 partial instead of storing Y.
//
// Exactness (the losses are compared to an fp64 oracle at 1e-5): the B
// operand is the exact integer q - z, MFMA accumulates one group in fp32 and
// the group's scale multiplies that fp32 partial; no dequantized weight is
// rounded to 16 bits.  (The linear layer's GEMM, gemm_f16.hip, rounds it to
// fp16 instead.)
//
// Tiling: a 256-thread workgroup computes a 256 x 128 tile of Y; each wave
// owns 128 x 64 (8 x 4 MFMA tiles of 16 x 16).  K advances in blocks of 128
// channels (one g128 group or two g64 groups).
//  * Activations: each 256 x 128 fp16 block goes from global memory straight
//    to LDS (buffer_load_dwordx4 ... lds), double-buffered.  16-byte chunk c
//    of row r is stored at chunk c ^ (r mod 16).
//  * Per group, a wave reads its A fragments from LDS once; columns are then
//    walked one 16-wide tile at a time: the lane dequantizes its codes of that
//    column and runs 8 MFMA chains (one per M tile) whose fp32 sums are
//    scaled into the accumulator.
//  * Packed weights, scales and zeros bypass LDS and are prefetched one block
//    ahead into registers.
//  * All global accesses go through buffer resources: out-of-range reads
//    return zero and out-of-range writes are dropped, so edge tiles need no
//    branches around loads.
//  * One s_barrier per block, after an explicit vmcnt(0): the LDS DMA's
//    writes are known complete only then.
//  * Block ids are remapped so each XCD works on a contiguous run of tiles.
// 32-bit buffer offsets: the launcher slices M so that X, Y and the reference
// output of one launch stay below 2 GiB.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kBN = 128, kBK = 128;
constexpr int kThreads = 256;
constexpr uint32_t kNone = 0xFFFFFFFFu; // an offset every range check rejects

enum Epi : int { kEpiStore = 0, kEpiLoss = 1 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with vmcnt = 0 and expcnt / lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace


template <class XT, int GS, int EPI, bool DENSE, int YT, int MT>
__device__ __forceinline__ void gemm_body(const uint16_t *__restrict__ X,
                                          const uint32_t *__restrict__ qweight,
                                          const uint16_t *__restrict__ Wdense,
                                          const uint16_t *__restrict__ scales,
                                          const uint8_t *__restrict__ zeros, int M, int N, int K,
                                          void *__restrict__ Y, const float *__restrict__ Yref,
                                          double *__restrict__ partials, SplitK sk) {
  constexpr bool kBF16 = __is_same(XT, TagBF16);
  constexpr int kGS = DENSE ? 128 : GS;
  constexpr int kWpl = kGS / 32;        // 8-channel words per lane per group
  constexpr int kGPB = kBK / kGS;       // groups per K block
  constexpr int kBM = 32 * MT;
  // Wave layout: 2 x 2 waves of (BM/2) x 64.
  constexpr int kMT = MT;                   // 16x16 tiles per wave along M
  constexpr int kNT = 4;                    // 16x16 tiles per wave along N
  constexpr int kWaveCols = 16 * kNT;
  constexpr int kRowsPerWave = kBM / 4; // rows of the A block each wave fetches
  constexpr int kDma = kRowsPerWave / 4;

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const DeqRegs dq;
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 15, kq = lane >> 4;

  const int tiles_n = (N + kBN - 1) / kBN;
  const int tiles = ((M + kBM - 1) / kBM) * tiles_n;
  const int bid = (int)xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int tile = bid % tiles, split = bid / tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int row0 = tm * kBM, col0 = tn * kBN;

  const int G = K / kGS;
  const int nkb = (K + kBK - 1) / kBK;
  const int kb_begin = (int)((int64_t)split * nkb / sk.splits);
  const int kb_end = (int)((int64_t)(split + 1) * nkb / sk.splits);

  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);

  // ---- activation block -> LDS: kDma DMA instructions per wave, 1 KiB each ---
  // Instruction r of wave w fills rows kRowsPerWave*w + 4r .. +3; lane l writes
  // row +l/16 at physical chunk l%16 and so fetches logical chunk
  // (l%16) ^ (row%16).  row%16 = 4*((r + b) % 4) + l/16 with b the wave's first
  // row / 4, so four lane offsets cover every r.
  uint32_t a_voff[4];
  {
    const int lrow = lane >> 4;
    const int wrow = kRowsPerWave * wave;
    const uint32_t base = (uint32_t)(row0 + wrow + lrow) * (uint32_t)K * 2u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      a_voff[q] = base + ((uint32_t)((lane & 15) ^ (4 * ((q + wrow / 4) & 3) + lrow)) << 4);
  }
  const uint32_t a_rstep = 8u * (uint32_t)K;   // bytes between rows 4 apart
  auto issue_a = [&](int kb, uint16_t *buf) {
#pragma unroll
    for (int r = 0; r < kDma; ++r) {
      const uint32_t off = a_voff[r & 3] + (uint32_t)r * a_rstep + (uint32_t)kb * (kBK * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rX, (lds_void *)(reinterpret_cast<char *>(buf) + (kDma * wave + r) * 1024), 16, off, 0,
          0, 0);
    }
  };

  // ---- packed weights, scales and zeros of one K block (registers) -------------
  const uint32_t lane_col = (uint32_t)(wn * kWaveCols + c);
  const rsrc_t rQ = make_rsrc(qweight, DENSE ? 0u : (uint32_t)N * (uint32_t)K / 2u);
  const rsrc_t rS = make_rsrc(scales, DENSE ? 0u : (uint32_t)N * (uint32_t)G * 2u);
  const rsrc_t rZ = make_rsrc(zeros, DENSE ? 0u : (uint32_t)N * (uint32_t)G);
  const uint32_t q_lane = lane_col * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  const uint32_t s_lane = lane_col * (uint32_t)G;

  // Scales and zero points keep the width they are loaded with: widening them
  // here would make the compiler wait for those loads right after issuing them.
  struct BRegs {
    uint32_t raw[kNT][kGPB][kWpl];
    uint16_t sc[kNT][kGPB];
    uint8_t zr[kNT][kGPB];
  };
  auto load_b = [&](int kb, BRegs &r) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const uint32_t ncol = (uint32_t)(col0 + j * 16);
#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        const uint32_t g = (uint32_t)(kb * kGPB + gi);
        const uint32_t qo = q_lane + ncol * (uint32_t)(K / 2) + g * (kGS / 2);
        if constexpr (kWpl == 4) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
#pragma unroll
          for (int w = 0; w < kWpl; ++w) r.raw[j][gi][w] = v[w];
        } else {
          const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rQ, qo, 0, 0));
#pragma unroll
          for (int w = 0; w < kWpl; ++w) r.raw[j][gi][w] = v[w];
        }
        const uint32_t so = s_lane + ncol * (uint32_t)G + g;
        r.sc[j][gi] = __builtin_amdgcn_raw_buffer_load_b16(rS, so * 2u, 0, 0);
        r.zr[j][gi] = __builtin_amdgcn_raw_buffer_load_b8(rZ, so, 0, 0);
      }
    }
  };

  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A fragment: M tile i, logical 16-byte chunk ch of the block row.
  auto a_frag = [&](const uint16_t *buf, int i, int ch) {
    const int row = wm * (16 * kMT) + i * 16 + c;
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(buf) + row * (kBK * 2) +
                                            ((ch ^ c) << 4));
  };

  const rsrc_t rW = make_rsrc(Wdense, DENSE ? (uint32_t)N * (uint32_t)K * 2u : 0u);
  const uint32_t w_lane = lane_col * (uint32_t)K * 2u + (uint32_t)(kq * 64);

  auto compute = [&](int kb, const uint16_t *buf, const BRegs &br) {
    if constexpr (DENSE) {
      u32x4 a[kMT][4];
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int st = 0; st < 4; ++st) a[i][st] = a_frag(buf, i, kq * 4 + st);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        u32x4 b[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kk = kb * kBK + kq * 32 + 8 * st;
          const uint32_t off = w_lane + (uint32_t)(col0 + j * 16) * (uint32_t)K * 2u +
                               (uint32_t)(kb * kBK * 2 + st * 16);
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
          b[st] = kk < K ? v : u32x4{0u, 0u, 0u, 0u};    // K tail of a g64-aligned K
        }
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int i = 0; i < kMT; ++i) acc[i][j] = mfma32<XT>(a[i][st], b[st], acc[i][j]);
      }
    } else {
#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        if (kGPB > 1 && kb * kGPB + gi >= G) break;
        u32x4 a[kMT][kWpl];
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
          for (int w = 0; w < kWpl; ++w) a[i][w] = a_frag(buf, i, gi * (kGS / 8) + kq * kWpl + w);
        f32x4 rs[kMT];
        if constexpr (kBF16) {
#pragma unroll
          for (int i = 0; i < kMT; ++i) {
            rs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWpl; ++w) rs[i] = mfma32<TagBF16>(a[i][w], bf16_ones(), rs[i]);
          }
        }
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          u32x4 bq[kWpl];
          if constexpr (!kBF16) {
            const DeqF16 deq((uint32_t)br.zr[j][gi]);
#pragma unroll
            for (int w = 0; w < kWpl; ++w) bq[w] = deq(br.raw[j][gi][w], dq);
          } else {
#pragma unroll
            for (int w = 0; w < kWpl; ++w) bq[w] = deq_bf16_biased(br.raw[j][gi][w], dq);
          }
          const float sc = half_bits_to_float(br.sc[j][gi]);
          f32x4 t[kMT];
#pragma unroll
          for (int i = 0; i < kMT; ++i) t[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kWpl; ++w)
#pragma unroll
            for (int i = 0; i < kMT; ++i) t[i] = mfma32<XT>(a[i][w], bq[w], t[i]);
#pragma unroll
          for (int i = 0; i < kMT; ++i) {
            if constexpr (kBF16) {
              const float cz = -(float)(128u + (uint32_t)br.zr[j][gi]);
#pragma unroll
              for (int e = 0; e < 4; ++e) t[i][e] = __builtin_fmaf(cz, rs[i][e], t[i][e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(t[i][e], sc, acc[i][j][e]);
          }
        }
      }
    }
  };

  // ---- main loop: two static buffers, one barrier per block -------------------
  // Prefetch indices are clamped to the last block instead of branched on, so
  // no load sits under a branch; the surplus prefetch of the last iteration
  // lands in a buffer nobody reads again.
  BRegs r0, r1;
  const int last = kb_end - 1;
  issue_a(kb_begin, sA0);
  if constexpr (!DENSE) load_b(kb_begin, r0);
  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    wait_vmem_all();
    __builtin_amdgcn_s_barrier();
    issue_a(kb + 1 < last ? kb + 1 : last, sA1);
    if constexpr (!DENSE) load_b(kb + 1 < last ? kb + 1 : last, r1);
    __builtin_amdgcn_sched_barrier(0);   // issue the prefetch before the math
    compute(kb, sA0, r0);
    if (kb + 1 >= kb_end) break;

    wait_vmem_all();
    __builtin_amdgcn_s_barrier();
    issue_a(kb + 2 < last ? kb + 2 : last, sA0);
    if constexpr (!DENSE) load_b(kb + 2 < last ? kb + 2 : last, r0);
    __builtin_amdgcn_sched_barrier(0);
    compute(kb + 1, sA1, r1);
  }
  wait_vmem_all();

  // ---- epilogue -------------------------------------------------------------
  // Lane (c, kq) holds rows 4*kq + e of column c of every 16x16 tile.
  if constexpr (EPI == kEpiStore) {
    constexpr int ysz = YT == (int)YType::F32 ? 4 : 2;
    const rsrc_t rY = make_rsrc(Y, (uint32_t)M * (uint32_t)N * (uint32_t)ysz);
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int n = col0 + wn * kWaveCols + j * 16 + c;
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + wm * (16 * kMT) + i * 16 + 4 * kq + e;
          const uint32_t o = n < N ? (uint32_t)m * (uint32_t)N + (uint32_t)n : kNone / 4u;
          const float v = acc[i][j][e];
          if constexpr (YT == (int)YType::F16)
            __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(v), rY, o * 2u, 0, 0);
          else if constexpr (YT == (int)YType::BF16)
            __builtin_amdgcn_raw_buffer_store_b16(float_to_bf16_bits(v), rY, o * 2u, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rY, o * 4u, 0, 0);
        }
      }
    }
  } else {
    const rsrc_t rR = make_rsrc(Yref, (uint32_t)M * (uint32_t)N * 4u);
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int n = col0 + wn * kWaveCols + j * 16 + c;
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // rows >= M and columns >= N read 0 and have acc = 0: they add nothing
          const int m = row0 + wm * (16 * kMT) + i * 16 + 4 * kq + e;
          const uint32_t o = n < N ? (uint32_t)m * (uint32_t)N + (uint32_t)n : kNone / 4u;
          const float ref = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, o * 4u, 0, 0));
          const double d = (double)ref - (double)acc[i][j][e];
          sum = __builtin_fma(d, d, sum);
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    __syncthreads();
    double *wsum = reinterpret_cast<double *>(sA0);
    if (lane == 0) wsum[wave] = sum;
    __syncthreads();
    if (tid == 0) partials[tm * tiles_n + tn] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

// The 128- and 256-row tiles keep one wave per SIMD and the whole register file
// (accumulators plus the weight window); smaller tiles run two workgroups per
// CU.
template <class XT, int GS, int EPI, bool DENSE, int YT, int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel_big(const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
                     const uint16_t *__restrict__ Wdense, const uint16_t *__restrict__ scales,
                     const uint8_t *__restrict__ zeros, int M, int N, int K, void *__restrict__ Y,
                     const float *__restrict__ Yref, double *__restrict__ partials, SplitK sk) {
  gemm_body<XT, GS, EPI, DENSE, YT, MT>(X, qweight, Wdense, scales, zeros, M, N, K, Y, Yref,
                                        partials, sk);
}

// Largest row count per launch that keeps every per-launch buffer below 2 GiB
// (a multiple of the row tile bm).
static int64_t rows_per_launch(int64_t N, int64_t K, int64_t bm) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  int64_t r = lim / (K * 2);
  const int64_t ry = lim / (N * 4);
  r = r < ry ? r : ry;
  return (r / bm) * bm;
}

bool gemm_supported(int64_t N, int64_t K, bool dense) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  return (dense ? N * K * 2 : N * K / 2) <= lim && rows_per_launch(N, K, 256) > 0;
}


GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, XType xt) {
  return gemm_f16_plan(M, N, K, xt == XType::BF16);
}

// The bf16 plan adds the row factors to the fp16 plan's workspace.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return gemm_f16_plan(M, N, K, true).workspace_bytes;
}

// The search's GEMMs: the 256-row tile, fp32 output or the loss epilogue.
template <int GS, int EPI, bool DENSE>
static hipError_t gemm_go(const uint16_t *X, const uint32_t *qw, const uint16_t *Wd,
                          const uint16_t *sc, const uint8_t *zr, int64_t M, int64_t N, int64_t K,
                          void *Y, const float *Yref, double *partials, hipStream_t st) {
  constexpr int MT = 8;
  constexpr int64_t bm = 32 * MT;
  const SplitK sk{1, nullptr};
  const int64_t rows = rows_per_launch(N, K, bm);
  if (rows <= 0) return hipErrorInvalidValue;
  int64_t tile_base = 0;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    void *y = Y ? reinterpret_cast<char *>(Y) + m0 * N * 4 : nullptr;
    const float *yr = Yref ? Yref + m0 * N : nullptr;
    double *pp = partials ? partials + tile_base : nullptr;
    gemm_kernel_big<TagF16, GS, EPI, DENSE, (int)YType::F32, MT><<<dim3((unsigned)tiles), kThreads, 0, st>>>(
        X + m0 * K, qw, Wd, sc, zr, (int)mm, (int)N, (int)K, y, yr, pp, sk);
    tile_base += tiles;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, void *workspace,
                       hipStream_t st) {
  return launch_gemm_f16(reinterpret_cast<const uint16_t *>(X), xt == XType::BF16, qweight,
                         scales, zeros, M, N, K, gs, Y, yt, workspace, st);
}

hipError_t launch_gemm_dense_f32(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N,
                                 int64_t K, float *Y, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  return gemm_go<128, kEpiStore, true>(X, nullptr, W, nullptr, nullptr, M, N, K, Y, nullptr,
                                       nullptr, st);
}

}  // namespace awq
