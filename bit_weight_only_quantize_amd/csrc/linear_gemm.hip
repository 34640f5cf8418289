// The scale search's reference GEMM on gfx950 MFMA: Y_ref = X * W^T with the
// unquantized fp16 W and fp32 output ("AWQ Advanced Usage Guide", "How AWQ
// Works": the per-alpha loss compares the scaled, quantized layer against the
// original one; ai.lansai.wang explainer, section "AWQ 的四步链路", the scale
// search).  It runs once per search.  (The quantized GEMMs, the linear layer's
// and the search's per-alpha loss, are in gemm_f16.hip.)
//
// Tiling: a 256-thread workgroup computes a 256 x 128 tile of Y; each wave
// owns 128 x 64 (8 x 4 MFMA tiles of 16 x 16).  K advances in blocks of 128
// channels.
//  * Activations: each 256 x 128 fp16 block goes from global memory straight
//    to LDS (buffer_load_dwordx4 ... lds), double-buffered.  16-byte chunk c
//    of row r is stored at chunk c ^ (r mod 16).
//  * W fragments are loaded from global memory per block (16 bytes per lane
//    and MFMA step); a K tail (K % 128 == 64) reads zero weights.
//  * All global accesses go through buffer resources: out-of-range reads
//    return zero and out-of-range writes are dropped, so edge tiles need no
//    branches around loads.
//  * One s_barrier per block, after an explicit vmcnt(0): the LDS DMA's
//    writes are known complete only then.
//  * Block ids are remapped so each XCD works on a contiguous run of tiles.
// 32-bit buffer offsets: the launcher slices M so that X and Y of one launch
// stay below 2 GiB.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kBN = 128, kBK = 128;
constexpr int kThreads = 256;
constexpr int kMT = 8;                    // 16x16 tiles per wave along M
constexpr int kNT = 4;                    // 16x16 tiles per wave along N
constexpr int kBM = 32 * kMT;             // rows per workgroup (2 waves along M)
constexpr uint32_t kNone = 0xFFFFFFFFu;   // an offset every range check rejects

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with vmcnt = 0 and expcnt / lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace

__device__ __forceinline__ void dense_gemm_body(const uint16_t *__restrict__ X,
                                                const uint16_t *__restrict__ W, int M, int N,
                                                int K, float *__restrict__ Y) {
  constexpr int kWaveCols = 16 * kNT;
  constexpr int kRowsPerWave = kBM / 4;   // rows of the A block each wave fetches
  constexpr int kDma = kRowsPerWave / 4;

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 15, kq = lane >> 4;

  const int tiles_n = (N + kBN - 1) / kBN;
  const int tile = (int)xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int row0 = tm * kBM, col0 = tn * kBN;
  const int nkb = (K + kBK - 1) / kBK;

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

  // Lane (c, kq) at MFMA step st multiplies channels kq*32 + 8*st .. +7 of the
  // block: logical chunk kq*4 + st of the A row and of W's row (col0 + 16j + c).
  const uint32_t lane_col = (uint32_t)(wn * kWaveCols + c);
  const rsrc_t rW = make_rsrc(W, (uint32_t)N * (uint32_t)K * 2u);
  const uint32_t w_lane = lane_col * (uint32_t)K * 2u + (uint32_t)(kq * 64);

  auto compute = [&](int kb, const uint16_t *buf) {
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
        for (int i = 0; i < kMT; ++i) acc[i][j] = mfma32<TagF16>(a[i][st], b[st], acc[i][j]);
    }
  };

  // ---- main loop: two static buffers, one barrier per block -------------------
  // Prefetch indices are clamped to the last block instead of branched on, so
  // no load sits under a branch; the surplus prefetch of the last iteration
  // lands in a buffer nobody reads again.
  const int last = nkb - 1;
  issue_a(0, sA0);
  for (int kb = 0; kb < nkb; kb += 2) {
    wait_vmem_all();
    __builtin_amdgcn_s_barrier();
    issue_a(kb + 1 < last ? kb + 1 : last, sA1);
    __builtin_amdgcn_sched_barrier(0);   // issue the prefetch before the math
    compute(kb, sA0);
    if (kb + 1 >= nkb) break;

    wait_vmem_all();
    __builtin_amdgcn_s_barrier();
    issue_a(kb + 2 < last ? kb + 2 : last, sA0);
    __builtin_amdgcn_sched_barrier(0);
    compute(kb + 1, sA1);
  }
  wait_vmem_all();

  // ---- epilogue: lane (c, kq) holds rows 4*kq + e of column c of every tile -----
  const rsrc_t rY = make_rsrc(Y, (uint32_t)M * (uint32_t)N * 4u);
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int n = col0 + wn * kWaveCols + j * 16 + c;
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + wm * (16 * kMT) + i * 16 + 4 * kq + e;
        const uint32_t o = n < N ? (uint32_t)m * (uint32_t)N + (uint32_t)n : kNone / 4u;
        // (a scalar copy first: bit-casting an element of a vector lvalue reads
        // the vector's first element with this compiler)
        const float v = acc[i][j][e];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rY, o * 4u, 0, 0);
      }
    }
  }
}

// One wave per SIMD: 128 fp32 accumulators per lane plus the A fragments of a
// block live in registers.  (The body is a __device__ function: the host stub
// of a __global__ template calling the LDS-DMA builtin directly was lost.)
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dense_gemm_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, int M,
                       int N, int K, float *__restrict__ Y) {
  dense_gemm_body(X, W, M, N, K, Y);
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

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, XType xt, Scratch sc) {
  return gemm_f16_plan(M, N, K, xt == XType::BF16, sc);
}

hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, const GemmPlan &plan,
                       void *workspace, hipStream_t st) {
  return launch_gemm_f16(reinterpret_cast<const uint16_t *>(X), xt == XType::BF16, qweight,
                         scales, zeros, M, N, K, gs, Y, yt, plan, workspace, st);
}

// ---- SiLU(gate) * up: the epilogue of the fused gate/up projections on the GEMM
// path ("AWQ Advanced Usage Guide", "Layer Fusion": gate and up projections fused).
// H[i] = silu(A[i]) * B[i] over fp32 A (gate) and B (up), rounded once to yt;
// silu(x) = x / (1 + e^-x).  HBM-bound: 8 bytes in, 2 or 4 out per element.
__global__ __launch_bounds__(256) void silu_mul_kernel(const float *__restrict__ A,
                                                       const float *__restrict__ B, int64_t n,
                                                       void *__restrict__ H, int yt) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n) return;
  float v[4];
  if (i4 + 4 <= n) {
    const float4 a = *reinterpret_cast<const float4 *>(A + i4);
    const float4 b = *reinterpret_cast<const float4 *>(B + i4);
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = av[e] / (1.0f + __expf(-av[e])) * bv[e];
  } else {
    for (int e = 0; e < 4; ++e) v[e] = i4 + e < n ? A[i4 + e] / (1.0f + __expf(-A[i4 + e])) * B[i4 + e] : 0.0f;
  }
  for (int e = 0; e < 4 && i4 + e < n; ++e) {
    if (yt == (int)YType::F32)
      reinterpret_cast<float *>(H)[i4 + e] = v[e];
    else if (yt == (int)YType::BF16)
      reinterpret_cast<uint16_t *>(H)[i4 + e] = float_to_bf16_bits(v[e]);
    else
      reinterpret_cast<uint16_t *>(H)[i4 + e] = float_to_half_bits(v[e]);
  }
}

hipError_t launch_silu_mul(const float *A, const float *B, int64_t n, void *H, YType yt,
                           hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  silu_mul_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(A, B, n, H, (int)yt);
  return hipGetLastError();
}

hipError_t launch_gemm_dense_f32(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N,
                                 int64_t K, float *Y, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t rows = rows_per_launch(N, K, kBM);
  if (rows <= 0) return hipErrorInvalidValue;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    dense_gemm_kernel<<<dim3((unsigned)tiles), kThreads, 0, st>>>(X + m0 * K, W, (int)mm, (int)N,
                                                                  (int)K, Y + m0 * N);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace awq
