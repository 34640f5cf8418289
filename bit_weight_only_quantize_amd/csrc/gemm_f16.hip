// Batched / prefill W4A16 GEMM for fp16 activations on gfx950 MFMA.
//
// The GEMM variant of the quantized linear layer ("AWQ Advanced Usage Guide",
// "WQLinear Kernel Variants": batch sizes above one), Y = X * deq(W)^T with
// deq = (q - z) * s per group of g input channels (the pages' zero-point,
// group-wise int4 configuration).
//
// Exactness: the B operand is the exact integer q - z in fp16, MFMA sums one
// group in fp32 and the group's scale multiplies that fp32 partial; no
// dequantized weight is rounded to 16 bits.
//
// Work split, chosen for the MI355X's balance of MFMA, VALU and LDS rates:
//  * A 256-thread workgroup owns a BM x 128 tile of Y (BM = 16 * MT rows).
//    Wave v owns columns 32v .. 32v+31 over all BM rows, so every weight word
//    is loaded and dequantized by exactly one lane of the workgroup, and each
//    dequantized B fragment feeds MT MFMAs (8 for the 128-row tile).
//  * The price is that every wave reads the whole activation block from LDS
//    (4x replication); gfx950's 64-bank LDS carries that at well under its
//    rate.  A 16-byte chunk c of block row r is stored at chunk c ^ (r % 16),
//    so the 16 rows one 128-bit LDS read touches fall in 16 distinct bank
//    groups.
//  * Per group, a lane dequantizes its 2 x (g/32) words up front; then per
//    16-row tile it reads g/32 activation fragments and runs two short MFMA
//    chains (one per 16-column tile) whose fp32 sums are scaled into the
//    accumulators.  Registers stay under half the file, so two workgroups
//    share each CU and one's VALU work overlaps the other's MFMAs.
//  * Compute-bound tiles (128 rows) stream activations straight into LDS with
//    buffer_load ... lds, double-buffered, one block ahead.  Memory-bound
//    tiles (32 and 64 rows, batched decode) stage activations through
//    registers instead, so that only ordinary loads are in flight and counted
//    waits can keep a window of several weight blocks streaming from HBM.
//  * Split K (when the M x N tiles cannot fill the CUs) and its fence-free
//    fixup follow the same scheme as the other GEMM kernels of this library.
//  * Tiles are visited in groups of four row tiles, row index fastest, so the
//    workgroups resident on one XCD share activation rows and weight columns
//    in that XCD's L2.
// 32-bit buffer offsets: the launcher slices M so that X and Y of one launch
// stay below 2 GiB; every access goes through a buffer resource whose range
// check turns edge-tile reads into zeros and drops edge-tile writes.

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;        // columns per workgroup (4 waves x 32)
constexpr int kBK = 128;        // input channels per K block
constexpr int kGroupRows = 4;   // row tiles per tile group
constexpr uint32_t kNone = 0xFFFFFFFFu;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(0), expcnt and lgkmcnt at their maxima.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace

template <int GS, int YT, int MT, bool DMA, bool KTAIL>
__device__ __forceinline__ void gemm_f16_body(const uint16_t *__restrict__ X,
                                              const uint32_t *__restrict__ qweight,
                                              const uint16_t *__restrict__ scales,
                                              const uint8_t *__restrict__ zeros, int M, int N,
                                              int K, void *__restrict__ Y, SplitK sk) {
  constexpr int kBM = 16 * MT;
  constexpr int kWpl = GS / 32;      // packed words per lane per group and column
  constexpr int kGPB = kBK / GS;     // groups per K block
  // Weight blocks in flight on the register-staged path (as many as the
  // register budget of two workgroups per CU allows).
  constexpr int kWin = (MT <= 2 ? 4 : 3) - (kGPB > 1 ? 1 : 0);

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  const DeqRegs dq;

  // ---- tile of this workgroup -------------------------------------------------
  const int tiles_n = (N + kBN - 1) / kBN;
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles = tiles_m * tiles_n;
  const int bid = (int)xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int tile = bid % tiles, split = bid / tiles;
  int tm, tn;
  {
    const int per = kGroupRows * tiles_n;
    const int grp = tile / per, first = grp * kGroupRows;
    const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
    const int r = tile - grp * per;
    tm = first + r % rows;
    tn = r / rows;
  }
  const int row0 = tm * kBM, col0 = tn * kBN;

  const int G = K / GS;
  const int nkb = (K + kBK - 1) / kBK;
  const int kb_begin = (int)((int64_t)split * nkb / sk.splits);
  const int kb_end = (int)((int64_t)(split + 1) * nkb / sk.splits);

  // ---- packed weights, scales and zeros of one K block (registers) -------------
  // Lane (c, kq) holds, for column tile j, words kq*kWpl .. kq*kWpl+kWpl-1 of
  // each group of column col0 + 32*wave + 16*j + c: channels
  // 8*(kq*kWpl + w) .. +7 of the group for MFMA step w.
  const uint32_t lane_col = (uint32_t)(col0 + wave * 32 + c);
  const rsrc_t rQ = make_rsrc(qweight, (uint32_t)N * (uint32_t)K / 2u);
  const rsrc_t rS = make_rsrc(scales, (uint32_t)N * (uint32_t)G * 2u);
  const rsrc_t rZ = make_rsrc(zeros, (uint32_t)N * (uint32_t)G);
  const uint32_t q_lane = lane_col * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  const uint32_t s_lane = lane_col * (uint32_t)G;

  // Scales and zero points keep their load width: widening them right after
  // the load would make the compiler wait for it there.
  struct BRegs {
    uint32_t raw[2][kGPB][kWpl];
    uint16_t sc[2][kGPB];
    uint8_t zr[2][kGPB];
  };
  auto load_b = [&](int kb, BRegs &r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        const uint32_t g = (uint32_t)(kb * kGPB + gi);
        // With KTAIL, a group past the end of K reads zero weights, scale and
        // zero point (and zero activations), so it adds exactly nothing.
        const bool in_k = !KTAIL || g < (uint32_t)G;
        const uint32_t qo =
            in_k ? q_lane + (uint32_t)(16 * j) * (uint32_t)(K / 2) + g * (GS / 2) : kNone;
        if constexpr (kWpl == 4) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
#pragma unroll
          for (int w = 0; w < kWpl; ++w) r.raw[j][gi][w] = v[w];
        } else {
          const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rQ, qo, 0, 0));
#pragma unroll
          for (int w = 0; w < kWpl; ++w) r.raw[j][gi][w] = v[w];
        }
        const uint32_t so = in_k ? s_lane + (uint32_t)(16 * j) * (uint32_t)G + g : kNone / 2u;
        r.sc[j][gi] = __builtin_amdgcn_raw_buffer_load_b16(rS, so * 2u, 0, 0);
        r.zr[j][gi] = __builtin_amdgcn_raw_buffer_load_b8(rZ, so, 0, 0);
      }
    }
  };

  f32x4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    acc[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // A fragment: 16-row tile i, logical 16-byte chunk ch of the block row.
  auto a_frag = [&](const uint16_t *buf, int i, int ch) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(buf) +
                                            (i * 16 + c) * (kBK * 2) + ((ch ^ c) << 4));
  };

  // One K block.  Per group: dequantize this lane's 2 x kWpl words, then walk
  // the 16-row tiles in a software pipeline: iteration i requests tile i+1's
  // activation fragments, runs tile i's two MFMA chains and scales tile i-1's
  // finished chains into the accumulators, so neither the LDS reads nor the
  // MFMA results are waited for right after they were issued.  The scheduling
  // barriers keep the compiler from hoisting every fragment read of the group
  // to the top (which would need 4 x MT x kWpl live registers).
  auto compute = [&](const uint16_t *buf, const BRegs &br) {
#pragma unroll
    for (int gi = 0; gi < kGPB; ++gi) {
      u32x4 bq[2][kWpl];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const DeqF16 deq((uint32_t)br.zr[j][gi]);
#pragma unroll
        for (int w = 0; w < kWpl; ++w) bq[j][w] = deq(br.raw[j][gi][w], dq);
      }
      const float s0 = half_bits_to_float(br.sc[0][gi]);
      const float s1 = half_bits_to_float(br.sc[1][gi]);
      u32x4 a[2][kWpl];
      f32x4 t[2][2];
#pragma unroll
      for (int w = 0; w < kWpl; ++w) a[0][w] = a_frag(buf, 0, gi * (GS / 8) + kq * kWpl + w);
#pragma unroll
      for (int i = 0; i <= MT; ++i) {
        const int cur = i & 1;
        if (i + 1 < MT) {
#pragma unroll
          for (int w = 0; w < kWpl; ++w)
            a[cur ^ 1][w] = a_frag(buf, i + 1, gi * (GS / 8) + kq * kWpl + w);
        }
        if (i < MT) {
          f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kWpl; ++w) {
            t0 = mfma32<TagF16>(a[cur][w], bq[0][w], t0);
            t1 = mfma32<TagF16>(a[cur][w], bq[1][w], t1);
          }
          t[cur][0] = t0;
          t[cur][1] = t1;
        }
        if (i > 0) {
          const int p = cur ^ 1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[i - 1][0][e] = __builtin_fmaf(t[p][0][e], s0, acc[i - 1][0][e]);
            acc[i - 1][1][e] = __builtin_fmaf(t[p][1][e], s1, acc[i - 1][1][e]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int last = kb_end - 1;
  auto clampk = [&](int k) { return k < last ? k : last; };
  // Byte offset of 16-byte activation chunk ch of block kb in row `row` of the
  // tile; with KTAIL (K % 128 == 64, g = 64) chunks past the end of K read as
  // zeros.
  auto a_off = [&](int row, int kb, int ch) {
    const uint32_t o = (uint32_t)(row0 + row) * (uint32_t)K * 2u + (uint32_t)kb * (kBK * 2) +
                       (uint32_t)ch * 16u;
    if constexpr (KTAIL) return kb * kBK + ch * 8 < K ? o : kNone;
    return o;
  };

  // Both main loops have no branch between a prefetch and the step that
  // consumes it; given one (a loop exit, a skipped tail group) the compiler
  // sinks the prefetch loads past the math down to that branch, right before
  // the wait that then drains them.
  if constexpr (DMA) {
    // ---- activations straight to LDS, two buffers, one barrier per block ------
    // DMA instruction d (wave*kDma + r) fills block rows 4d .. 4d+3; lane l
    // writes row 4d + l/16 at physical chunk l%16, i.e. logical chunk
    // (l%16) ^ (row%16).  The DMA's LDS writes are known complete only after
    // vmcnt(0), so block k+1's weights are requested together with its
    // activations at the top of step k and both are waited for at the top of
    // step k+1; the weight registers rotate by one copy per step.
    constexpr int kDma = kBM / 16;
    auto issue_a = [&](int kb, uint16_t *buf) {
#pragma unroll
      for (int r = 0; r < kDma; ++r) {
        const int d = wave * kDma + r;
        const int row = 4 * d + (lane >> 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rX, (lds_void *)(reinterpret_cast<char *>(buf) + d * 1024), 16,
            a_off(row, kb, (lane & 15) ^ (row & 15)), 0, 0, 0);
      }
    };
    BRegs cur, nxt;
    issue_a(kb_begin, sA0);
    load_b(kb_begin, nxt);
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      wait_vmem_all();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      cur = nxt;
      const bool odd = ((kb - kb_begin) & 1) != 0;
      issue_a(clampk(kb + 1), odd ? sA0 : sA1);
      load_b(clampk(kb + 1), nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute(odd ? sA1 : sA0, cur);
    }
    wait_vmem_all();
  } else {
    // ---- activations staged through registers, kWin weight blocks in flight ---
    // Every wait is a counted vmcnt on ordinary loads.  Step k writes block
    // k+1's activations (loaded during step k-1) to LDS, requests block k+2's,
    // computes block k and refills its weight slot with block k+kWin.  The
    // main loop runs whole windows of kWin steps so that every slot's refill
    // is consumed in the next iteration; the last steps follow unrolled.
    constexpr int kARounds = kBM / 16;     // 16-byte chunks per thread per block
    u32x4 areg[kARounds];
    auto load_a = [&](int kb) {
#pragma unroll
      for (int r = 0; r < kARounds; ++r) {
        const int q = tid + kThreads * r;
        areg[r] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, a_off(q >> 4, kb, q & 15), 0, 0));
      }
    };
    auto store_a = [&](uint16_t *buf) {
#pragma unroll
      for (int r = 0; r < kARounds; ++r) {
        const int q = tid + kThreads * r, row = q >> 4, ch = q & 15;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(buf) + row * (kBK * 2) +
                                   ((ch ^ (row & 15)) << 4)) = areg[r];
      }
    };
    BRegs rw[kWin];
    auto step = [&](int k, BRegs &slot) {
      const bool odd = ((k - kb_begin) & 1) != 0;
      store_a(odd ? sA0 : sA1);           // block k+1 (a copy of the last block at the end)
      load_a(clampk(k + 2));
      __builtin_amdgcn_sched_barrier(0);
      compute(odd ? sA1 : sA0, slot);
      load_b(clampk(k + kWin), slot);
      __builtin_amdgcn_sched_barrier(0);
      wait_lds_all();
      __builtin_amdgcn_s_barrier();
    };
    // The prologue ends with the issue order of a steady-state step
    // (activations, then one weight block) so the counted waits the compiler
    // derives at the loop header equal the steady-state ones.
    load_a(kb_begin);
#pragma unroll
    for (int u = 0; u < kWin - 1; ++u) load_b(clampk(kb_begin + u), rw[u]);
    store_a(sA0);
    load_a(clampk(kb_begin + 1));
    load_b(clampk(kb_begin + kWin - 1), rw[kWin - 1]);
    wait_lds_all();
    __builtin_amdgcn_s_barrier();
    int k = kb_begin;
    for (; k + kWin <= kb_end; k += kWin) {
#pragma unroll
      for (int u = 0; u < kWin; ++u) step(k + u, rw[u]);
    }
#pragma unroll
    for (int u = 0; u < kWin - 1; ++u)
      if (k + u < kb_end) step(k + u, rw[u]);
    wait_vmem_all();
  }

  // ---- split K: publish the partial tile; the last workgroup sums them --------
  // Partials are stored write-through and read back bypassing both cache
  // levels (sc0 sc1), and the per-tile counter is an atomic, so no device-scope
  // fence (a whole-L2 write-back and invalidate) is needed across XCDs.
  // vmcnt(0) orders the stores before the atomic.
  if (sk.splits > 1) {
    constexpr int kTiles = MT * 2;       // f32x4 accumulators per lane
    constexpr int kSys = 1 | 16;         // sc0 | sc1
    // layout: [tile][split][wave][16x16 tile][lane] of 16 bytes
    const uint32_t wave_bytes = (uint32_t)kTiles * 64u * 16u;
    const uint32_t tile_bytes = 4u * wave_bytes;
    const rsrc_t rP = make_rsrc(sk.partials, 0x7FFFFFF0u);
    const uint32_t lane_off = (uint32_t)wave * wave_bytes + (uint32_t)lane * 16u;
    const uint32_t mine =
        ((uint32_t)tile * (uint32_t)sk.splits + (uint32_t)split) * tile_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 v = acc[i][j];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rP,
                                               mine + (uint32_t)(i * 2 + j) * 1024u, 0, kSys);
      }
    wait_vmem_all();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&sk.counters[tile], 1u) == (uint32_t)(sk.splits - 1);
    __syncthreads();
    if (!s_last) return;
    const uint32_t base = (uint32_t)tile * (uint32_t)sk.splits * tile_bytes + lane_off;
    for (int sp = 0; sp < sk.splits; ++sp) {
      const uint32_t p = base + (uint32_t)sp * tile_bytes;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 v = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, p + (uint32_t)(i * 2 + j) * 1024u,
                                                           0, kSys));
          acc[i][j] = sp == 0 ? v : acc[i][j] + v;
        }
    }
    if (tid == 0) atomicExch(&sk.counters[tile], 0u);   // ready for the next launch
  }

  // ---- epilogue: lane (c, kq) holds rows 4*kq + e of column c of each tile ------
  constexpr int ysz = YT == (int)YType::F32 ? 4 : 2;
  const rsrc_t rY = make_rsrc(Y, (uint32_t)M * (uint32_t)N * (uint32_t)ysz);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = col0 + wave * 32 + j * 16 + c;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + i * 16 + 4 * kq + e;
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
}

template <int GS, int YT, int MT, bool DMA, bool KTAIL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_f16_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
                     const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                     int M, int N, int K, void *__restrict__ Y, SplitK sk) {
  gemm_f16_body<GS, YT, MT, DMA, KTAIL>(X, qweight, scales, zeros, M, N, K, Y, sk);
}

namespace {

// Two workgroups per CU.
constexpr int64_t kSlots = 512;

int64_t f16_rows_per_launch(int64_t N, int64_t K, int64_t bm) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  int64_t r = lim / (K * 2);
  const int64_t ry = lim / (N * 4);
  r = r < ry ? r : ry;
  return (r / bm) * bm;
}

template <int GS, int YT, int MT, bool DMA, bool KTAIL>
hipError_t f16_launch_mt(const uint16_t *X, const uint32_t *qw, const uint16_t *sc,
                         const uint8_t *zr, int64_t M, int64_t N, int64_t K, void *Y, SplitK sk,
                         hipStream_t st) {
  constexpr int64_t bm = 16 * MT;
  const int ysize = YT == (int)YType::F32 ? 4 : 2;
  const int64_t rows = sk.splits > 1 ? M : f16_rows_per_launch(N, K, bm);
  if (rows <= 0) return hipErrorInvalidValue;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    const dim3 grid((unsigned)(tiles * sk.splits));
    void *y = reinterpret_cast<char *>(Y) + m0 * N * ysize;
    gemm_f16_kernel<GS, YT, MT, DMA, KTAIL><<<grid, kThreads, 0, st>>>(X + m0 * K, qw, sc, zr, (int)mm,
                                                                (int)N, (int)K, y, sk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int GS, int YT, bool KTAIL>
hipError_t f16_go2(const uint16_t *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                   int64_t M, int64_t N, int64_t K, void *Y, int mt, SplitK sk, hipStream_t st) {
  if (mt == 2) return f16_launch_mt<GS, YT, 2, false, KTAIL>(X, qw, sc, zr, M, N, K, Y, sk, st);
  if (mt == 4) return f16_launch_mt<GS, YT, 4, false, KTAIL>(X, qw, sc, zr, M, N, K, Y, sk, st);
  return f16_launch_mt<GS, YT, 8, true, KTAIL>(X, qw, sc, zr, M, N, K, Y, sk, st);
}

// K is a multiple of the group size; only g = 64 can leave half a K block.
template <int GS, int YT>
hipError_t f16_go(const uint16_t *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                  int64_t M, int64_t N, int64_t K, void *Y, int mt, SplitK sk, hipStream_t st) {
  if constexpr (GS < kBK) {
    if (K % kBK != 0) return f16_go2<GS, YT, true>(X, qw, sc, zr, M, N, K, Y, mt, sk, st);
  }
  return f16_go2<GS, YT, false>(X, qw, sc, zr, M, N, K, Y, mt, sk, st);
}

}  // namespace

// Row tile and K split.  M <= 32 and M <= 64 take 32- and 64-row tiles (the
// weight stream dominates there), larger M the 128-row tile.  When the tiles
// cannot fill every CU's two workgroup slots, K is split into as many parts
// as still fit in one round of slots (at most 8, at least two K blocks each).
GemmPlan gemm_f16_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  p.mt = M <= 32 ? 2 : M <= 64 ? 4 : 8;
  const int64_t bm = 16 * p.mt;
  p.tiles = ((M + bm - 1) / bm) * ((N + kBN - 1) / kBN);
  const int64_t nkb = (K + kBK - 1) / kBK;
  p.splits = 1;
  if (p.tiles < kSlots) {
    int64_t sp = kSlots / p.tiles;
    const int64_t cap = nkb / 2 < 8 ? nkb / 2 : 8;
    sp = sp < cap ? sp : cap;
    p.splits = sp > 1 ? (int)sp : 1;
  }
  if (p.splits > 1) {
    p.counter_bytes = kSplitCounterBytes;
    p.workspace_bytes = p.counter_bytes + (size_t)p.tiles * p.splits * bm * kBN * 4;
  }
  return p;
}

hipError_t launch_gemm_f16(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                           const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int gs, void *Y,
                           YType yt, void *workspace, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const GemmPlan p = gemm_f16_plan(M, N, K);
  SplitK sk{1, nullptr, nullptr};
  if (p.splits > 1) {
    if (!workspace) return hipErrorInvalidValue;
    sk.splits = p.splits;
    sk.counters = reinterpret_cast<uint32_t *>(workspace);
    sk.partials = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.counter_bytes);
  }
  if (gs == 128) {
    if (yt == YType::F32) return f16_go<128, (int)YType::F32>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
    if (yt == YType::BF16) return f16_go<128, (int)YType::BF16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
    return f16_go<128, (int)YType::F16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
  }
  if (yt == YType::F32) return f16_go<64, (int)YType::F32>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
  if (yt == YType::BF16) return f16_go<64, (int)YType::BF16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
  return f16_go<64, (int)YType::F16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, st);
}

}  // namespace awq
