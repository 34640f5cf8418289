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
// Tiling for the MI355X: a 256-thread workgroup computes a BM x 128 tile of Y,
// BM = 32 * MT (MT = 1, 2, 4 or 8 MFMA row tiles per wave); each wave owns
// BM/2 x 64 (MT x 4 MFMA tiles of 16 x 16).  Small M takes a small BM so the
// matrix core does not multiply padding rows.  K advances in blocks of 128
// channels (one g128 group or two g64 groups).
//  * Split K: when the M x N tiles alone cannot fill the 256 CUs (batched
//    decode), the K blocks of each tile are divided among S workgroups.  Each
//    writes its fp32 partial tile to a workspace; the last of the S to finish
//    (a per-tile counter, reset by that workgroup) adds the S partials in
//    split order -- the same order whichever finishes last -- and runs the
//    epilogue.
//  * Activations: each BM x 128 fp16 block goes from global memory
//    straight to LDS (buffer_load_dwordx4 ... lds, no VGPR staging),
//    double-buffered in two arrays.  16-byte chunk c of row r is stored
//    at chunk c ^ (r mod 16): the 16 rows read by one 128-bit LDS access land
//    in 16 distinct bank groups.
//  * Per group, a wave reads all its A fragments (8 tiles x 32 channels) from
//    LDS once; they are MFMA-only operands, so the register allocator may keep
//    them in AGPRs.  Columns are then walked one 16-wide tile at a time: the
//    lane dequantizes its 32 codes of that column (16 VGPRs live) and runs 8
//    MFMA chains (one per M tile) whose fp32 sums are scaled into the
//    accumulator.  Each dequantized fragment feeds 8 MFMAs.
//  * Packed weights, scales and zeros bypass LDS and are prefetched one block
//    ahead into registers.
//  * All global accesses go through buffer resources: out-of-range reads return
//    zero and out-of-range writes are dropped by the hardware, so edge tiles
//    need no clamping or branches around loads.
//  * One s_barrier per block, after an explicit vmcnt(0): the data waited for
//    was issued a whole block earlier.  __syncthreads() is avoided in the loop
//    because its release fence would also drain the prefetches in flight.
//  * Block ids are remapped so each XCD works on a contiguous run of tiles
//    along N that share one activation block in that XCD's L2.
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
  // Wave layout: 2 x 2 waves of (BM/2) x 64, or (kTall) 1 x 4 waves of
  // BM x 32, where every dequantized weight fragment feeds twice as many MFMAs.
  constexpr bool kTall = false;
  constexpr int kMT = kTall ? 2 * MT : MT;  // 16x16 tiles per wave along M
  constexpr int kNT = kTall ? 2 : 4;        // 16x16 tiles per wave along N
  constexpr int kWaveCols = 16 * kNT;
  constexpr int kRowsPerWave = kBM / 4; // rows of the A block each wave fetches
  constexpr int kDma = kRowsPerWave / 4;
  // Tiles up to 128 rows stage activations through registers and keep a window
  // of kWin weight blocks in flight; the 256-row tile (search GEMMs) uses DMA.
  constexpr bool kRegA = MT <= 4 && !DENSE;
  constexpr int kWin = kGPB > 1 ? 3 : 4;

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const DeqRegs dq;
  const int wm = kTall ? 0 : wave >> 1, wn = kTall ? wave : wave & 1;
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

  if constexpr (kRegA) {
    // ---- main loop, register-staged activations --------------------------------
    // Every wait here is a counted vmcnt on ordinary loads, so the weight window
    // of kWin blocks stays in flight while the math runs.  Activations: block
    // k+1 is written to LDS during step k (its loads were issued in step k-1)
    // and block k+2 is requested; one barrier per step orders LDS writes and
    // reads.  Weights, scales and zeros: slot u holds block k, refilled with
    // block k+kWin as soon as block k has been used.
    constexpr int kARounds = kBM / 16;            // 16-byte chunks per thread per block
    u32x4 areg[kARounds];
    const rsrc_t rXa = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
    auto load_a = [&](int kb) {
#pragma unroll
      for (int r = 0; r < kARounds; ++r) {
        const int q = tid + kThreads * r, row = q >> 4, ch = q & 15;
        const uint32_t off = (uint32_t)(row0 + row) * (uint32_t)K * 2u + (uint32_t)kb * (kBK * 2) +
                             (uint32_t)ch * 16u;
        areg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rXa, off, 0, 0));
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
    // Loads are never under a branch (prefetch indices are clamped to the last
    // block; the surplus loads of the last steps are never consumed), so every
    // step issues the same sequence and the compiler's counted waits stay exact.
    BRegs rw[kWin];
    const int last = kb_end - 1;
    auto clampk = [&](int k) { return k < last ? k : last; };
    // The prologue ends with the same issue order as every step (activations,
    // then one weight block) so that the wait counts the compiler derives at
    // the loop header equal the steady-state ones.
    load_a(kb_begin);
#pragma unroll
    for (int u = 0; u < kWin - 1; ++u) load_b(clampk(kb_begin + u), rw[u]);
    store_a(sA0);
    load_a(clampk(kb_begin + 1));
    load_b(clampk(kb_begin + kWin - 1), rw[kWin - 1]);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes landed
    __builtin_amdgcn_s_barrier();
    for (int kb = kb_begin; kb < kb_end; kb += kWin) {
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int k = kb + u;
        if (k >= kb_end) break;
        const bool odd = ((k - kb_begin) & 1) != 0;
        uint16_t *buf = odd ? sA1 : sA0;
        uint16_t *nbuf = odd ? sA0 : sA1;
        store_a(nbuf);                      // block k+1 (a copy of the last block at the end)
        load_a(clampk(k + 2));
        __builtin_amdgcn_sched_barrier(0);
        compute(k, buf, rw[u]);
        load_b(clampk(k + kWin), rw[u]);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
      }
    }
  } else {
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
  }

  // ---- split K: publish the partial tile; the last workgroup sums them ------
  // The partials cross workgroups that may sit on different XCDs, whose L2s
  // are not coherent with each other.  A device-scope fence would write back
  // and invalidate a whole L2 per workgroup; instead the partials are stored
  // write-through and read back bypassing both cache levels (the sc0 sc1
  // cache-policy bits), and the per-tile counter is an atomic, which is
  // coherent across XCDs.  vmcnt(0) orders the stores before the atomic.
  // (compiled only for the tiles the plan may split: the 256-row tile's
  // registers are all taken by its main loop)
  if constexpr (MT < 8) if (sk.splits > 1) {
    constexpr int kTiles = kMT * kNT;     // f32x4 accumulators per lane
    constexpr int kSys = 1 | 16;          // sc0 | sc1: system-coherent access
    // partial layout: [tile][split][wave][16x16 tile][lane] of 16 bytes
    const uint32_t wave_bytes = (uint32_t)kTiles * 64u * 16u;
    const uint32_t tile_bytes = 4u * wave_bytes;
    const rsrc_t rP = make_rsrc(sk.partials, 0x7FFFFFF0u);
    const uint32_t lane_off = (uint32_t)wave * wave_bytes + (uint32_t)lane * 16u;
    const uint32_t mine = ((uint32_t)tile * (uint32_t)sk.splits + (uint32_t)split) * tile_bytes +
                          lane_off;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const f32x4 v = acc[i][j];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rP,
                                               mine + (uint32_t)(i * kNT + j) * 1024u, 0, kSys);
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
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const f32x4 v = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, p + (uint32_t)(i * kNT + j) * 1024u,
                                                           0, kSys));
          acc[i][j] = sp == 0 ? v : acc[i][j] + v;
        }
    }
    if (tid == 0) atomicExch(&sk.counters[tile], 0u);   // ready for the next launch
  }

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

template <class XT, int GS, int EPI, bool DENSE, int YT, int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel_small(const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
                       const uint16_t *__restrict__ Wdense, const uint16_t *__restrict__ scales,
                       const uint8_t *__restrict__ zeros, int M, int N, int K,
                       void *__restrict__ Y, const float *__restrict__ Yref,
                       double *__restrict__ partials, SplitK sk) {
  gemm_body<XT, GS, EPI, DENSE, YT, MT>(X, qweight, Wdense, scales, zeros, M, N, K, Y, Yref,
                                        partials, sk);
}

// The search's dense and loss GEMMs use the 256-row tile and no K split.
int64_t gemm_tile_count(int64_t M, int64_t N) {
  return ((M + 255) / 256) * ((N + kBN - 1) / kBN);
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


// Row tile and K split of a quantized GEMM launch.  M <= 32 and M <= 64 take
// 32- and 64-row tiles, larger M the 128-row tile (the 256-row tile needs more
// registers than one wave of two per SIMD has and spends its VALU time moving
// accumulators through AGPRs).  When the tiles
// cannot give every CU two workgroups, K is split (at most 8 ways, at least
// two K blocks per split).
static GemmPlan gemm_bf16_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  p.mt = M <= 32 ? 1 : M <= 64 ? 2 : 4;
  const int64_t bm = 32 * p.mt;
  p.tiles = ((M + bm - 1) / bm) * ((N + kBN - 1) / kBN);
  const int64_t nkb = (K + kBK - 1) / kBK;
  p.splits = 1;
  if (p.mt < 8 && p.tiles < 512) {
    int64_t sp = (512 + p.tiles - 1) / p.tiles;
    const int64_t cap = nkb / 2 < 8 ? nkb / 2 : 8;
    sp = sp < cap ? sp : cap;
    p.splits = sp > 1 ? (int)sp : 1;
  }
  if (p.splits > 1) {
    // A fixed counter region: K is split only when there are fewer than 512
    // tiles, and every plan must find its counters at the same place (the
    // partials of one shape must never overlap the counters of another).
    p.counter_bytes = kSplitCounterBytes;
    p.workspace_bytes = p.counter_bytes + (size_t)p.tiles * p.splits * bm * kBN * 4;
  }
  return p;
}

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, XType xt) {
  return xt == XType::F16 ? gemm_f16_plan(M, N, K) : gemm_bf16_plan(M, N, K);
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t a = gemm_f16_plan(M, N, K).workspace_bytes;
  const size_t b = gemm_bf16_plan(M, N, K).workspace_bytes;
  return a > b ? a : b;
}

template <class XT, int GS, int EPI, bool DENSE, int YT, int MT>
static hipError_t gemm_launch_mt(const uint16_t *X, const uint32_t *qw, const uint16_t *Wd,
                                 const uint16_t *sc, const uint8_t *zr, int64_t M, int64_t N,
                                 int64_t K, void *Y, const float *Yref, double *partials,
                                 SplitK sk, hipStream_t st) {
  constexpr int64_t bm = 32 * MT;
  const int ysize = YT == (int)YType::F32 ? 4 : 2;
  const int64_t rows = sk.splits > 1 ? M : rows_per_launch(N, K, bm);
  if (rows <= 0) return hipErrorInvalidValue;
  int64_t tile_base = 0;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    const dim3 grid((unsigned)(tiles * sk.splits));
    void *y = Y ? reinterpret_cast<char *>(Y) + m0 * N * ysize : nullptr;
    const float *yr = Yref ? Yref + m0 * N : nullptr;
    double *pp = partials ? partials + tile_base : nullptr;
    if constexpr (MT >= 4)
      gemm_kernel_big<XT, GS, EPI, DENSE, YT, MT><<<grid, kThreads, 0, st>>>(
          X + m0 * K, qw, Wd, sc, zr, (int)mm, (int)N, (int)K, y, yr, pp, sk);
    else
      gemm_kernel_small<XT, GS, EPI, DENSE, YT, MT><<<grid, kThreads, 0, st>>>(
          X + m0 * K, qw, Wd, sc, zr, (int)mm, (int)N, (int)K, y, yr, pp, sk);
    tile_base += tiles;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class XT, int GS, int EPI, bool DENSE, int YT>
static hipError_t gemm_go1(const uint16_t *X, const uint32_t *qw, const uint16_t *Wd,
                           const uint16_t *sc, const uint8_t *zr, int64_t M, int64_t N, int64_t K,
                           void *Y, const float *Yref, double *partials, int mt, SplitK sk,
                           hipStream_t st) {
  if constexpr (EPI == kEpiStore && !DENSE) {
    if (mt == 1)
      return gemm_launch_mt<XT, GS, EPI, DENSE, YT, 1>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                       partials, sk, st);
    if (mt == 2)
      return gemm_launch_mt<XT, GS, EPI, DENSE, YT, 2>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                       partials, sk, st);
    if (mt == 4)
      return gemm_launch_mt<XT, GS, EPI, DENSE, YT, 4>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                       partials, sk, st);
  }
  return gemm_launch_mt<XT, GS, EPI, DENSE, YT, 8>(X, qw, Wd, sc, zr, M, N, K, Y, Yref, partials,
                                                   sk, st);
}

template <class XT, int GS, int EPI, bool DENSE>
static hipError_t gemm_go(const uint16_t *X, const uint32_t *qw, const uint16_t *Wd,
                          const uint16_t *sc, const uint8_t *zr, int64_t M, int64_t N, int64_t K,
                          void *Y, int yt, const float *Yref, double *partials, int mt,
                          SplitK sk, hipStream_t st) {
  if (EPI == kEpiLoss || yt == (int)YType::F32)
    return gemm_go1<XT, GS, EPI, DENSE, (int)YType::F32>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                         partials, mt, sk, st);
  if (yt == (int)YType::BF16)
    return gemm_go1<XT, GS, EPI, DENSE, (int)YType::BF16>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                          partials, mt, sk, st);
  return gemm_go1<XT, GS, EPI, DENSE, (int)YType::F16>(X, qw, Wd, sc, zr, M, N, K, Y, Yref,
                                                       partials, mt, sk, st);
}

hipError_t launch_gemm(const void *X, XType xt, const uint32_t *qweight,
                       const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                       int64_t K, int gs, void *Y, YType yt, void *workspace,
                       hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (xt == XType::F16)
    return launch_gemm_f16(reinterpret_cast<const uint16_t *>(X), qweight, scales, zeros, M, N, K,
                           gs, Y, yt, workspace, st);
  const GemmPlan p = gemm_bf16_plan(M, N, K);
  SplitK sk{1, nullptr, nullptr};
  if (p.splits > 1) {
    if (!workspace) return hipErrorInvalidValue;
    sk.splits = p.splits;
    sk.counters = reinterpret_cast<uint32_t *>(workspace);
    sk.partials = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.counter_bytes);
  }
  const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
  const int y = (int)yt;
  if (xt == XType::F16)
    return gs == 128 ? gemm_go<TagF16, 128, kEpiStore, false>(x, qweight, nullptr, scales, zeros,
                                                              M, N, K, Y, y, nullptr, nullptr,
                                                              p.mt, sk, st)
                     : gemm_go<TagF16, 64, kEpiStore, false>(x, qweight, nullptr, scales, zeros,
                                                             M, N, K, Y, y, nullptr, nullptr,
                                                             p.mt, sk, st);
  return gs == 128 ? gemm_go<TagBF16, 128, kEpiStore, false>(x, qweight, nullptr, scales, zeros,
                                                             M, N, K, Y, y, nullptr, nullptr,
                                                             p.mt, sk, st)
                   : gemm_go<TagBF16, 64, kEpiStore, false>(x, qweight, nullptr, scales, zeros,
                                                            M, N, K, Y, y, nullptr, nullptr,
                                                            p.mt, sk, st);
}

hipError_t launch_gemm_dense_f32(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N,
                                 int64_t K, float *Y, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  return gemm_go<TagF16, 128, kEpiStore, true>(X, nullptr, W, nullptr, nullptr, M, N, K, Y,
                                               (int)YType::F32, nullptr, nullptr, 8,
                                               SplitK{1, nullptr, nullptr}, st);
}

hipError_t launch_gemm_loss(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales,
                            const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int gs,
                            const float *Yref, double *partials, hipStream_t st) {
  const SplitK one{1, nullptr, nullptr};
  return gs == 128 ? gemm_go<TagF16, 128, kEpiLoss, false>(A, qweight, nullptr, scales, zeros, M,
                                                           N, K, nullptr, 0, Yref, partials, 8,
                                                           one, st)
                   : gemm_go<TagF16, 64, kEpiLoss, false>(A, qweight, nullptr, scales, zeros, M,
                                                          N, K, nullptr, 0, Yref, partials, 8,
                                                          one, st);
}

}  // namespace awq
