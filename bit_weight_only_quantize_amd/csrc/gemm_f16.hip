// Batched / prefill W4A16 GEMM on gfx950 MFMA: fp16 activations, bf16 ones
// scaled into fp16 per row, and the scale search's loss GEMM.
//
// The GEMM variant of the quantized linear layer ("AWQ Advanced Usage Guide",
// "WQLinear Kernel Variants": batch sizes above one), Y = X * deq(W)^T with
// deq = (q - z) * s per group of g input channels (the pages' zero-point,
// group-wise int4 configuration).  The pages do not say how a kernel
// dequantizes.  Tiles of 64 rows and more (MFMA-bound from M = 256 on) use
// the B operand fp16((q - z) * s), the exact integer q - z times the group's
// fp16 scale rounded once (relative error at most 2^-11 per weight, within
// the output tolerance on the layer configurations: about 3e-4 relative
// Frobenius error), so the MFMAs accumulate straight into the tile.  The
// 32-row tile and the search's loss variant (EPI = 1) keep B the exact
// integer q - z and scale each group's fp32 sum; the loss variant reduces
// (Yref - Y)^2 of its tile instead of storing Y.
//
// Work split, chosen from measured MI355X rates (one wave keeps the MFMA unit
// busy when it issues about two VALU operations or fewer per 16x16x32 MFMA;
// a CU's LDS delivers about 160 bytes per clock to ds_read_b128):
//  * A workgroup owns a BM x 256 tile of Y (BM = 16 * MT rows): four waves
//    of 64 columns each for BM >= 128, eight of 32 columns for the 32- and
//    64-row tiles (two waves per SIMD), each over all BM rows.  Each packed
//    weight word is loaded and dequantized by exactly one lane and feeds MT
//    MFMAs; each activation fragment read from LDS feeds four (two with
//    eight waves).
//  * Dequantizing costs 13 VALU operations per word (8 weights): 4 and-or
//    into the mantissa of 1024.0 or 64.0, 4 packed subtractions of the biased
//    zero point (exact), 4 packed multiplies by the scale (rounded once).  A
//    block's 16 words per lane are dequantized while the previous block's
//    MFMAs run, so the VALU work overlaps the matrix core.
//  * Activations are double-buffered in LDS: 16-byte chunk c of block row r
//    lives at chunk c ^ (r % 16) ^ f(c), where f flips bit 3 for the odd lane
//    quarters of an MFMA fragment read (measured free of bank conflicts).
//    Tiles of up to 128 rows stage them through registers, so only ordinary
//    loads are in flight and counted vmcnt waits keep a window of kWin
//    weight blocks streaming from HBM while the math runs.
//  * Split K (when the M x N tiles cannot fill the CUs): every split stores
//    its fp32 partial tile and a second kernel, spread over all CUs, sums
//    them in split order (deterministic) and stores Y.
//  * The 256-row tile (large M) stages activations by LDS DMA and never
//    splits K.
//  * Tiles are visited in groups of four row tiles, row index fastest, so the
//    workgroups resident on one XCD share activation rows and weight columns
//    in that XCD's L2.
// 32-bit buffer offsets: the launcher slices M so that X and Y of one launch
// stay below 2 GiB; every access goes through a buffer resource whose range
// check turns edge-tile reads into zeros and drops edge-tile writes.

#include "awq_internal.h"
#include "device_common.h"
#include <type_traits>

namespace awq {

namespace {

constexpr int kBN = 256;          // columns per workgroup
constexpr int kBK = 128;          // input channels per K block
constexpr int kSteps = kBK / 32;  // MFMA K steps per block
constexpr int kGroupRows = 4;     // row tiles per tile group
// Waves per workgroup: eight (32 columns each, two waves per SIMD) for the
// 32- and 64-row tiles, four (64 columns each) for the larger ones, whose
// registers hold one wave per SIMD.  Eight waves measured 3-9% faster at
// M = 24-64, bit-identical; at 128 rows they spill and gain nothing.
constexpr int gemm_waves(int mt) { return mt <= 4 ? 8 : 4; }
// One workgroup per CU; K is split only when there are fewer tiles than
// slots (CUs).
constexpr int kSlots = 256;
constexpr int kMaxSplits = 16;    // K splits per tile (the reduction loads them all at once)
constexpr uint32_t kNone = 0xFFFFFFFFu;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(0), expcnt and lgkmcnt at their maxima.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Physical 16-byte chunk of logical chunk ch in block row `row`: an XOR with
// the row, and bit 3 flipped by bit KQ_BIT of ch.
template <int KQ_BIT>
__device__ __forceinline__ int a_chunk(int row, int ch) {
  return ch ^ (row & 15) ^ (((ch >> KQ_BIT) & 1) << 3);
}

// Logical chunk held by physical chunk p of block row `row` (inverse of
// a_chunk: bit KQ_BIT is left alone by the bit-3 flip).
template <int KQ_BIT>
__device__ __forceinline__ int a_chunk_inv(int row, int p) {
  const int t = p ^ (row & 15);
  return t ^ (((t >> KQ_BIT) & 1) << 3);
}

// Instruction order of one row tile (for the scheduler): each MFMA followed
// by up to V VALU operations.  One wave issues in order, so VALU work
// clustered after the MFMAs would leave the matrix core idle.
template <int M, int V>
__device__ __forceinline__ void tile_order() {
  if constexpr (M > 0) {
    tile_order<M - 1, V>();
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);          // V VALU
  }
}

// Row and column tile of tile index t: groups of kGroupRows row tiles, row
// index fastest within a group.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per = kGroupRows * tiles_n;
  const int grp = t / per, first = grp * kGroupRows;
  const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
  const int r = t - grp * per;
  tm = first + r % rows;
  tn = r / rows;
}

}  // namespace

// EPI: 0 stores Y; 1 (the search's loss) reduces (Yref - Y)^2 of the tile to
// one fp64 partial instead of storing Y.  The B operand is the exact integer
// q - z with the group scale applied to fp32 group sums for the loss and for
// the 32-row tile (batched decode, where the VALU work per MFMA is highest
// anyway and exact products keep the error independent of the activations'
// mean); larger tiles use fp16((q - z) * s).
template <int GS, int YT, int MT, bool KTAIL, bool BF16X, int EPI, int NW>
__device__ __forceinline__ void gemm_f16_body(const uint16_t *__restrict__ X,
                                              const uint32_t *__restrict__ qweight,
                                              const uint16_t *__restrict__ scales,
                                              const uint8_t *__restrict__ zeros, int M, int N,
                                              int K, void *__restrict__ Y, SplitK sk,
                                              const float *__restrict__ rowf,
                                              const float *__restrict__ Yref,
                                              double *__restrict__ partials) {
  constexpr bool kExact = EPI == 1 || MT <= 2;
  constexpr int kBM = 16 * MT;
  constexpr int kNTw = 16 / NW;      // 16-column MFMA tiles per wave
  constexpr int kThr = 64 * NW;
  using SZV = std::conditional_t<kNTw == 4, u32x4, u32x2>;
  constexpr int kWpl = GS / 32;      // packed words per lane per group and column
  constexpr int kGPB = kBK / GS;     // groups per K block
  // Chunk bit whose value flips bit 3 of the physical chunk: 2 for both group
  // sizes.  (With g = 64 the lane quarter's lowest bit sits at chunk bit 1,
  // but flipping on it measured 39% of LDS cycles with bank conflicts, bit 2
  // 2%: rocprofv3 SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE.)
  constexpr int kKqBit = 2;
  constexpr int kWin = MT >= 8 ? 2 : 4;   // weight blocks in flight (even: bq buffers alternate)
  constexpr int kWords = kNTw * kSteps;         // packed words per lane per block
  constexpr int kWordsPerTile = kWords / MT;    // dequantized alongside each row tile
  // The 256-row tile's 256 accumulators fill the AGPRs: its activations go to
  // LDS by DMA (buffer_load ... lds), without staging registers.
  constexpr bool kDMA = MT == 16;
  static_assert(!kDMA || NW == 4, "the DMA tile runs four waves");
  // (bf16 input reaches it already scaled and converted to fp16 by the row
  // prescan; only the epilogue's row factors remain)
  static_assert(!(kDMA && kExact), "the 256-row tile stores Y");

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint32_t sSZ0[256 * kGPB];
  __shared__ __attribute__((aligned(16))) uint32_t sSZ1[256 * kGPB];

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
  tile_coords(tile, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * kBM, col0 = tn * kBN;

  const int G = K / GS;
  const int nkb = (K + kBK - 1) / kBK;
  const int kb_begin = (int)((int64_t)split * nkb / sk.splits);
  const int kb_end = (int)((int64_t)(split + 1) * nkb / sk.splits);

  // ---- packed weights of one K block (registers) ------------------------------
  // Lane (c, kq) holds, for column tile j, words kq*kWpl .. kq*kWpl+kWpl-1 of
  // each group of column col0 + 16*kNTw*wave + 16*j + c: channels
  // 8*(kq*kWpl + w) .. +7 of the group, for MFMA step gi*kWpl + w.
  const uint32_t lane_col = (uint32_t)(col0 + wave * 16 * kNTw + c);
  const rsrc_t rQ = make_rsrc(qweight, (uint32_t)N * (uint32_t)K / 2u);
  const uint32_t q_lane = lane_col * (uint32_t)(K / 2) + (uint32_t)(kq * kWpl * 4);
  struct Raw {
    uint32_t w[kNTw][kGPB][kWpl];
  };
  // Column tile j of block kb (one load).  With KTAIL (K % 128 == 64, g = 64)
  // a group past the end of K reads zero weights and, below, zero scale and
  // activations: it adds nothing.
  auto load_w = [&](int kb, int j, Raw &r) {
#pragma unroll
    for (int gi = 0; gi < kGPB; ++gi) {
      const uint32_t g = (uint32_t)(kb * kGPB + gi);
      const bool in_k = !KTAIL || g < (uint32_t)G;
      const uint32_t qo =
          in_k ? q_lane + (uint32_t)(16 * j) * (uint32_t)(K / 2) + g * (GS / 2) : kNone;
      if constexpr (kWpl == 4) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
#pragma unroll
        for (int w = 0; w < kWpl; ++w) r.w[j][gi][w] = v[w];
      } else {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rQ, qo, 0, 0));
#pragma unroll
        for (int w = 0; w < kWpl; ++w) r.w[j][gi][w] = v[w];
      }
    }
  };

  // ---- scales and zero points: one column per thread, handed over in LDS ------
  // Thread t loads column col0 + t's scale(s) and zero point(s) of a block
  // (one or two loads instead of one per lane and column tile) and stores
  // them as u32 (zero << 16 | scale) at [group][wave][c][j] with
  // t = 16 * kNTw * wave + 16 * j + c, so that lane (c, kq) reads its kNTw
  // column tiles' values with one LDS read per group.  (Eight waves: the
  // first four load and store, one thread per column of the tile.)
  const rsrc_t rS = make_rsrc(scales, (uint32_t)N * (uint32_t)G * 2u);
  // no zeros (the symmetric grid): every zero load reads 0, and 8 is added
  const rsrc_t rZ = make_rsrc(zeros, zeros ? (uint32_t)N * (uint32_t)G : 0u);
  const uint32_t zfix = zeros ? 0u : (8u << 16);
  const uint32_t sz_col = (uint32_t)(col0 + tid) * (uint32_t)G;
  struct SZ {
    uint32_t sc;     // kGPB scales: u16, or two u16 in one u32 (g = 64)
    uint32_t zr;     // kGPB zero points: u8, or two u8 in one u16 (g = 64)
    uint16_t sc1;    // second group (KTAIL only: loaded separately)
    uint8_t zr1;
  };
  auto load_sz = [&](int kb, SZ &r) {
    const uint32_t g = (uint32_t)(kb * kGPB);
    if constexpr (kGPB == 1) {
      r.sc = __builtin_amdgcn_raw_buffer_load_b16(rS, (sz_col + g) * 2u, 0, 0);
      r.zr = __builtin_amdgcn_raw_buffer_load_b8(rZ, sz_col + g, 0, 0);
    } else if constexpr (!KTAIL) {
      // G even and g even: both groups' scales (4 bytes) and zeros (2 bytes)
      // are naturally aligned.
      r.sc = __builtin_amdgcn_raw_buffer_load_b32(rS, (sz_col + g) * 2u, 0, 0);
      r.zr = __builtin_amdgcn_raw_buffer_load_b16(rZ, sz_col + g, 0, 0);
    } else {
      const uint32_t o1 = g + 1 < (uint32_t)G ? sz_col + g + 1 : kNone / 2u;
      r.sc = __builtin_amdgcn_raw_buffer_load_b16(rS, (sz_col + g) * 2u, 0, 0);
      r.zr = __builtin_amdgcn_raw_buffer_load_b8(rZ, sz_col + g, 0, 0);
      r.sc1 = __builtin_amdgcn_raw_buffer_load_b16(rS, o1 * 2u, 0, 0);
      r.zr1 = __builtin_amdgcn_raw_buffer_load_b8(rZ, o1, 0, 0);
    }
  };
  const bool sz_thread = NW == 4 || tid < 256;        // one thread per column of the tile
  const int sz_slot = NW == 4 ? ((wave * 16 + c) * 4 + kq) * 4   // this thread's column: j = kq
                              : (((tid / (16 * kNTw)) * 16 + (tid & 15)) * kNTw + (tid / 16) % kNTw) * 4;
  auto store_sz = [&](uint32_t *buf, const SZ &r) {
    if constexpr (kGPB == 1) {
      buf[sz_slot / 4] = (((uint32_t)(uint8_t)r.zr << 16) + zfix) | (uint16_t)r.sc;
    } else if constexpr (!KTAIL) {
      buf[sz_slot / 4] = (((r.zr & 0xFFu) << 16) + zfix) | (r.sc & 0xFFFFu);
      buf[256 + sz_slot / 4] = (((r.zr & 0xFF00u) << 8) + zfix) | (r.sc >> 16);
    } else {
      buf[sz_slot / 4] = (((uint32_t)(uint8_t)r.zr << 16) + zfix) | (uint16_t)r.sc;
      buf[256 + sz_slot / 4] = (((uint32_t)r.zr1 << 16) + zfix) | (uint32_t)r.sc1;
    }
  };

  // ---- dequantized B fragments of one block: bq[j][step] ------------------------
  typedef u32x4 BQ[kNTw][kSteps];
  // Words (j, gi, *) of a block: fp16((q - z) * s) of 8 channels each, in the
  // MFMA B-operand order; sz is the column's (zero << 16 | scale).
  auto deq_word = [&](const Raw &r, uint32_t sz, int j, int gi, int w, BQ &out) {
    const DeqF16 deq(sz >> 16);
    const u32x4 e = deq(r.w[j][gi][w], dq);
    if constexpr (kExact) {
      out[j][gi * kWpl + w] = e;        // q - z exactly; the scale comes later
      return;
    }
    const uint32_t s1 = sz & 0xFFFFu;
    const f16x2 s2 = __builtin_bit_cast(f16x2, s1 | (s1 << 16));
    // (scalar copies first: bit-casting an element of a vector lvalue reads
    // the vector's first element with this compiler)
    const uint32_t e0 = e[0], e1 = e[1], e2 = e[2], e3 = e[3];
    out[j][gi * kWpl + w] =
        u32x4{__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, e0) * s2),
              __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, e1) * s2),
              __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, e2) * s2),
              __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, e3) * s2)};
  };
  auto read_sz = [&](const uint32_t *buf, int gi) {
    return *reinterpret_cast<const SZV *>(buf + gi * 256 + (wave * 16 + c) * kNTw);
  };

  f32x4 acc[MT][kNTw];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < kNTw; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A fragment: 16-row tile i, logical 16-byte chunk ch of the block row.
  auto a_frag = [&](const uint16_t *buf, int i, int ch) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(buf) +
                                            (i * 16 + c) * (kBK * 2) +
                                            (a_chunk<kKqBit>(c, ch) << 4));
  };
  auto a_ch = [&](int st) { return (st / kWpl) * (GS / 8) + kq * kWpl + (st % kWpl); };

  const rsrc_t rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int last = kb_end - 1;
  auto clampk = [&](int k) { return k < last ? k : last; };

  // ---- activations staged through registers ----------------------------------
  constexpr int kARounds = kBM * 16 / kThr;   // 16-byte chunks per thread per block
  u32x4 areg[kARounds];
  auto load_a1 = [&](int kb, int r) {
    const int q = tid + kThr * r, row = q >> 4, ch = q & 15;
    uint32_t off = (uint32_t)(row0 + row) * (uint32_t)K * 2u + (uint32_t)kb * (kBK * 2) +
                   (uint32_t)ch * 16u;
    if constexpr (KTAIL) off = kb * kBK + ch * 8 < K ? off : kNone;   // zeros past K
    areg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
  };
  // bf16 activations: chunk r's 8 values times its row's power-of-two factor
  // (exact), converted to fp16: exact for every value in fp16's normal range,
  // which the factor guarantees for the row's largest value; smaller values
  // below that range are truncated to fp16 subnormals.
  float rf[kARounds];
  if constexpr (BF16X && !kDMA) {
    const rsrc_t rR = make_rsrc(rowf, (uint32_t)M * 4u);
#pragma unroll
    for (int r = 0; r < kARounds; ++r) {
      const uint32_t row = (uint32_t)(row0 + ((tid + kThr * r) >> 4));
      rf[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, row * 4u, 0, 0));
    }
  }
  auto store_a1 = [&](uint16_t *buf, int r) {
    const int q = tid + kThr * r, row = q >> 4, ch = q & 15;
    u32x4 v = areg[r];
    if constexpr (BF16X) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t u = v[x];
        const float lo = __builtin_bit_cast(float, u << 16) * rf[r];
        const float hi = __builtin_bit_cast(float, u & 0xFFFF0000u) * rf[r];
        v[x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      }
    }
    *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(buf) + row * (kBK * 2) +
                               (a_chunk<kKqBit>(row, ch) << 4)) = v;
  };
  auto store_a = [&](uint16_t *buf) {
#pragma unroll
    for (int r = 0; r < kARounds; ++r) store_a1(buf, r);
  };
  // DMA r of this wave (kDMA): block rows 4d .. 4d+3, d = wave + 4r, 1 KiB.
  // Lane l writes physical chunk l & 15 of row 4d + (l >> 4), so it loads the
  // logical chunk that a_chunk maps there.
  typedef __attribute__((address_space(3))) void lds_t;
  auto dma_a1 = [&](uint16_t *buf, int kb, int r) {
    const int d = wave + 4 * r, row = 4 * d + (lane >> 4);
    const int ch = a_chunk_inv<kKqBit>(row, lane & 15);
    uint32_t off = (uint32_t)(row0 + row) * (uint32_t)K * 2u + (uint32_t)kb * (kBK * 2) +
                   (uint32_t)ch * 16u;
    if constexpr (KTAIL) off = kb * kBK + ch * 8 < K ? off : kNone;   // zeros past K
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_t *)(reinterpret_cast<char *>(buf) + d * 1024),
                                             16, off, 0, 0, 0);
  };

  // ---- main loop ------------------------------------------------------------------
  // Block b's data moves in stages: its activations are loaded during step
  // b-2 and written to LDS during step b-1; its weights' scales are loaded
  // during step b-3 and written to LDS at the start of step b-2; its packed weights are loaded during
  // step b-kWin; its words are dequantized during step b-1; its MFMAs run in
  // step b.  One barrier per step (at its end) orders every LDS write before
  // the reads of the next step.  Each step issues its 16-byte and smaller
  // prefetch loads spread over the row tiles, between MFMAs: a load takes
  // tens of clocks to issue, and one wave per SIMD stalls on each.  Every wait
  // is a counted vmcnt on ordinary loads.  The main loop runs whole windows
  // of kWin steps so that no branch separates a prefetch from the step that
  // consumes it (given one, the compiler sinks the prefetch loads down to it,
  // right before the wait that then drains them); the last steps follow
  // unrolled.
  constexpr int kLoads = kARounds + kNTw + 1;     // prefetch loads per step
  // row tiles that issue them: all, or with the DMA the first half, so the
  // last ones still have half a step to land before the step's vmcnt(0)
  constexpr int kIssueTiles = kDMA ? MT / 2 : MT;
  Raw rw[kWin];
  BQ bq[2];
  SZ szr;
  SZV szc[2][kGPB];                      // exact path: blocks' scales, by step parity
  // Load n of a step: scales first and activations next (both are needed at
  // the start of the next step), then the weight window's refill.  Each
  // activation chunk's register first goes to LDS (block k+1, into the
  // buffer this step does not read), then is refilled with block k+2's chunk.
  auto issue = [&](int n, int k, int u, uint16_t *nbuf) {
    if constexpr (kDMA) {
      // weights first: every load of a step must land by its end (the DMA
      // is waited for with vmcnt(0)); then scales, then block k+1's
      // activations straight into the buffer this step does not read
      if (n < kNTw) load_w(clampk(k + kWin), n, rw[u]);
      else if (n == kNTw) load_sz(clampk(k + 3), szr);
      else dma_a1(nbuf, clampk(k + 1), n - kNTw - 1);
      return;
    }
    if (n == 0) {
      if (sz_thread) load_sz(clampk(k + 3), szr);
    } else if (n <= kARounds) {
      store_a1(nbuf, n - 1);
      load_a1(clampk(k + 2), n - 1);
    } else {
      load_w(clampk(k + kWin), n - 1 - kARounds, rw[u]);
    }
  };
  auto step = [&](int k, int u) {
    const int p = u & 1;
    const bool odd = ((k - kb_begin) & 1) != 0;
    uint16_t *abuf = odd ? sA1 : sA0;
    if (sz_thread) store_sz(((k - kb_begin) & 1) ? sSZ1 : sSZ0, szr);    // block k+2
    const uint32_t *zbuf = ((k - kb_begin) & 1) ? sSZ0 : sSZ1;   // block k+1
    SZV szv[kGPB];
#pragma unroll
    for (int gi = 0; gi < kGPB; ++gi) szv[gi] = read_sz(zbuf, gi);
    float sk[kGPB][kNTw];                 // block k's scales (exact path)
    if constexpr (kExact) {
#pragma unroll
      for (int gi = 0; gi < kGPB; ++gi) {
        const SZV zz = szc[p][gi];
#pragma unroll
        for (int j = 0; j < kNTw; ++j) {
          const uint32_t z1 = zz[j];
          sk[gi][j] = half_bits_to_float((uint16_t)(z1 & 0xFFFFu));
        }
        szc[p ^ 1][gi] = szv[gi];
      }
    }
    const Raw &nx = rw[(u + 1) % kWin];
    u32x4 a[2][kSteps];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) a[0][st] = a_frag(abuf, 0, a_ch(st));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int cur = i & 1;
      if (i + 1 < MT) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) a[cur ^ 1][st] = a_frag(abuf, i + 1, a_ch(st));
      }
      if constexpr (kExact) {
#pragma unroll
        for (int gi = 0; gi < kGPB; ++gi) {
          f32x4 t[kNTw];
#pragma unroll
          for (int j = 0; j < kNTw; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kWpl; ++w)
#pragma unroll
            for (int j = 0; j < kNTw; ++j)
              t[j] = mfma32<TagF16>(a[cur][gi * kWpl + w], bq[p][j][gi * kWpl + w], t[j]);
#pragma unroll
          for (int j = 0; j < kNTw; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j][e] = __builtin_fmaf(t[j][e], sk[gi][j], acc[i][j][e]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
#pragma unroll
          for (int j = 0; j < kNTw; ++j)
            acc[i][j] = mfma32<TagF16>(a[cur][st], bq[p][j][st], acc[i][j]);
      }
      // dequantize words [i*kWordsPerTile, (i+1)*kWordsPerTile) of block k+1
#pragma unroll
      for (int q = i * kWordsPerTile; q < (i + 1) * kWordsPerTile; ++q) {
        const int j = q / kSteps, st = q % kSteps, gi = st / kWpl, w = st % kWpl;
        const SZV zz = szv[gi];
        const uint32_t sz = zz[j];
        deq_word(nx, sz, j, gi, w, bq[p ^ 1]);
      }
      if (i < kIssueTiles) {
#pragma unroll
        for (int n = i * kLoads / kIssueTiles; n < (i + 1) * kLoads / kIssueTiles; ++n)
          issue(n, k, u, odd ? sA0 : sA1);
      }
      tile_order<kNTw * kSteps, (kWordsPerTile * (kExact ? 9 : 13) + (kExact ? 4 * kNTw * kGPB : 0) +
                                kNTw * kSteps - 1) / (kNTw * kSteps) + 1>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kDMA)
      __builtin_amdgcn_s_waitcnt(0x0070);     // vmcnt(0) lgkmcnt(0): the DMA has landed
    else
      wait_lds_all();
    __builtin_amdgcn_s_barrier();
  };

  // Prologue: blocks kb0 .. kb0+kWin-1's weights, kb0's and kb0+1's scales in
  // LDS, kb0+2's in registers, kb0's activations in LDS and kb0+1's in
  // registers, kb0 dequantized.
  {
    const int kb0 = kb_begin;
    if constexpr (kDMA) {
#pragma unroll
      for (int r = 0; r < kARounds; ++r) dma_a1(sA0, kb0, r);
    } else {
#pragma unroll
      for (int r = 0; r < kARounds; ++r) load_a1(kb0, r);
    }
#pragma unroll
    for (int u = 0; u < kWin; ++u)
#pragma unroll
      for (int j = 0; j < kNTw; ++j) load_w(clampk(kb0 + u), j, rw[u]);
    SZ s0, s1;
    if (sz_thread) {
      load_sz(kb0, s0);
      load_sz(clampk(kb0 + 1), s1);
      load_sz(clampk(kb0 + 2), szr);
    }
    if constexpr (!kDMA) {
      store_a(sA0);
#pragma unroll
      for (int r = 0; r < kARounds; ++r) load_a1(clampk(kb0 + 1), r);
    }
    if (sz_thread) {
      store_sz(sSZ0, s0);
      store_sz(sSZ1, s1);
    }
    if constexpr (kDMA)
      __builtin_amdgcn_s_waitcnt(0x0070);
    else
      wait_lds_all();
    __builtin_amdgcn_s_barrier();
    SZV szv[kGPB];
#pragma unroll
    for (int gi = 0; gi < kGPB; ++gi) szv[gi] = read_sz(sSZ0, gi);
#pragma unroll
    for (int gi = 0; gi < kGPB; ++gi) szc[0][gi] = szv[gi];
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const int j = q / kSteps, st = q % kSteps, gi = st / kWpl, w = st % kWpl;
      const SZV zz = szv[gi];
      const uint32_t sz = zz[j];
      deq_word(rw[0], sz, j, gi, w, bq[0]);
    }
  }
  int k = kb_begin;
  for (; k + kWin <= kb_end; k += kWin) {
#pragma unroll
    for (int u = 0; u < kWin; ++u) step(k + u, u);
  }
#pragma unroll
  for (int u = 0; u < kWin - 1; ++u)
    if (k + u < kb_end) step(k + u, u);
  wait_vmem_all();

  // ---- split K: store this split's partial tile --------------------------------
  // Layout [tile][split][wave][16x16 tile][lane] of 16 bytes.  Plain stores:
  // the kernel boundary makes them visible to the reduction kernel, which
  // sums the splits in order and stores Y (and reads no row tile that starts
  // at or past row M).  (Not compiled for the 256-row tile, which the plan
  // never splits.)
  if (!kDMA && sk.splits > 1) {
    constexpr int kTiles = MT * kNTw;    // f32x4 accumulators per lane
    const uint32_t wave_bytes = (uint32_t)kTiles * 64u * 16u;
    const uint32_t tile_bytes = (uint32_t)NW * wave_bytes;
    const rsrc_t rP = make_rsrc(sk.partials, 0x7FFFFFF0u);
    const uint32_t mine = ((uint32_t)tile * (uint32_t)sk.splits + (uint32_t)split) * tile_bytes +
                          (uint32_t)wave * wave_bytes + (uint32_t)lane * 16u;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      // For the 32-row tile (M <= 32: decode batches, where rows 16..31 are
      // often all past M) a row tile that starts at or past M stores out of
      // range, where the stores are dropped.  A branch here, or the test in
      // larger tiles, changed the code of their main loop or epilogue and
      // cost more than it saved.
      const bool live = MT > 2 || row0 + i * 16 < M;   // uniform
#pragma unroll
      for (int j = 0; j < kNTw; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, acc[i][j]), rP,
            live ? mine + (uint32_t)(i * kNTw + j) * 1024u : 0x7FFFFFF0u, 0, 0);
    }
    return;
  }

  // ---- epilogue: lane (c, kq) holds rows 4*kq + e of column c of each tile ------
  if constexpr (EPI == 1) {
    // sum of (Yref - Y)^2 over the tile, fp64, in a fixed order (lanes, then
    // waves); rows >= M and columns >= N read 0 and have Y = 0
    const rsrc_t rR = make_rsrc(Yref, (uint32_t)M * (uint32_t)N * 4u);
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < kNTw; ++j) {
      const int n = col0 + wave * 16 * kNTw + j * 16 + c;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + i * 16 + 4 * kq + e;
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
    if (tid == 0) {
      double t = wsum[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += wsum[w];
      partials[tile] = t;
    }
    return;
  }
  if constexpr (BF16X) {
    // undo the rows' activation factors (exact powers of two; rows past M
    // read 0 and keep their unused values)
    const rsrc_t rR = make_rsrc(rowf, (uint32_t)M * 4u);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const f32x4 f = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, (uint32_t)(row0 + i * 16 + 4 * kq) * 4u, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fe = f[e];
        // 1 / 2^k exactly: the exponent field mirrored around the bias
        const float inv = fe > 0.0f ? __builtin_bit_cast(float, 0x7F000000u - __builtin_bit_cast(uint32_t, fe))
                                    : 1.0f;
#pragma unroll
        for (int j = 0; j < kNTw; ++j) acc[i][j][e] *= inv;
      }
    }
  }
  constexpr int ysz = YT == (int)YType::F32 ? 4 : 2;
  const rsrc_t rY = make_rsrc(Y, (uint32_t)M * (uint32_t)N * (uint32_t)ysz);
  if constexpr (YT != (int)YType::F32 && MT >= 8) {
    // 16-bit output of the 128- and 256-row tiles through LDS: an MFMA result
    // lane holds 4 rows of one column, so direct stores write 32-byte pieces
    // of 4 rows each (measured about twice the bytes of Y reaching HBM).
    // Each wave turns its 16 * kNTw columns, half the rows at a time, into
    // rows in LDS (with four waves: 128 bytes, 144 apart, so the 4 row groups
    // of a store start 16 banks apart) and stores them as whole 16-byte
    // pieces, kLpr lanes per row.  The first half of the waves use sA0, the
    // rest sA1, once every wave is past the main loop.
    constexpr int kRowB = 16 * kNTw * 2 + 16;
    constexpr int kLpr = 2 * kNTw;                      // lanes per row: 16 bytes each
    constexpr int kHalf = kBM / 2;
    static_assert(NW / 2 * kHalf * kRowB <= kBM * kBK * 2, "epilogue staging exceeds the A buffers");
    __syncthreads();
    char *region = reinterpret_cast<char *>(wave < NW / 2 ? sA0 : sA1) + (wave % (NW / 2)) * kHalf * kRowB;
    const int nb = col0 + wave * 16 * kNTw;
    const bool vec = (N & 7) == 0;                      // 16-byte aligned rows of Y
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = h * (MT / 2); i < (h + 1) * (MT / 2); ++i)
#pragma unroll
        for (int j = 0; j < kNTw; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = (i - h * (MT / 2)) * 16 + 4 * kq + e;
            const float v = acc[i][j][e];
            *reinterpret_cast<uint16_t *>(region + r * kRowB + (16 * j + c) * 2) =
                YT == (int)YType::F16 ? float_to_half_bits(v) : float_to_bf16_bits(v);
          }
      __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0): this wave's writes landed
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < kHalf * kLpr / 64; ++it) {
        const int r = it * (64 / kLpr) + lane / kLpr, q = lane % kLpr;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(region + r * kRowB + q * 16);
        const int m = row0 + h * kHalf + r, n = nb + 8 * q;
        if (m >= M || n >= N) continue;
        const uint32_t o = ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 2u;
        if (vec && n + 8 <= N) {
          __builtin_amdgcn_raw_buffer_store_b128(v, rY, o, 0, 0);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (n + t < N)
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[t >> 1] >> (16 * (t & 1))), rY,
                                                    o + 2u * t, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);                // reads done before the next half
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kNTw; ++j) {
    const int n = col0 + wave * 16 * kNTw + j * 16 + c;
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

// NW / 4 waves per SIMD: accumulators, two dequantized blocks and the weight
// window (two or four blocks) live in registers.
template <int GS, int YT, int MT, bool KTAIL, bool BF16X, int EPI, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_f16_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ qweight,
                     const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                     int M, int N, int K, void *__restrict__ Y, SplitK sk,
                     const float *__restrict__ rowf, const float *__restrict__ Yref,
                     double *__restrict__ partials) {
  gemm_f16_body<GS, YT, MT, KTAIL, BF16X, EPI, NW>(X, qweight, scales, zeros, M, N, K, Y, sk, rowf,
                                               Yref, partials);
}

// Second pass of a split-K GEMM: one thread per 16-byte partial fragment
// (lane l of 16x16 tile t of wave w of a tile) sums the splits' fragments in
// split order and stores its four outputs (rows 4*(l >> 4) + e of column
// l & 15).  Every CU takes a share of the partials: summing them in the GEMM
// kernel's last workgroup of each tile was bound by that one CU's load
// bandwidth (measured 25% slower at 6 splits, 3% at 2).
template <int YT, int MT, bool BF16X, int NS, int NW>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partials,
                                                            int splits, int M, int N,
                                                            void *__restrict__ Y,
                                                            const float *__restrict__ rowf) {
  constexpr int kNTw = 16 / NW;
  constexpr int kTiles = MT * kNTw;    // fragments per GEMM wave
  constexpr int kBM = 16 * MT;
  const int tiles_n = (N + kBN - 1) / kBN, tiles_m = (M + kBM - 1) / kBM;
  // kTiles workgroups per output tile (4 GEMM waves x kTiles fragments x 64
  // lanes): workgroup b < kTiles of a tile takes the fragments of GEMM wave
  // b / MT in row tile i = b % MT, its own wave j those of 16x16 tile (i, j).
  // Everything but j and the lane is uniform per workgroup, so the tile's
  // coordinates and the dead-row test are scalar work.
  const int tile = (int)(blockIdx.x / (4 * MT));
  if (tile >= tiles_m * tiles_n) return;
  // fragment f of the tile, in the partials' [wave][i][j] order
  const int f = (int)(blockIdx.x % (4 * MT)) * 4 + (threadIdx.x >> 6);
  const int wave = f / kTiles, i = (f / kNTw) % MT, j = f % kNTw;
  const int lane = threadIdx.x & 63;
  const int t = i * kNTw + j;
  // one row of tiles (M within one tile: the common split-K case) needs no
  // division before the loads can start
  int tm = 0, tn = tile;
  if (tiles_m > 1) tile_coords(tile, tiles_m, tiles_n, tm, tn);
  // a row tile that starts at or past row M holds nothing to sum (and was
  // not stored by the 32-row tile)
  if (tm * kBM + i * 16 >= M) return;
  const int c = lane & 15, kq = lane >> 4;
  // [tile][split][wave][t][lane] of 16 bytes (below 32 MiB: K is split only
  // for fewer than kSlots tiles of at most 128 x 256)
  constexpr uint32_t kSplitBytes = (uint32_t)NW * kTiles * 64u * 16u;
  const rsrc_t rP = make_rsrc(partials, (uint32_t)(tiles_m * tiles_n) * (uint32_t)splits * kSplitBytes);
  const uint32_t base = ((uint32_t)tile * (uint32_t)splits * (uint32_t)(NW * kTiles) +
                         (uint32_t)(wave * kTiles + t)) * 1024u + (uint32_t)lane * 16u;
  // Every split's load is issued before the first is used (a loop adding
  // each as it arrived waited for them one by one).  NS >= splits is the
  // launch's bucket (2, 4, 8 or 16) so few loads are wasted; splits past the
  // last read out of range (zero) and are skipped, so the sum runs in split
  // order.
  f32x4 part[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const uint32_t o = sp < splits ? base + (uint32_t)sp * kSplitBytes : 0x7FFFFFF0u;
    part[sp] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, o, 0, 0));
  }
  f32x4 sum = part[0];
#pragma unroll
  for (int sp = 1; sp < NS; ++sp)
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] = sp < splits ? sum[e] + part[sp][e] : sum[e];
  const int n = tn * kBN + wave * 16 * kNTw + j * 16 + c;
  if (n >= N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = tm * kBM + i * 16 + 4 * kq + e;
    if (m >= M) break;
    float v = sum[e];
    if constexpr (BF16X) {
      const float f = rowf[m];     // a power of two: its inverse is exact
      v *= f > 0.0f ? __builtin_bit_cast(float, 0x7F000000u - __builtin_bit_cast(uint32_t, f)) : 1.0f;
    }
    const int64_t o = (int64_t)m * N + n;
    if constexpr (YT == (int)YType::F16)
      reinterpret_cast<uint16_t *>(Y)[o] = float_to_half_bits(v);
    else if constexpr (YT == (int)YType::BF16)
      reinterpret_cast<uint16_t *>(Y)[o] = float_to_bf16_bits(v);
    else
      reinterpret_cast<float *>(Y)[o] = v;
  }
}

// Per-row activation factor for bf16 input: the power of two that brings the
// row's largest magnitude into [2^14, 2^15), so every value of the row is
// within fp16's range.  Scaled values of at least 2^-17 (every value at least
// 2^-31 times the row's largest) are fp16 numbers and keep their full 8-bit
// precision; smaller ones fall on fp16's subnormal grid (spacing 2^-24) and
// are truncated, with an absolute error below 2^-38 times the row's largest
// magnitude (exponent capped to stay a normal fp32); 1 for rows that are all
// zero or hold inf or NaN.  One workgroup per row.  With Xh, the row is also
// written there multiplied by its factor and converted to fp16 (round toward
// zero, as the GEMM's own staging does), for the 256-row tile.
__global__ __launch_bounds__(256) void bf16_row_factor_kernel(const uint16_t *__restrict__ X,
                                                              int K, float *__restrict__ rowf,
                                                              uint16_t *__restrict__ Xh) {
  __shared__ float red[4];
  __shared__ float fsh;
  const int64_t row = blockIdx.x;
  const rsrc_t rX = make_rsrc(X + row * K, (uint32_t)K * 2u);
  float mx = 0.0f;
  for (int c = threadIdx.x; c * 8 < K; c += 256) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, (uint32_t)c * 16u, 0, 0));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t u = v[x];
      mx = __builtin_fmaxf(mx, __builtin_fabsf(__builtin_bit_cast(float, u << 16)));
      mx = __builtin_fmaxf(mx, __builtin_fabsf(__builtin_bit_cast(float, u & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    float f = 1.0f;
    if (m > 0.0f && __builtin_isfinite(m)) {
      // floor(log2 m) from the fp32 bits (bf16 subnormals widen to fp32
      // subnormals: biased exponent 0, read here as -127, so they scale up by
      // at most the cap)
      const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
      int e = 14 - ex;                                  // m * 2^e in [2^14, 2^15)
      e = e > 126 ? 126 : e;
      f = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
    }
    rowf[row] = f;
    fsh = f;
  }
  if (!Xh) return;
  __syncthreads();
  const float f = fsh;
  const rsrc_t rH = make_rsrc(Xh + row * K, (uint32_t)K * 2u);
  for (int c = threadIdx.x; c * 8 < K; c += 256) {
    u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, (uint32_t)c * 16u, 0, 0));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t u = v[x];
      const float lo = __builtin_bit_cast(float, u << 16) * f;
      const float hi = __builtin_bit_cast(float, u & 0xFFFF0000u) * f;
      v[x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    __builtin_amdgcn_raw_buffer_store_b128(v, rH, (uint32_t)c * 16u, 0, 0);
  }
}

namespace {


int64_t f16_rows_per_launch(int64_t N, int64_t K, int64_t bm) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  int64_t r = lim / (K * 2);
  const int64_t ry = lim / (N * 4);
  r = r < ry ? r : ry;
  return (r / bm) * bm;
}

template <int GS, int YT, int MT, bool KTAIL, bool BF16X>
hipError_t f16_launch_mt(const uint16_t *X, const uint32_t *qw, const uint16_t *sc,
                         const uint8_t *zr, int64_t M, int64_t N, int64_t K, void *Y, SplitK sk,
                         const float *rowf, hipStream_t st) {
  constexpr int64_t bm = 16 * MT;
  const int ysize = YT == (int)YType::F32 ? 4 : 2;
  const int64_t rows = sk.splits > 1 ? M : f16_rows_per_launch(N, K, bm);
  if (rows <= 0 || sk.splits > kMaxSplits) return hipErrorInvalidValue;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    const dim3 grid((unsigned)(tiles * sk.splits));
    void *y = reinterpret_cast<char *>(Y) + m0 * N * ysize;
    constexpr int NW = gemm_waves(MT);
    gemm_f16_kernel<GS, YT, MT, KTAIL, BF16X, 0, NW><<<grid, 64 * NW, 0, st>>>(
        X + m0 * K, qw, sc, zr, (int)mm, (int)N, (int)K, y, sk, rowf ? rowf + m0 : nullptr,
        nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (MT < 16) {
      if (sk.splits > 1) {
        // 4 * MT reduction workgroups per output tile (four fragments each)
        const dim3 rgrid((unsigned)(tiles * MT * 4));
        const float *rf = rowf ? rowf + m0 : nullptr;
        if (sk.splits <= 2)
          splitk_reduce_kernel<YT, MT, BF16X, 2, NW><<<rgrid, 256, 0, st>>>(sk.partials, sk.splits, (int)mm, (int)N, y, rf);
        else if (sk.splits <= 4)
          splitk_reduce_kernel<YT, MT, BF16X, 4, NW><<<rgrid, 256, 0, st>>>(sk.partials, sk.splits, (int)mm, (int)N, y, rf);
        else if (sk.splits <= 8)
          splitk_reduce_kernel<YT, MT, BF16X, 8, NW><<<rgrid, 256, 0, st>>>(sk.partials, sk.splits, (int)mm, (int)N, y, rf);
        else
          splitk_reduce_kernel<YT, MT, BF16X, kMaxSplits, NW><<<rgrid, 256, 0, st>>>(sk.partials, sk.splits, (int)mm, (int)N, y, rf);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

template <int GS, int YT, bool KTAIL, bool BF16X>
hipError_t f16_go3(const uint16_t *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                   int64_t M, int64_t N, int64_t K, void *Y, int mt, SplitK sk, const float *rowf,
                   hipStream_t st) {
  if constexpr (!KTAIL) {
    if (mt == 16) {
      if (sk.splits > 1) return hipErrorInvalidValue;
      return f16_launch_mt<GS, YT, 16, KTAIL, BF16X>(X, qw, sc, zr, M, N, K, Y, sk, rowf, st);
    }
  }
  if (mt == 2) return f16_launch_mt<GS, YT, 2, KTAIL, BF16X>(X, qw, sc, zr, M, N, K, Y, sk, rowf, st);
  if (mt == 4) return f16_launch_mt<GS, YT, 4, KTAIL, BF16X>(X, qw, sc, zr, M, N, K, Y, sk, rowf, st);
  return f16_launch_mt<GS, YT, 8, KTAIL, BF16X>(X, qw, sc, zr, M, N, K, Y, sk, rowf, st);
}

template <int GS, int YT, bool KTAIL>
hipError_t f16_go2(const uint16_t *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                   int64_t M, int64_t N, int64_t K, void *Y, int mt, SplitK sk, const float *rowf,
                   hipStream_t st) {
  if (rowf) return f16_go3<GS, YT, KTAIL, true>(X, qw, sc, zr, M, N, K, Y, mt, sk, rowf, st);
  return f16_go3<GS, YT, KTAIL, false>(X, qw, sc, zr, M, N, K, Y, mt, sk, nullptr, st);
}

// K is a multiple of the group size; only g = 64 can leave half a K block.
template <int GS, int YT>
hipError_t f16_go(const uint16_t *X, const uint32_t *qw, const uint16_t *sc, const uint8_t *zr,
                  int64_t M, int64_t N, int64_t K, void *Y, int mt, SplitK sk, const float *rowf,
                  hipStream_t st) {
  if constexpr (GS < kBK) {
    if (K % kBK != 0) return f16_go2<GS, YT, true>(X, qw, sc, zr, M, N, K, Y, mt, sk, rowf, st);
  }
  return f16_go2<GS, YT, false>(X, qw, sc, zr, M, N, K, Y, mt, sk, rowf, st);
}

}  // namespace

// Row tile and K split.  M <= 32 and M <= 64 take 32- and 64-row tiles (the
// weight stream dominates there), larger M the 128-row tile, and shapes whose
// 256-row tiles fill every CU without a K split the 256-row tile (not for
// bf16 input under Scratch::Bounded, which has no room for its converted
// copy of X).  When the tiles cannot give every CU a workgroup, K is split
// (unless Scratch::None) into as many parts as still fit in one round (up to
// 8 with at least two K blocks each, up to 16 with at least four), with the
// fp32 partial tiles in the workspace.  bf16 input adds one fp32 activation
// factor per row, and with the 256-row tile its fp16 copy scaled by them.
GemmPlan gemm_f16_plan(int64_t M, int64_t N, int64_t K, bool bf16, Scratch sc) {
  GemmPlan p{};
  p.mt = M <= 32 ? 2 : M <= 64 ? 4 : 8;
  // 256-row tiles that alone fill every CU: the 256-row tile (each
  // dequantized weight then feeds 16 MFMAs instead of 8)
  if (K % kBK == 0 && ((M + 255) / 256) * ((N + kBN - 1) / kBN) >= kSlots &&
      !(bf16 && sc == Scratch::Bounded))
    p.mt = 16;
  const int64_t bm = 16 * p.mt;
  p.tiles = ((M + bm - 1) / bm) * ((N + kBN - 1) / kBN);
  const int64_t nkb = (K + kBK - 1) / kBK;
  p.splits = 1;
  if (p.tiles < kSlots && sc != Scratch::None) {
    int64_t sp = kSlots / p.tiles;
    // at least 2 K blocks per split up to 8 splits, at least 4 beyond (up to
    // 16): a split of few blocks is mostly pipeline fill and drain
    const int64_t c2 = nkb / 2 < 8 ? nkb / 2 : 8;
    const int64_t c4 = nkb / 4 < kMaxSplits ? nkb / 4 : kMaxSplits;
    const int64_t cap = c2 > c4 ? c2 : c4;
    sp = sp < cap ? sp : cap;
    p.splits = sp > 1 ? (int)sp : 1;
  }
  size_t bytes = 0;
  if (p.splits > 1) bytes = (size_t)p.tiles * p.splits * bm * kBN * 4;   // partials
  if (bf16) {
    p.rowf_offset = (bytes + 255) / 256 * 256;
    bytes = p.rowf_offset + (size_t)M * 4;
    if (p.mt == 16) {
      p.xh_offset = (bytes + 255) / 256 * 256;
      bytes = p.xh_offset + (size_t)M * (size_t)K * 2;
    }
  }
  p.workspace_bytes = bytes;
  return p;
}

hipError_t launch_gemm_f16(const uint16_t *X, bool bf16, const uint32_t *qweight,
                           const uint16_t *scales, const uint8_t *zeros, int64_t M, int64_t N,
                           int64_t K, int gs, void *Y, YType yt, const GemmPlan &p,
                           void *workspace, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (p.workspace_bytes > 0 && !workspace) return hipErrorInvalidValue;
  SplitK sk{1, nullptr};
  if (p.splits > 1) {
    sk.splits = p.splits;
    sk.partials = reinterpret_cast<float *>(workspace);
  }
  float *rowf = nullptr;
  if (bf16) {
    rowf = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.rowf_offset);
    uint16_t *xh = p.xh_offset ? reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(workspace) + p.xh_offset)
                               : nullptr;
    bf16_row_factor_kernel<<<dim3((unsigned)M), 256, 0, st>>>(X, (int)K, rowf, xh);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (xh) X = xh;
  }
  if (gs == 128) {
    if (yt == YType::F32) return f16_go<128, (int)YType::F32>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
    if (yt == YType::BF16) return f16_go<128, (int)YType::BF16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
    return f16_go<128, (int)YType::F16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
  }
  if (yt == YType::F32) return f16_go<64, (int)YType::F32>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
  if (yt == YType::BF16) return f16_go<64, (int)YType::BF16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
  return f16_go<64, (int)YType::F16>(X, qweight, scales, zeros, M, N, K, Y, p.mt, sk, rowf, st);
}

// ---- the search's loss GEMM ------------------------------------------------------
int64_t gemm_tile_count(int64_t M, int64_t N) {
  return ((M + 127) / 128) * ((N + kBN - 1) / kBN);
}

template <int GS, bool KTAIL>
static hipError_t loss_go(const uint16_t *A, const uint32_t *qw, const uint16_t *sc,
                          const uint8_t *zr, int64_t M, int64_t N, int64_t K, const float *Yref,
                          double *partials, hipStream_t st) {
  constexpr int64_t bm = 128;
  const int64_t rows = f16_rows_per_launch(N, K, bm);
  if (rows <= 0) return hipErrorInvalidValue;
  int64_t tile_base = 0;
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mm = M - m0 < rows ? M - m0 : rows;
    const int64_t tiles = ((mm + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    gemm_f16_kernel<GS, (int)YType::F32, 8, KTAIL, false, 1, 4><<<dim3((unsigned)tiles), 256, 0, st>>>(
        A + m0 * K, qw, sc, zr, (int)mm, (int)N, (int)K, nullptr, SplitK{1, nullptr},
        nullptr, Yref + m0 * N, partials + tile_base);
    tile_base += tiles;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_loss(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales,
                            const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int gs,
                            const float *Yref, double *partials, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (gs == 128) return loss_go<128, false>(A, qweight, scales, zeros, M, N, K, Yref, partials, st);
  if (K % kBK != 0) return loss_go<64, true>(A, qweight, scales, zeros, M, N, K, Yref, partials, st);
  return loss_go<64, false>(A, qweight, scales, zeros, M, N, K, Yref, partials, st);
}

}  // namespace awq
