// Scale + group-quantize + pack for gfx950.
//
// Follows the pages' quantizer config ("AWQ Advanced Usage Guide", "Group Size
// Configuration" and "Zero-Point Quantization": w_bit = 4, q_group_size, an
// asymmetric grid with a zero point) and the sW side of Y = (X/s)(sW)
// (ai.lansai.wang explainer, section "AWQ 的四步链路").  Per group of g
// consecutive input channels of one output row:
//   v = fp32(s_k * W_nk); lo = min(min v, 0); hi = max(max v, 0)
//   scale = fp16(max((hi - lo) / 15, 2^-14)); zero = clamp(rint(-lo/scale), 0, 15)
//   code  = clamp(rint(v / scale) + zero, 0, 15)
// with IEEE correctly rounded fp32 division and rint half-to-even, so the codes
// are reproducible bit for bit on any IEEE machine.  Without a zero point
// ("Zero-Point Quantization": zero_point = False, the symmetric variant):
//   scale = fp16(max(max |v| / 7, 2^-14)); code = clamp(rint(v/scale), -8, 7) + 8
// and no zero point is stored.
//
// Mapping: one lane per output word (8 input channels, 16 bytes of W);
// g/8 consecutive lanes form a group and exchange min/max with DPP moves.
// The kernel moves 2 bytes in and 0.5 + 3/g bytes out per weight and is
// close to bound by its VALU work: the per-weight division is replaced by a
// reciprocal multiply whose rounding provably agrees except next to
// half-integers (checked per lane), and that same check catches non-finite
// values, so the common path carries no separate test for them.

#include <type_traits>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

// Largest value over the g/8 lanes of a group (aligned runs of 8 or 16 lanes)
// with DPP lane exchanges: swap neighbours, swap pairs, mirror within 8, then
// (g = 128) mirror within 16.  Each step pairs every lane with one of the other
// half of its current run, so after log2(g/8) steps every lane of a group
// holds the group's maximum.  Applied to the bit patterns of floats of one
// sign it is an exact float reduction: non-negative floats order like their
// patterns, and non-positive ones in reverse (so the largest pattern is the
// minimum).  Integer maxima need no NaN quieting before each exchange, which
// a float min or max does (two more instructions per step).
template <int LANES>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  auto step = [](uint32_t x, auto ctrl_tag) {
    constexpr int kCtrl = decltype(ctrl_tag)::value;
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, true);
    return x > y ? x : y;
  };
  v = step(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  v = step(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  v = step(v, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (LANES == 16) v = step(v, std::integral_constant<int, 0x140>{});   // row_mirror
  return v;
}
// Minimum of non-positive floats and maximum of non-negative floats over the
// group (lo <= 0 <= hi by construction).
template <int LANES>
__device__ __forceinline__ float group_min_nonpos(float v) {
  return __builtin_bit_cast(float, group_umax<LANES>(__builtin_bit_cast(uint32_t, v)));
}
template <int LANES>
__device__ __forceinline__ float group_max_nonneg(float v) {
  return __builtin_bit_cast(float, group_umax<LANES>(__builtin_bit_cast(uint32_t, v)));
}

// Grid: x covers the words of one row in chunks of 256 (a multiple of the
// group's word count, so no group straddles workgroups), y the rows (looped
// when N exceeds the grid's y limit).  No per-lane 64-bit division.
template <int GS, bool SYM>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const uint16_t *__restrict__ W, int64_t N, int64_t K, const float *__restrict__ s,
    uint32_t *__restrict__ qweight, uint16_t *__restrict__ scales,
    uint8_t *__restrict__ zeros, int32_t *__restrict__ nonfinite) {
  constexpr int kLanesPerGroup = GS / 8;
  const int wpr = (int)(K / 8);                       // words per row
  const int c = blockIdx.x * 256 + threadIdx.x;       // word within the row
  // words_per_row is a multiple of kLanesPerGroup and groups start at
  // multiples of it, so a group is either entirely active or entirely idle.
  const bool active = c < wpr;
  float sv[8];
  if (s != nullptr && active) {
    const float4 s0 = *reinterpret_cast<const float4 *>(s + (int64_t)c * 8);
    const float4 s1 = *reinterpret_cast<const float4 *>(s + (int64_t)c * 8 + 4);
    sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
    sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
  }
  int bad = 0;
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    float v[8];
    if (active) {
      const u32x4 raw = *reinterpret_cast<const u32x4 *>(W + n * K + (int64_t)c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t r = raw[i];
        v[2 * i] = half_bits_to_float((uint16_t)(r & 0xFFFFu));
        v[2 * i + 1] = half_bits_to_float((uint16_t)(r >> 16));
      }
      if (s != nullptr) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = sv[i] * v[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }

    float lo = 0.0f, hi = 0.0f, step;
    if constexpr (SYM) {
      // the largest magnitude of the group on level +-7: one IEEE division
      // per lane and group
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
      amax = group_max_nonneg<kLanesPerGroup>(amax);
      step = amax / 7.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo = fminf(lo, v[i]);
        hi = fmaxf(hi, v[i]);
      }
      lo = group_min_nonpos<kLanesPerGroup>(lo);
      hi = group_max_nonneg<kLanesPerGroup>(hi);

      // (hi - lo) / 15, correctly rounded, from the product with RN(1/15)
      // and one exact-remainder correction (Markstein): checked against IEEE
      // division for every non-negative finite fp32 dividend; an infinite
      // dividend (the only other value hi - lo takes) passes through as the
      // division would give it.
      const float d = hi - lo;
      const float q0 = d * 0x1.111112p-4f;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-15.0f, q0, d), 0x1.111112p-4f, q0);
      step = d == __builtin_inff() ? d : q1;
    }
    const _Float16 sh = (_Float16)fmaxf(step, 0x1p-14f);
    const float sf = (float)sh;

    // rint(v / sf) with the correctly rounded quotient q, without eight
    // divisions: |v / sf| < 16 (|v| <= hi - lo <= 15 sf (1 + 2^-10), or
    // symmetric |v| <= max |v| <= 7 sf (1 + 2^-10)), so q
    // lies within 2^-20 of the exact v / sf, and y = fl(v * rcp(sf)), with
    // the hardware reciprocal (specified to 1 ulp; up to 7 ulp would do),
    // within 2^-16 - 2^-20.  Unless y is within 2^-16 of a half-integer, both
    // round to the same integer (ties included: a q exactly at k + 1/2 puts
    // y that close to it); the rare lanes that are that close divide.  The
    // zero point's -lo / sf (also below 16) takes the same path.  The test is
    // written so that a NaN y also fails it: every non-finite v makes its own
    // lane's y NaN (v * rcp(sf) is NaN or +-inf, and inf - rint(inf) is NaN;
    // an inf in the group makes sf inf and rcp(sf) 0), so those lanes take
    // the slow path too, where they are counted.
    const float rs = __builtin_amdgcn_rcpf(sf);
    const float zy = -lo * rs;          // symmetric: lo = 0, so zq = 0
    float zq = __builtin_rintf(zy);
    bool near_half = !(__builtin_fabsf(zy - zq) <= 0.5f - 0x1p-16f);
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = v[i] * rs;
      qv[i] = __builtin_rintf(y);
      // y - rint(y) is exact
      near_half |= !(__builtin_fabsf(y - qv[i]) <= 0.5f - 0x1p-16f);
    }
    if (near_half) {
      if constexpr (!SYM) zq = __builtin_rintf(-lo / sf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qv[i] = __builtin_rintf(v[i] / sf);
        bad += !__builtin_isfinite(v[i]);
      }
    }
    // asymmetric: codes rint(v/s) + z clamped to [0, 15]; symmetric:
    // rint(v/s) clamped to [-8, 7], plus 8
    const float zf = SYM ? 8.0f : fminf(fmaxf(zq, 0.0f), 15.0f);
    const float qlo = SYM ? -8.0f : 0.0f, qhi = SYM ? 7.0f : 15.0f;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float qf = SYM ? fminf(fmaxf(qv[i], qlo), qhi) + zf
                           : fminf(fmaxf(qv[i] + zf, qlo), qhi);
      word |= ((uint32_t)qf) << (4 * nibble_of_channel(i));
    }

    if (active) {
      qweight[n * wpr + c] = word;
      if ((c % kLanesPerGroup) == 0) {
        const int64_t gi = n * (K / GS) + c / kLanesPerGroup;
        scales[gi] = __builtin_bit_cast(uint16_t, sh);
        if constexpr (!SYM) zeros[gi] = (uint8_t)zf;
      }
    }
  }

  if (nonfinite != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off, 64);
    if ((threadIdx.x & 63) == 0 && bad) atomicAdd(nonfinite, bad);
  }
}

hipError_t launch_quantize_pack(const uint16_t *W, int64_t N, int64_t K, int gs,
                                const float *s, uint32_t *qweight, uint16_t *scales,
                                uint8_t *zeros, int32_t *nonfinite, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const int64_t wpr = K / 8;
  // At most 2048 rows of workgroups; each walks every 2048th row.  One
  // workgroup per row (22016 of them, 1 KiB of W per wave, for an 11008-row
  // layer) measured 4-12% slower on the 7B-class layers (28.0 -> 24.6 us on
  // 11008 x 4096, 29.4 -> 26.5 on 4096 x 11008, 12.0 -> 11.5 on 4096^2;
  // 1024 rows was within 1%, 512 and fewer slower), bit-identical.
  const dim3 grid((unsigned)((wpr + 255) / 256), (unsigned)(N < 2048 ? N : 2048));
  if (zeros == nullptr) {
    if (gs == 128)
      quantize_pack_kernel<128, true><<<grid, 256, 0, st>>>(W, N, K, s, qweight, scales, zeros, nonfinite);
    else
      quantize_pack_kernel<64, true><<<grid, 256, 0, st>>>(W, N, K, s, qweight, scales, zeros, nonfinite);
  } else {
    if (gs == 128)
      quantize_pack_kernel<128, false><<<grid, 256, 0, st>>>(W, N, K, s, qweight, scales, zeros, nonfinite);
    else
      quantize_pack_kernel<64, false><<<grid, 256, 0, st>>>(W, N, K, s, qweight, scales, zeros, nonfinite);
  }
  return hipGetLastError();
}

}  // namespace awq

namespace awq {

// ---- dequantize: packed codes back to weights --------------------------------------
// The pseudo-quantization step of the pages' pipeline (ai.lansai.wang explainer,
// four-stage table, "伪量化评测" row: simulate the low-bit weights without the
// target kernel): W'[n][k] = (q - z) * s, the value the linear kernels multiply
// by, written as fp32 (exact) or fp16 (rounded once).  One lane per packed word
// (8 weights): 4 bytes of codes in, 16 or 32 bytes out; a 2-D grid as above.
template <int GS, bool F32OUT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t *__restrict__ qweight,
                                                         const uint16_t *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros,
                                                         int64_t N, int64_t K, void *__restrict__ out) {
  const int wpr = (int)(K / 8);
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= wpr) return;
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    const uint32_t w = qweight[n * wpr + c];
    const int64_t gi = n * (K / GS) + (c * 8) / GS;
    const float s = half_bits_to_float(scales[gi]);
    const float z = zeros ? (float)zeros[gi] : 8.0f;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ((float)((w >> (4 * nibble_of_channel(i))) & 0xFu) - z) * s;
    if constexpr (F32OUT) {
      float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + n * K + (int64_t)c * 8);
      o[0] = float4{v[0], v[1], v[2], v[3]};
      o[1] = float4{v[4], v[5], v[6], v[7]};
    } else {
      u32x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[i] = (uint32_t)float_to_half_bits(v[2 * i]) | ((uint32_t)float_to_half_bits(v[2 * i + 1]) << 16);
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + n * K + (int64_t)c * 8) = h;
    }
  }
}

hipError_t launch_dequantize(const uint32_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, int gs, void *out, bool f32, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const int64_t wpr = K / 8;
  const dim3 grid((unsigned)((wpr + 255) / 256), (unsigned)(N < 65535 ? N : 65535));
  if (gs == 128) {
    if (f32) dequantize_kernel<128, true><<<grid, 256, 0, st>>>(qweight, scales, zeros, N, K, out);
    else dequantize_kernel<128, false><<<grid, 256, 0, st>>>(qweight, scales, zeros, N, K, out);
  } else {
    if (f32) dequantize_kernel<64, true><<<grid, 256, 0, st>>>(qweight, scales, zeros, N, K, out);
    else dequantize_kernel<64, false><<<grid, 256, 0, st>>>(qweight, scales, zeros, N, K, out);
  }
  return hipGetLastError();
}

}  // namespace awq
