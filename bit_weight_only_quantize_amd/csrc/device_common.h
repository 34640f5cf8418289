// Device helpers shared by the gfx950 kernels: vector types, the 16x16x32 MFMA
// wrappers and the exact integer dequantization of one packed word.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct TagF16 {};
struct TagBF16 {};

// D = A * B + C for a 16x16 fp32 tile and K = 32.  Lane l supplies row
// (l & 15) of A and column (l & 15) of B, each as 8 consecutive elements of
// its K-slot (l >> 4); it receives D rows 4*(l >> 4) .. +3 of column (l & 15).
template <class T>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mfma32<TagF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma32<TagBF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Packed nibble order: nibble p of a word holds input channel ORDER[p] of its
// 8, ORDER = {0,2,4,6,1,3,5,7}; channel i therefore sits at nibble
// (i >> 1) + 4 * (i & 1).  Masking 0x000F000F after a shift of 4*j leaves the
// pair (2j, 2j+1) in the two 16-bit halves.
__device__ __forceinline__ int nibble_of_channel(int i) { return (i >> 1) + 4 * (i & 1); }

// fp16: the exact integers (q - z) for the 8 channels of word w, as 8 fp16 in
// channel order.  OR-ing a code into the mantissa of 1024.0 (0x6400) gives
// 1024 + q exactly; subtracting (1024 + z) leaves q - z exactly.  Codes that
// sit 4 bits higher give 1024 + 16q, and (1024 + 16q) / 16 - (64 + z) is
// q - z exactly as well, which saves two shifts per word.
struct DeqF16 {
  f16x2 nz1024;  // -(1024 + z) in both halves
  f16x2 nz64;    // -(64 + z) in both halves
  __device__ __forceinline__ explicit DeqF16(uint32_t z) {
    const _Float16 a = (_Float16)(-(float)(1024 + z));
    const _Float16 b = (_Float16)(-(float)(64 + z));
    nz1024 = f16x2{a, a};
    nz64 = f16x2{b, b};
  }
  __device__ __forceinline__ u32x4 operator()(uint32_t w) const {
    const uint32_t kMagic = 0x64006400u;
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    const f16x2 p0 = __builtin_bit_cast(f16x2, (w & 0x000F000Fu) | kMagic);
    const f16x2 p1 = __builtin_bit_cast(f16x2, (w & 0x00F000F0u) | kMagic);
    const f16x2 p2 = __builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) | kMagic);
    const f16x2 p3 = __builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) | kMagic);
    const f16x2 h0 = p0 + nz1024;
    const f16x2 h1 = __builtin_elementwise_fma(p1, sixteenth, nz64);
    const f16x2 h2 = p2 + nz1024;
    const f16x2 h3 = __builtin_elementwise_fma(p3, sixteenth, nz64);
    return u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                 __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
  }
};

// bf16: 128 + q exactly (OR into the mantissa of 128.0 = 0x4300).  gfx950 has
// no packed bf16 add, so the zero point is removed after the product:
// sum_k a_k (q_k - z) = sum_k a_k (128 + q_k) - (128 + z) sum_k a_k.
struct DeqBF16 {
  __device__ __forceinline__ u32x4 operator()(uint32_t w) const {
    const uint32_t kMagic = 0x43004300u;
    return u32x4{(w & 0x000F000Fu) | kMagic, ((w >> 4) & 0x000F000Fu) | kMagic,
                 ((w >> 8) & 0x000F000Fu) | kMagic, ((w >> 12) & 0x000F000Fu) | kMagic};
  }
};

// bf16 1.0 in all 8 slots: an MFMA against it yields the row sums of A.
__device__ __forceinline__ u32x4 bf16_ones() {
  return u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the MI355X.  Map
// the hardware block id so that each XCD receives a contiguous run of logical
// tiles (which then share operands in that XCD's L2).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  constexpr int64_t kXcd = 8;
  const int64_t per = nblocks / kXcd;
  if (bid >= per * kXcd) return bid;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace awq
