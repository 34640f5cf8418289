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

// Bit-pattern constants of the dequantization, held in registers.  gfx9-family
// VOP3 encodings take no literal operand, so with literal masks every
// (w & mask) | exponent would split into a v_and and a v_or; with the masks in
// VGPRs and the exponent patterns in SGPRs it is one v_and_or_b32.  Build one
// DeqRegs per kernel, outside the loops (the empty asm statements only hide
// the constant values from the optimizer so that they stay in registers).
struct DeqRegs {
  uint32_t lo, hi;      // 0x000F000F, 0x00F000F0
  uint32_t e1024, e64;  // fp16 1024.0 and fp16 64.0 in both halves
  __device__ __forceinline__ DeqRegs()
      : lo(0x000F000Fu), hi(0x00F000F0u), e1024(0x64006400u), e64(0x54005400u) {
    asm volatile("" : "+v"(lo));
    asm volatile("" : "+v"(hi));
    asm volatile("" : "+s"(e1024));
    asm volatile("" : "+s"(e64));
  }
};

// fp16: the exact integers (q - z) for the 8 channels of word w, as 8 fp16 in
// channel order.  OR-ing a code held in bits 0..3 of a half into the mantissa
// of 1024.0 (0x6400) gives 1024 + q exactly, a code held in bits 4..7 OR-ed
// into 64.0 (0x5400) gives 64 + q exactly (channel pairs (0,1) and (4,5) come
// out as 1024 + q, pairs (2,3) and (6,7) as 64 + q); a packed half
// subtraction of 1024 + z or 64 + z then leaves q - z, exactly, since every
// value involved is an integer of at most 11 bits.  Nine VALU instructions
// per 8 weights (a shift, four and-or, four packed subtractions).
struct DeqF16 {
  uint32_t nz1024, nz64;  // -(1024 + z), -(64 + z) in both halves (fp16 bits)
  __device__ __forceinline__ explicit DeqF16(uint32_t z) {
    const uint32_t a = 0xE400u | z;
    const uint32_t b = 0xD400u + (z << 4);
    nz1024 = a | (a << 16);
    nz64 = b | (b << 16);
  }
  __device__ __forceinline__ u32x4 operator()(uint32_t w, const DeqRegs &r) const {
    // (scalar copies first: bit-casting an element of a vector lvalue reads
    // the vector's first element with this compiler)
    const uint32_t w8 = w >> 8;
    const uint32_t p0 = (w & r.lo) | r.e1024, p1 = (w & r.hi) | r.e64;
    const uint32_t p2 = (w8 & r.lo) | r.e1024, p3 = (w8 & r.hi) | r.e64;
    const f16x2 h0 = __builtin_bit_cast(f16x2, p0) + __builtin_bit_cast(f16x2, nz1024);
    const f16x2 h1 = __builtin_bit_cast(f16x2, p1) + __builtin_bit_cast(f16x2, nz64);
    const f16x2 h2 = __builtin_bit_cast(f16x2, p2) + __builtin_bit_cast(f16x2, nz1024);
    const f16x2 h3 = __builtin_bit_cast(f16x2, p3) + __builtin_bit_cast(f16x2, nz64);
    return u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                 __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
  }
};

// bf16: the exact integers (q - z) as 8 bf16 in channel order, from the fp16
// ones.  gfx950 has no packed bf16 arithmetic; widening each fp16 half to
// fp32 is exact, and an integer of at most 4 significant bits has zero low
// 16 bits in fp32, so the upper half of its fp32 pattern is its bf16
// encoding.  Three VALU operations per pair (two conversions and one byte
// permute) on top of DeqF16.
__device__ __forceinline__ u32x4 f16_pairs_to_bf16(u32x4 h) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hi = h[i];
    const f16x2 p = __builtin_bit_cast(f16x2, hi);
    const uint32_t lo32 = __builtin_bit_cast(uint32_t, (float)p[0]);
    const uint32_t hi32 = __builtin_bit_cast(uint32_t, (float)p[1]);
    // bytes 2,3 of lo32 -> bytes 0,1; bytes 2,3 of hi32 -> bytes 2,3
    out[i] = __builtin_amdgcn_perm(hi32, lo32, 0x07060302u);
  }
  return out;
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
