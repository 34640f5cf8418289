// Correctly rounded quotient of a 64-bit integer by a small one, for the
// activation statistic: its column sums are exact integers (numbers of 2^-24
// units), and the mean is their quotient by the row count rounded once to
// fp64.  Plain C++ (host and device); the host build is checked against exact
// rational division by tests/test_kernel_identities.py.
#pragma once

#include <stdint.h>

#ifndef AWQ_HOST_DEVICE
#define AWQ_HOST_DEVICE __host__ __device__
#endif

namespace awq {

// RN(S / M) in fp64, round half to even, for 0 < M < 2^24.
AWQ_HOST_DEVICE inline double rn_quotient_u64(uint64_t S, uint32_t M) {
  // Below 2^53 both operands are exact fp64 values: one IEEE division.
  if (S < ((uint64_t)1 << 53)) return (double)S / (double)M;
  // Otherwise S / M >= 2^29.  T = floor(S * 2^24 / M) holds its integer part
  // and 24 fraction bits (at least 54 significant bits in all), `sticky`
  // whether anything is left below them.
  const uint64_t I = S / M, R = S % M;              // R < 2^24
  const uint64_t FR = R << 24;                       // < 2^48
  const uint64_t F = FR / M;
  const bool sticky = (FR % M) != 0;
  const unsigned __int128 T = ((unsigned __int128)I << 24) | F;
  const uint64_t hi = (uint64_t)(T >> 64), lo = (uint64_t)T;
  const int bits = hi ? 128 - __builtin_clzll(hi) : 64 - __builtin_clzll(lo);
  const int sh = bits - 53;                          // >= 1
  uint64_t keep = (uint64_t)(T >> sh);
  const unsigned __int128 rem = T & ((((unsigned __int128)1) << sh) - 1);
  const unsigned __int128 half = ((unsigned __int128)1) << (sh - 1);
  if (rem > half || (rem == half && (sticky || (keep & 1)))) ++keep;   // 2^53 is still exact
  return __builtin_ldexp((double)keep, sh - 24);
}

}  // namespace awq
