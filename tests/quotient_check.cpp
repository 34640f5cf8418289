// Host build of the activation statistic's rounding (exact_quotient.h): reads
// "S M" pairs from stdin and prints the fp64 bits of RN(S / M) in hex.
// Built and run by tests/test_kernel_identities.py.
#include <cinttypes>
#include <cstdio>
#include <cstring>
#define AWQ_HOST_DEVICE
#include "exact_quotient.h"
int main() {
  unsigned long long S;
  unsigned M;
  while (std::scanf("%llu %u", &S, &M) == 2) {
    const double q = awq::rn_quotient_u64(S, M);
    uint64_t b;
    std::memcpy(&b, &q, 8);
    std::printf("%016" PRIx64 "\n", b);
  }
  return 0;
}
