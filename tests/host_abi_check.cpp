// Host-only driver of the C ABI for sanitizer builds: every entry point with
// arguments its validation rejects (so no HIP call is made), and the
// workspace-size functions over a sweep of shapes (their plan arithmetic).
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
// by tests/test_host_sanitizers.py; prints "host ABI check ok" at the end.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "awq355.h"

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main() {
  void *F = reinterpret_cast<void *>(0x10000);   // aligned, never dereferenced
  const awq_config c128{4, 128, 1}, c64{4, 64, 1}, sym{4, 128, 0}, bad{4, 96, 1};
  const uint32_t *qw = static_cast<const uint32_t *>(F);
  const uint16_t *sc = static_cast<const uint16_t *>(F);
  const uint8_t *zr = static_cast<const uint8_t *>(F);

  EXPECT(awq_quantize_pack(F, 4, 200, c128, nullptr, (uint32_t *)F, (uint16_t *)F, (uint8_t *)F,
                           nullptr, nullptr) == AWQ_ERR_INVALID_ARG);
  EXPECT(awq_quantize_pack(F, 4, 256, bad, nullptr, (uint32_t *)F, (uint16_t *)F, (uint8_t *)F,
                           nullptr, nullptr) == AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_quantize_pack(F, 0, 256, sym, nullptr, (uint32_t *)F, (uint16_t *)F, nullptr,
                           nullptr, nullptr) == AWQ_OK);
  EXPECT(awq_dequantize(qw, sc, zr, 4, 256, c128, F, 1, nullptr) == AWQ_ERR_INVALID_ARG);
  EXPECT(awq_linear(F, 2, qw, sc, zr, 3, 64, 256, c128, F, 0, nullptr) == AWQ_ERR_INVALID_ARG);
  EXPECT(awq_linear(F, 1, qw, sc, zr, 64, 13824, 5120, c128, F, 2, nullptr) == AWQ_ERR_WORKSPACE);
  EXPECT(awq_linear_ex(F, 0, qw, sc, zr, 17, 64, 256, c128, F, 0, AWQ_KERNEL_GEMV, nullptr, 0,
                       nullptr) == AWQ_ERR_INVALID_ARG);
  EXPECT(awq_linear_ws(F, 0, qw, sc, zr, 64, 13824, 5120, c128, F, 0, F, 1, nullptr) ==
         AWQ_ERR_WORKSPACE);
  EXPECT(awq_linear_noalloc(F, 1, qw, sc, zr, 9000000, 4096, 4096, c128, F, 2, nullptr) ==
         AWQ_ERR_WORKSPACE);
  awq_linear_part parts[5];
  for (auto &p : parts) p = awq_linear_part{qw, sc, zr, 64, F};
  EXPECT(awq_linear_fused(F, 0, parts, 5, 3, 256, c128, 0, nullptr, 0, 0, nullptr, 0, nullptr) ==
         AWQ_ERR_INVALID_ARG);
  EXPECT(awq_linear_fused(F, 0, parts, 3, 3, 256, c128, AWQ_EPILOGUE_SILU_MUL, F, 0, 0, nullptr,
                          0, nullptr) == AWQ_ERR_INVALID_ARG);
  int32_t best = -1;
  EXPECT(awq_scale_search(F, F, 0, 64, 256, c128, nullptr, 20, F, 1 << 30, &best, nullptr,
                          (float *)F, (uint32_t *)F, (uint16_t *)F, (uint8_t *)F, nullptr) ==
         AWQ_ERR_INVALID_ARG);
  const awq_search_options bad_opts{0, 2};
  EXPECT(awq_scale_search_ex(F, F, 64, 64, 256, c128, nullptr, 20, &bad_opts, F, 1 << 30, &best,
                             nullptr, (float *)F, (uint32_t *)F, (uint16_t *)F, (uint8_t *)F,
                             nullptr, nullptr) == AWQ_ERR_INVALID_ARG);
  EXPECT(best == -1);

  // size functions over a sweep of shapes (plan, split and layout arithmetic)
  const int64_t Ms[] = {0, 1, 3, 16, 17, 33, 64, 65, 200, 256, 1000, 4096, 65536};
  const int64_t Ns[] = {1, 77, 256, 4096, 5120, 11008, 13824, 28672, 131072};
  const int64_t Ks[] = {128, 320, 1024, 4096, 5120, 11008, 13824, 28672};
  size_t total = 0;
  for (int64_t M : Ms)
    for (int64_t N : Ns)
      for (int64_t K : Ks)
        for (const awq_config &c : {c128, c64, sym})
          for (int xd = 0; xd < 2; ++xd)
            for (int kern = 0; kern < 3; ++kern) {
              if (K % c.group_size) continue;
              total += awq_linear_workspace_size(M, N, K, c, xd, kern);
              awq_linear_part pp[2] = {{nullptr, nullptr, nullptr, N, nullptr},
                                       {nullptr, nullptr, nullptr, N, nullptr}};
              total += awq_linear_fused_workspace_size(pp, 2, M, K, c, xd, 1, kern);
              total += awq_linear_fused_workspace_size(pp, 1, M, K, c, xd, 0, kern);
            }
  for (int64_t M : {1, 100, 4096, 34278})
    for (int64_t N : {1, 77, 4096})
      for (int64_t K : {128, 384, 4096})
        for (int duo = 0; duo < 2; ++duo)
          for (int clip = 0; clip < 2; ++clip) {
            const awq_search_options o{duo, clip};
            total += awq_scale_search_workspace_size_ex(M, N, K, c128, 20, &o);
          }
  for (int s = 0; s < 7; ++s) total += awq_status_string((awq_status)s)[0];
  std::printf("sizes checksum %zu\n", total);
  if (failures) return 1;
  std::printf("host ABI check ok\n");
  return 0;
}
