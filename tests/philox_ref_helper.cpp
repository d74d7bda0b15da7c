// Host-only known-answer helper: prints Philox4x32-10 words from an independent
// library so the oracle's generator can be checked against it.
// Build with -DUSE_TORCH (torch's ATen PhiloxRNGEngine.h, g++) or -DUSE_ROCRAND
// (rocRAND's philox4x32_10 engine, hipcc host compile).
// stdin: lines "seed subsequence counter_lo64 word"; stdout: one hex word per line.
#include <cstdint>
#include <cstdio>
#if defined(USE_TORCH)
#include <ATen/core/PhiloxRNGEngine.h>
#elif defined(USE_ROCRAND)
#include <rocrand/rocrand_philox4x32_10.h>
#endif

int main() {
  unsigned long long seed, sub, ctr, word;
  while (std::scanf("%llu %llu %llu %llu", &seed, &sub, &ctr, &word) == 4) {
    uint32_t w = 0;
#if defined(USE_TORCH)
    at::philox_engine e(seed, sub, ctr);
    for (unsigned long long i = 0; i <= word; ++i) w = e();
#elif defined(USE_ROCRAND)
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ULL * ctr + word);
    w = e.next();
#endif
    std::printf("%08x\n", w);
  }
  return 0;
}
