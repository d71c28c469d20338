// Independent Philox4x32-10 for pinning the oracle: PyTorch's header-only philox_engine.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal) and prints the four output words of that counter/key.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    const uint64_t subsequence = (uint64_t)c2 | ((uint64_t)c3 << 32);
    const uint64_t offset = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::Philox4_32 eng(seed, subsequence, offset);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
