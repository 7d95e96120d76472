// Runs PyTorch's header-only Philox4x32-10 engine (ATen/core/PhiloxRNGEngine.h)
// as an implementation independent of the oracle's.  Reads lines
// "seed subsequence offset" and prints the four 32-bit words of that block.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cinttypes>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine eng(seed, sub, off);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
