// Host-only driver for PyTorch's at::philox_engine (ATen/core/PhiloxRNGEngine.h),
// an independent Philox4x32-10 implementation used to pin the oracle's generator.
// Reads lines "seed subsequence offset" (decimal) and prints the four 32-bit words
// of the block at that position, in hex.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cinttypes>
#include <cstdio>

int main() {
  unsigned long long seed, subseq, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
    at::philox_engine eng(seed, subseq, offset);
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) w[i] = eng();
    std::printf("%08" PRIx32 " %08" PRIx32 " %08" PRIx32 " %08" PRIx32 "\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
