// Test-only cross-check of the oracle's Philox4x32-10: prints, for each input
// line "c0 c1 c2 c3 k0 k1" (decimal 32-bit words), the four output words of
// PyTorch's open-source at::philox_engine for that counter and key.
// at::philox_engine(seed, subsequence, offset) keys on seed, puts
// subsequence in counter words 2..3 and offset in words 0..1; successive
// calls return words 0..3 of that block.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (k1 << 32) | k0;
    uint64_t subseq = (c3 << 32) | c2;
    uint64_t offset = (c1 << 32) | c0;
    at::philox_engine eng(seed, subseq, 0);
    eng.incr_n(offset);
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) w[i] = eng();
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
