// Prints Philox4x32-10 blocks from PyTorch's header-only at::Philox4_32 engine (a library routine
// used to cross-check the oracle's own Philox).  Reads lines "seed subsequence offset" on stdin and
// prints the four 32-bit words of the block at counter (offset, subsequence) for key = seed.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cinttypes>
#include <cstdio>

int main() {
  unsigned long long seed, subseq, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
    at::Philox4_32 eng(seed, subseq, offset);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
