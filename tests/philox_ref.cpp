// Independent Philox4x32-10 reference for the oracle's pin test: it runs
// PyTorch's open-source engine (ATen/core/PhiloxRNGEngine.h) and prints its raw
// words.  Input lines: "seed subsequence offset"; output: four words per line.
// The engine keys Philox with the 64-bit seed and starts from the counter
// (offset low, offset high, subsequence low, subsequence high).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cinttypes>
#include <cstdio>

int main() {
  unsigned long long seed, subseq, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
    at::philox_engine eng(seed, subseq, offset);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
