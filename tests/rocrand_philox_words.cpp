// Philox4x32-10 words from rocRAND's implementation (its state engine,
// compiled for the host), as an independent reference for the oracle's
// generator. rocrand_init(seed, subsequence, offset) places the counter at
// (offset / 4, subsequence) with key = seed, and rocrand() returns word
// offset % 4 of that block.
//
// stdin: lines "seed subsequence index" (decimal); stdout: one word per line.
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed, subseq, index;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &index) == 3) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, subseq, index, &st);
    std::printf("%u\n", rocrand(&st));
  }
  return 0;
}
