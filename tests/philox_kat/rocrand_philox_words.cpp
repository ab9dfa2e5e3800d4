// Known-answer source for the oracle's Philox4x32-10: rocRAND's header-only engine, run on the
// host CPU. Reads "seed counter" pairs (decimal, 64-bit) from stdin and prints the four 32-bit
// output words of Philox4x32-10 at key (seed lo, seed hi) and counter (counter lo, counter hi,
// 0, 0). Test infrastructure; not part of the library.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, counter;
  while (std::scanf("%llu %llu", &seed, &counter) == 2) {
    // subsequence 0, offset 4 * counter: the engine's counter becomes (counter, 0, 0) words
    rocrand_device::philox4x32_10_engine eng(seed, 0ull, 4ull * counter);
    unsigned int w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
