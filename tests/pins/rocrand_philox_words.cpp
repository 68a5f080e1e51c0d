// Host-side reference words from rocRAND's philox4x32_10 engine (open-source
// header, compiled here for the CPU).  Used only to pin the oracle's Philox.
//
// Reads lines "seed plan_id round counter" from stdin and prints the four
// 32-bit output words of Philox-4x32-10 at counter (counter, round, plan_id, 0)
// under key (seed low, seed high).  rocRAND's engine places `subsequence` in
// counter words 2..3 and offset/4 in words 0..1, so the engine is seeded with
// subsequence = plan_id and offset = 4 * (round * 2^32 + counter).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, plan, rnd, ctr;
  while (std::scanf("%llu %llu %llu %llu", &seed, &plan, &rnd, &ctr) == 4) {
    unsigned long long offset = 4ull * ((rnd << 32) + ctr);
    rocrand_device::philox4x32_10_engine eng(seed, plan, offset);
    unsigned w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
