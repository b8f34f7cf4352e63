// Independent Philox4x32-10 reference for the oracle's pins: calls rocRAND's
// header-only host/device engine (a library routine; nothing here is part of
// the library under test).  Reads lines "seed c0 c1 c2 c3" (decimal) on stdin
// and prints the four 32-bit output words of Philox4x32-10 for counter
// (c0, c1, c2, c3) and key (seed mod 2^32, seed div 2^32) as hex.
//
// rocrand_init(seed, subsequence, offset) keys the engine with the 64-bit
// seed, puts the subsequence into counter words 2..3 and advances words 0..1
// by offset/4 blocks.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, c2 | (c3 << 32), 0ull, &st);
    // word 1 += c1 in four pieces so that no single offset overflows 64 bits
    for (int k = 0; k < 4; ++k) skipahead((c1 / 4) << 34, &st);
    skipahead((c1 % 4) << 34, &st);
    skipahead(c0 * 4, &st);
    uint4 v = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
