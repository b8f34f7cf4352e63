// Host build of the library's own philox.hpp (the code the kernels use), for
// a bit-exact check against the oracle.  Reads "seed c0 c1 c2 c3 thresh" lines,
// prints the four words and the eight keep bits, then the four words of each
// hoisted form the kernels call (fixed c1..c3; fixed c0, c2, c3).
#include <cstdio>
#include "philox.hpp"

int main() {
  unsigned long long seed, c0, c1, c2, c3, t;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3, &t) == 6) {
    const srat::Philox4 r = srat::philox4x32_10((uint32_t)c0, (uint32_t)c1, (uint32_t)c2, (uint32_t)c3,
                                                (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32));
    // the kernels' form with the c0-independent parts of rounds 1-2 hoisted
    const srat::PhiloxRow f = srat::philox_row((uint32_t)c1, (uint32_t)c2, (uint32_t)c3,
                                               (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32));
    const srat::Philox4 q = srat::philox4x32_10_row((uint32_t)c0, f);
    const srat::PhiloxCol fc = srat::philox_col((uint32_t)c0, (uint32_t)c2, (uint32_t)c3,
                                                (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32));
    const srat::Philox4 u = srat::philox4x32_10_col((uint32_t)c1, fc);
    std::printf("%08x %08x %08x %08x %02x %08x %08x %08x %08x %08x %08x %08x %08x\n", r.w[0], r.w[1], r.w[2],
                r.w[3], srat::keep_bits8(r, (uint32_t)t), q.w[0], q.w[1], q.w[2], q.w[3], u.w[0], u.w[1], u.w[2],
                u.w[3]);
  }
  return 0;
}
