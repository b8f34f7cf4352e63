// Counter-based dropout: Philox4x32 with 10 rounds (Salmon, Moraes, Dror and
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) and the two
// keep-mask keyings used by the attention core and the norm region.
//
// Why counter-based: under selective recomputation the backward pass re-runs
// the attention core, its softmax dropout included ("Reducing Activation
// Recomputation in Large Transformer Models", LIT-736 record, Key takeaways
// bullet 4).  A mask that is a pure function of (seed, position) is rebuilt
// bit-exactly instead of stored as an s x s tensor.
//
// Host and device inline so that the CPU build can check it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SRAT_HD __host__ __device__ __forceinline__
#else
#define SRAT_HD inline
#endif

namespace srat {

struct Philox4 {
  uint32_t w[4];
};

// a ^ b ^ k with k uniform across the wavefront: one v_bitop3_b32 (truth
// table 0x96) on gfx950 instead of two xors.
SRAT_HD uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
#if defined(__HIP_DEVICE_COMPILE__) && defined(__gfx950__)
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
#else
  return a ^ b ^ k;
#endif
}

// One call: counter (c0..c3), key (k0, k1).  Each round multiplies counter
// words 0 and 2 by the round constants (32x32 -> 64 bits), xors the high
// halves into the other two words and the key, keeps the low halves, and
// advances the key by the two Weyl increments.
SRAT_HD Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                              uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#if defined(__HIPCC__)
#pragma unroll
#endif
  for (int r = 0; r < 10; ++r) {
    const uint64_t pa = (uint64_t)c0 * kMulA;
    const uint64_t pb = (uint64_t)c2 * kMulB;
    const uint32_t n0 = xor3((uint32_t)(pb >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(pa >> 32), c3, k1);
    c1 = (uint32_t)pb;
    c3 = (uint32_t)pa;
    c0 = n0;
    c2 = n2;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Drop threshold on 16-bit draws: drop iff draw < T, T = floor(p*65536 + 1/2).
inline uint32_t drop_threshold16(float p) {
  return (uint32_t)((double)p * 65536.0 + 0.5);
}

// Keep bits of the eight elements covered by one call: bit e is set iff the
// 16-bit value e (word e/2, low half for even e) is >= thresh.
SRAT_HD uint32_t keep_bits8(const Philox4& r, uint32_t thresh) {
  uint32_t bits = 0;
#if defined(__HIPCC__)
#pragma unroll
#endif
  for (int e = 0; e < 8; ++e) {
    const uint32_t u = (r.w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    bits |= (uint32_t)(u >= thresh) << e;
  }
  return bits;
}

// Attention: elements (query i, keys 8*g .. 8*g+7) of (batch bb, global head hg).
SRAT_HD uint32_t attn_keep8(uint32_t k0, uint32_t k1, uint32_t bb, uint32_t hg, uint32_t i,
                            uint32_t g, uint32_t thresh) {
  return keep_bits8(philox4x32_10(g, i, hg, bb, k0, k1), thresh);
}

// Hidden dropout: elements (global position sg, batch bb, columns 8*g ..
// 8*g+7) of dropout site `site` (0..127); bit 31 of word 3 separates this
// stream from the attention stream.
SRAT_HD uint32_t hidden_tag(uint32_t site) { return ((site & 0x7Fu) << 24) | 0x80000000u; }
SRAT_HD uint32_t hidden_keep8(uint32_t k0, uint32_t k1, uint32_t tag, uint32_t sg, uint32_t bb,
                              uint32_t g, uint32_t thresh) {
  return keep_bits8(philox4x32_10(g, sg, bb, tag, k0, k1), thresh);
}

}  // namespace srat
