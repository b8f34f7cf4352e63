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

// a ^ b ^ k: one v_bitop3_b32 (truth table 0x96) on gfx950 instead of two xors.
SRAT_HD uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
#if defined(__HIP_DEVICE_COMPILE__) && defined(__gfx950__)
  return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
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

// The same generator for a fixed (c1, c2, c3) and key, with counter word c0
// varying: the parts of rounds 1 and 2 that do not involve c0 are computed
// once (PhiloxRow), so each call costs two multiplies and one xor fewer.
// Bit-identical to philox4x32_10(c0, c1, c2, c3, k0, k1).
struct PhiloxRow {
  uint32_t f0;        // round 1: word 0 = hi(c2 * B) ^ c1 ^ k0
  uint32_t f2;        // round 1: word 2 = hi(c0 * A) ^ f2, f2 = c3 ^ k1
  uint32_t f5;        // round 2: word 0 = hi(w2 * B) ^ f5, f5 = lo(c2 * B) ^ (k0 + WA)
  uint32_t f6;        // round 2: word 2 = f6 ^ lo(c0 * A), f6 = hi(f0 * A) ^ (k1 + WB)
  uint32_t f4;        // round 2: word 3 = lo(f0 * A)
  uint32_t k0, k1;    // key of round 3
};

SRAT_HD PhiloxRow philox_row(uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
  PhiloxRow r;
  const uint64_t pb = (uint64_t)c2 * kMulB;
  r.f0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
  r.f2 = c3 ^ k1;
  const uint64_t pa2 = (uint64_t)r.f0 * kMulA;
  r.f5 = (uint32_t)pb ^ (k0 + kWeylA);
  r.f6 = (uint32_t)(pa2 >> 32) ^ (k1 + kWeylB);
  r.f4 = (uint32_t)pa2;
  r.k0 = k0 + 2u * kWeylA;
  r.k1 = k1 + 2u * kWeylB;
  return r;
}

SRAT_HD Philox4 philox4x32_10_row(uint32_t c0, const PhiloxRow& f) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
  // round 1
  const uint64_t pa = (uint64_t)c0 * kMulA;
  const uint32_t w2 = (uint32_t)(pa >> 32) ^ f.f2;
  // round 2 (word 1 after round 1 is lo(c2 * B), folded into f5)
  const uint64_t pb2 = (uint64_t)w2 * kMulB;
  uint32_t c0r = (uint32_t)(pb2 >> 32) ^ f.f5;
  uint32_t c1r = (uint32_t)pb2;
  uint32_t c2r = f.f6 ^ (uint32_t)pa;
  uint32_t c3r = f.f4;
  uint32_t k0 = f.k0, k1 = f.k1;
#if defined(__HIPCC__)
#pragma unroll
#endif
  for (int r = 2; r < 10; ++r) {
    const uint64_t qa = (uint64_t)c0r * kMulA;
    const uint64_t qb = (uint64_t)c2r * kMulB;
    const uint32_t n0 = xor3((uint32_t)(qb >> 32), c1r, k0);
    const uint32_t n2 = xor3((uint32_t)(qa >> 32), c3r, k1);
    c1r = (uint32_t)qb;
    c3r = (uint32_t)qa;
    c0r = n0;
    c2r = n2;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return Philox4{{c0r, c1r, c2r, c3r}};
}

// The generator for fixed (c0, c2, c3) and key with counter word c1 varying
// (one key group, successive queries): everything of rounds 1-3 that does
// not involve c1 is computed once (PhiloxCol).  Bit-identical to
// philox4x32_10(c0, c1, c2, c3, k0, k1).
struct PhiloxCol {
  uint32_t h0;        // round 1: word 0 = c1 ^ h0,  h0 = hi(c2 * B) ^ k0
  uint32_t r1w1;      // round 1: word 1 = lo(c2 * B)
  uint32_t r1w3;      // round 1: word 3 = lo(c0 * A)
  uint32_t r2w0;      // round 2: word 0 = hi(w2 * B) ^ w1 ^ k0', w2 = hi(c0 * A) ^ c3 ^ k1 (all fixed)
  uint32_t r2w1;      // round 2: word 1 = lo(w2 * B)
  uint32_t r3hi;      // round 3: hi(r2w0 * A) ^ k1''
  uint32_t r3lo;      // round 3: word 3 = lo(r2w0 * A)
  uint32_t k0, k1;    // key of round 4
};

SRAT_HD PhiloxCol philox_col(uint32_t c0, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
  PhiloxCol r;
  const uint64_t pa = (uint64_t)c0 * kMulA;
  const uint64_t pb = (uint64_t)c2 * kMulB;
  r.h0 = (uint32_t)(pb >> 32) ^ k0;
  r.r1w1 = (uint32_t)pb;
  r.r1w3 = (uint32_t)pa;
  const uint32_t w2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
  const uint64_t pb2 = (uint64_t)w2 * kMulB;
  r.r2w0 = (uint32_t)(pb2 >> 32) ^ r.r1w1 ^ (k0 + kWeylA);
  r.r2w1 = (uint32_t)pb2;
  const uint64_t pa3 = (uint64_t)r.r2w0 * kMulA;
  r.r3hi = (uint32_t)(pa3 >> 32) ^ (k1 + 2u * kWeylB);
  r.r3lo = (uint32_t)pa3;
  r.k0 = k0 + 3u * kWeylA;
  r.k1 = k1 + 3u * kWeylB;
  return r;
}

SRAT_HD Philox4 philox4x32_10_col(uint32_t c1, const PhiloxCol& f) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
  // round 1: only word 0 depends on c1
  const uint32_t w0 = c1 ^ f.h0;
  // round 2: word 0 * A varies; word 2 * B is fixed (folded into r2w0, r2w1)
  const uint64_t pa2 = (uint64_t)w0 * kMulA;
  const uint32_t w2 = (uint32_t)(pa2 >> 32) ^ f.r1w3 ^ (f.k1 - 2u * kWeylB);
  const uint32_t w3 = (uint32_t)pa2;
  // round 3: word 0 * A is fixed (r3hi, r3lo); word 2 * B varies
  const uint64_t pb3 = (uint64_t)w2 * kMulB;
  uint32_t c0r = xor3((uint32_t)(pb3 >> 32), f.r2w1, f.k0 - kWeylA);
  uint32_t c1r = (uint32_t)pb3;
  uint32_t c2r = f.r3hi ^ w3;
  uint32_t c3r = f.r3lo;
  uint32_t k0 = f.k0, k1 = f.k1;
#if defined(__HIPCC__)
#pragma unroll
#endif
  for (int r = 3; r < 10; ++r) {
    const uint64_t qa = (uint64_t)c0r * kMulA;
    const uint64_t qb = (uint64_t)c2r * kMulB;
    const uint32_t n0 = xor3((uint32_t)(qb >> 32), c1r, k0);
    const uint32_t n2 = xor3((uint32_t)(qa >> 32), c3r, k1);
    c1r = (uint32_t)qb;
    c3r = (uint32_t)qa;
    c0r = n0;
    c2r = n2;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return Philox4{{c0r, c1r, c2r, c3r}};
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
