"""Oracle: counter-based Philox4x32-10 and the two dropout keep-masks.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

Why a counter-based generator: under selective recomputation the backward
pass re-runs the attention core instead of storing its activations, the
softmax-dropout mask included ("Reducing Activation Recomputation in Large
Transformer Models", LIT-736 record, Key takeaways bullet 4; the "5as/h" term
of the per-token formula on the "Recomputing Activations" plate, "What you
will learn").  A mask that is a pure function of (seed, position) is
regenerated bit-identically instead of stored.

Generator: Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  A round takes
the two 32x32->64-bit products of the multipliers with counter words 0 and 2,
and builds the next counter from their high halves xor'ed with the other two
words and the key, and their low halves.  The key gets the two Weyl
increments between rounds.

Mask definitions (the reading fixed for this library; the pages name no RNG):

* key        = (seed mod 2^32, seed div 2^32)
* attention  : element (query i, key j) of (batch bb, global head hg) uses
               counter (j div 8, i, hg, bb); hidden dropout: element (global
               sequence position sg, batch bb, column c) of dropout site `site`
               uses counter (c div 8, sg, bb, site * 2^24 + 2^31).  Bit 31 of
               word 3 separates the two domains.
* each call gives four 32-bit words = eight 16-bit values, little-endian:
  element index e = (j mod 8) takes word e div 2, bits 16*(e mod 2) .. +15.
* keep  iff  u16 >= T,  T = floor(p * 65536 + 1/2) with p the fp32 value of
  the drop probability, evaluated in double precision.
"""
from __future__ import annotations

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
# round multipliers and Weyl key increments of Philox4x32 (SC'11 paper)
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)   # golden ratio
PHILOX_W1 = np.uint64(0xBB67AE85)   # sqrt(3) - 1
ATTN_DOMAIN = 0
HIDDEN_DOMAIN = 1 << 31


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on broadcastable uint32-valued arrays.

    Returns the four output words as uint64 arrays holding 32-bit values.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((prod1 >> np.uint64(32)) ^ c1 ^ k0,
                          prod1 & MASK32,
                          (prod0 >> np.uint64(32)) ^ c3 ^ k1,
                          prod0 & MASK32)
    return c0, c1, c2, c3


def drop_threshold(p: float) -> int:
    """16-bit threshold T: an element is dropped iff its u16 < T."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("drop probability must lie in [0, 1)")
    T = int(np.floor(p32 * 65536.0 + 0.5))
    # T = 65536 would drop everything, yet no 16-bit value could reach it and
    # the threshold no longer fits a 16-bit half: such p are refused
    if T > 0xFFFF:
        raise ValueError("drop probability rounds to a 16-bit threshold of 65536 (p >= 1 - 2^-17)")
    return T


def _u16_of(words, e):
    """Pick the 16-bit value e (0..7) out of the four words of each call."""
    w0, w1, w2, w3 = words
    e = np.asarray(e, dtype=np.uint64)
    word = np.where(e >> np.uint64(1) == 0, w0,
           np.where(e >> np.uint64(1) == 1, w1,
           np.where(e >> np.uint64(1) == 2, w2, w3)))
    return (word >> (np.uint64(16) * (e & np.uint64(1)))) & np.uint64(0xFFFF)


def attn_u16(seed: int, bb: int, head: int, i, j):
    """16-bit draws for attention elements (query i, key j); i, j broadcast."""
    i = np.asarray(i, dtype=np.uint64)
    j = np.asarray(j, dtype=np.uint64)
    words = philox4x32_10(j >> np.uint64(3), i, np.uint64(head),
                          np.uint64(bb | ATTN_DOMAIN), seed & 0xFFFFFFFF, seed >> 32)
    return _u16_of(words, j & np.uint64(7))


def attn_keep_mask(seed: int, p: float, bb: int, head: int, s_q: int, s_k: int,
                   row0: int = 0) -> np.ndarray:
    """Boolean keep mask of shape [s_q, s_k] for query rows row0..row0+s_q-1."""
    T = drop_threshold(p)
    if T == 0:
        return np.ones((s_q, s_k), dtype=bool)
    i = np.arange(row0, row0 + s_q, dtype=np.uint64)[:, None]
    j = np.arange(s_k, dtype=np.uint64)[None, :]
    return attn_u16(seed, bb, head, i, j) >= np.uint64(T)


def hidden_u16(seed: int, site: int, bb, seq, col):
    """16-bit draws for hidden-dropout elements; bb, seq, col broadcast."""
    col = np.asarray(col, dtype=np.uint64)
    tag = np.uint64(((site & 0x7F) << 24) | HIDDEN_DOMAIN)
    words = philox4x32_10(col >> np.uint64(3), np.asarray(seq, dtype=np.uint64),
                          np.asarray(bb, dtype=np.uint64), tag,
                          seed & 0xFFFFFFFF, seed >> 32)
    return _u16_of(words, col & np.uint64(7))


def hidden_keep_mask(seed: int, p: float, site: int, s_local: int, b: int, h: int,
                     seq_offset: int = 0) -> np.ndarray:
    """Boolean keep mask of shape [s_local, b, h] for one rank's sequence slice."""
    T = drop_threshold(p)
    if T == 0:
        return np.ones((s_local, b, h), dtype=bool)
    seq = np.arange(seq_offset, seq_offset + s_local, dtype=np.uint64)[:, None, None]
    bb = np.arange(b, dtype=np.uint64)[None, :, None]
    col = np.arange(h, dtype=np.uint64)[None, None, :]
    return hidden_u16(seed, site, bb, seq, col) >= np.uint64(T)
