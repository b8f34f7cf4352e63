"""Pins for the oracle's Philox4x32-10 and dropout masks.

External pin: rocRAND's own Philox4x32-10 engine (header-only host code,
compiled here with g++), an implementation independent of the oracle.
"""
import numpy as np
import pytest

from oracle import philox as ph
from tests.support.rocrand_ref import philox_words

M32 = 0xFFFFFFFF


def _cases(n, seed=1234):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        s = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(x) for x in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        out.append((s, *c))
    # edges: all-zero, all-ones, carries in the key schedule
    out += [(0, 0, 0, 0, 0), (2**64 - 1, M32, M32, M32, M32), (M32, 1, 2, 3, 4),
            (1 << 32, M32, 0, M32, 0)]
    return out


def test_philox_matches_rocrand_engine():
    cases = _cases(3000)
    ref = philox_words(cases)
    seeds = np.array([c[0] for c in cases], dtype=np.uint64)
    ctr = np.array([c[1:] for c in cases], dtype=np.uint64)
    got = np.zeros_like(ref)
    # one key per call of the oracle: group by seed
    for idx, s in enumerate(seeds):
        w = ph.philox4x32_10(ctr[idx, 0], ctr[idx, 1], ctr[idx, 2], ctr[idx, 3],
                             int(s) & M32, int(s) >> 32)
        got[idx] = [int(x) for x in w]
    np.testing.assert_array_equal(got, ref)


def test_philox_vectorised_same_as_scalar():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 2**32, size=(4, 500), dtype=np.uint64)
    vec = np.stack(ph.philox4x32_10(c[0], c[1], c[2], c[3], 0xDEADBEEF, 0x12345678))
    for n in range(0, 500, 37):
        sc = ph.philox4x32_10(c[0, n], c[1, n], c[2, n], c[3, n], 0xDEADBEEF, 0x12345678)
        assert [int(x) for x in sc] == [int(x) for x in vec[:, n]]


def test_attention_u16_layout_against_rocrand():
    """Element (i, j) of (batch bb, head hg) takes half-word j%8 of call (j//8, i, hg, bb)."""
    seed, bb, hg = 0x0123456789ABCDEF, 3, 11
    i = np.array([0, 1, 17, 2047, 8191])
    j = np.array([0, 7, 8, 13, 8190])
    ref = philox_words([(seed, int(jj) >> 3, int(ii), hg, bb) for ii, jj in zip(i, j)])
    want = [(int(r[(jj & 7) >> 1]) >> (16 * (jj & 1))) & 0xFFFF for r, jj in zip(ref, j)]
    got = ph.attn_u16(seed, bb, hg, i, j)
    np.testing.assert_array_equal(got, np.array(want, dtype=np.uint64))


def test_hidden_u16_layout_against_rocrand():
    seed, site = 99, 2
    seq = np.array([0, 255, 256, 70000])
    bb = np.array([0, 3, 1, 0])
    col = np.array([0, 9, 6143, 20479])
    tag = (site << 24) | (1 << 31)
    ref = philox_words([(seed, int(c) >> 3, int(s), int(b), tag) for s, b, c in zip(seq, bb, col)])
    want = [(int(r[(c & 7) >> 1]) >> (16 * (c & 1))) & 0xFFFF for r, c in zip(ref, col)]
    np.testing.assert_array_equal(ph.hidden_u16(seed, site, bb, seq, col),
                                  np.array(want, dtype=np.uint64))


def test_threshold_values():
    assert ph.drop_threshold(0.0) == 0
    assert ph.drop_threshold(0.1) == 6554          # 6553.6 rounds up
    assert ph.drop_threshold(0.5) == 32768
    assert ph.drop_threshold(0.25) == 16384
    with pytest.raises(ValueError):
        ph.drop_threshold(1.0)
    with pytest.raises(ValueError):
        ph.drop_threshold(-0.01)


def test_p_zero_keeps_everything():
    assert ph.attn_keep_mask(5, 0.0, 0, 0, 64, 64).all()
    assert ph.hidden_keep_mask(5, 0.0, 1, 4, 2, 40).all()


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_keep_rate_statistics(p):
    m = ph.attn_keep_mask(0, p, 1, 2, 512, 2048)
    keep = 1.0 - ph.drop_threshold(p) / 65536.0
    n = m.size
    sigma = np.sqrt(keep * (1 - keep) / n)
    assert abs(m.mean() - keep) < 5 * sigma
    hm = ph.hidden_keep_mask(0, p, 1, 256, 4, 1024)
    sigma = np.sqrt(keep * (1 - keep) / hm.size)
    assert abs(hm.mean() - keep) < 5 * sigma


def test_masks_differ_across_keys():
    base = ph.attn_keep_mask(0, 0.1, 0, 0, 64, 64)
    for other in (ph.attn_keep_mask(1, 0.1, 0, 0, 64, 64),       # seed
                  ph.attn_keep_mask(0, 0.1, 1, 0, 64, 64),       # batch
                  ph.attn_keep_mask(0, 0.1, 0, 1, 64, 64),       # head
                  ph.attn_keep_mask(0, 0.1, 0, 0, 64, 64, row0=64)):  # rows
        assert (base != other).mean() > 0.1


def test_row_offset_is_a_slice():
    full = ph.attn_keep_mask(3, 0.1, 0, 5, 256, 256)
    part = ph.attn_keep_mask(3, 0.1, 0, 5, 64, 256, row0=128)
    np.testing.assert_array_equal(full[128:192], part)


def test_hidden_seq_offset_is_a_slice():
    full = ph.hidden_keep_mask(3, 0.1, 1, 64, 2, 96, seq_offset=0)
    part = ph.hidden_keep_mask(3, 0.1, 1, 16, 2, 96, seq_offset=32)
    np.testing.assert_array_equal(full[32:48], part)


def test_domains_do_not_collide():
    # word 3 of an attention counter is the batch index (< 2^31); of a hidden
    # counter it has bit 31 set, so the two streams never share a counter.
    i = np.arange(8)
    a = ph.attn_u16(0, 0, 0, i, np.arange(8))
    h = ph.hidden_u16(0, 0, np.zeros(8, np.uint64), i, np.arange(8))
    assert not np.array_equal(a, h)


def test_mask_element_indexing_against_rocrand():
    """mask[i, j] (and hidden mask[s, b, c]) decided from rocRAND's words by hand."""
    seed, p, bb, hg = 5, 0.4, 2, 6
    T = ph.drop_threshold(p)
    m = ph.attn_keep_mask(seed, p, bb, hg, 40, 48, row0=100)
    picks = [(0, 47), (39, 0), (3, 17), (21, 8)]
    ref = philox_words([(seed, j >> 3, 100 + i, hg, bb) for i, j in picks])
    for (i, j), r in zip(picks, ref):
        u = (int(r[(j & 7) >> 1]) >> (16 * (j & 1))) & 0xFFFF
        assert bool(m[i, j]) == (u >= T)
    hm = ph.hidden_keep_mask(seed, p, 1, 6, 3, 40, seq_offset=10)
    tag = (1 << 24) | (1 << 31)
    hp = [(0, 0, 39), (5, 2, 8), (3, 1, 17)]
    ref = philox_words([(seed, c >> 3, 10 + sl, b, tag) for sl, b, c in hp])
    for (sl, b, c), r in zip(hp, ref):
        u = (int(r[(c & 7) >> 1]) >> (16 * (c & 1))) & 0xFFFF
        assert bool(hm[sl, b, c]) == (u >= T)
