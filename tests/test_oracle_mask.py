"""Pins for oracle.mask: SplitMix64 known answers, a second loop-based
implementation, the extremes of the 16-bit fraction, and a binomial check."""
import math
import os

import numpy as np
import pytest

from oracle import mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_kat.txt")


def test_splitmix64_known_answers():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        seed, n, val = line.split()
        assert mask.splitmix64_int(int(seed), int(n)) == int(val, 16)
        assert int(mask.splitmix64(int(seed), np.array([int(n)]))[0]) == int(val, 16)


def test_splitmix64_sequential_state():
    # the counter form equals stepping the state one increment at a time
    seed = 0x1234_5678_9ABC_DEF0
    state = seed
    for n in range(50):
        state = (state + mask.GAMMA) & mask.MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask.MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask.MASK64
        assert (z ^ (z >> 31)) == mask.splitmix64_int(seed, n)


def brute_mask(B, Hq, S_q, S_k, tm, tn, G, f16, seed, W):
    n_qt, n_kt = -(-S_q // tm), -(-S_k // tn)
    n_g = -(-n_kt // G)
    out = np.zeros((B, Hq, n_qt, W), dtype=np.uint64)
    for b in range(B):
        for h in range(Hq):
            T = math.floor((f16[h] if isinstance(f16, (list, tuple)) else f16) * 2 ** 32)
            for qt in range(n_qt):
                words = [0] * W
                for g in range(n_g):
                    idx = ((b * Hq + h) * n_qt + qt) * n_g + g
                    r = mask.splitmix64_int(seed, idx)
                    if not (r >> 32) < T:
                        words[g // 64] |= 1 << (g % 64)
                out[b, h, qt] = words
    return out


@pytest.mark.parametrize("shape", [
    (1, 1, 256, 256, 64, 64, 1, 0.5, 2001, 1),
    (2, 3, 300, 300, 128, 64, 4, 0.25, 7, 1),
    (1, 2, 8192, 8192, 128, 64, 1, 0.3, 9, 2),
    (1, 1, 100, 100, 64, 64, 1, 0.5, 11, 3),
])
def test_matches_brute_force(shape):
    B, Hq, S_q, S_k, tm, tn, G, f16, seed, W = shape
    got = mask.build_mask(B, Hq, S_q, S_k, tm, tn, G, f16, seed, W)
    assert (got == brute_mask(*shape)).all()


@pytest.mark.parametrize("shape", [
    (2, 4, 300, 300, 128, 64, 4, [0.0, 0.25, 0.9, 1.0], 17, 1),
    (1, 3, 8192, 8192, 128, 64, 1, [0.1, 0.5, 0.3], 23, 2),
])
def test_per_head_matches_brute_force(shape):
    B, Hq, S_q, S_k, tm, tn, G, f16, seed, W = shape
    got = mask.build_mask(B, Hq, S_q, S_k, tm, tn, G, f16, seed, W)
    assert (got == brute_mask(*shape)).all()


def test_per_head_equal_fractions_is_scalar():
    a = mask.build_mask(2, 5, 700, 700, 128, 64, 2, [0.3] * 5, 4, 1)
    assert (a == mask.build_mask(2, 5, 700, 700, 128, 64, 2, 0.3, 4, 1)).all()
    with pytest.raises(ValueError):
        mask.group_bits(1, 3, 64, 64, 64, 64, 1, [0.1, 0.2], 1)
    with pytest.raises(ValueError):
        mask.group_bits(1, 2, 64, 64, 64, 64, 1, [0.1, 1.5], 1)


def test_extremes_and_padding():
    n_kt = 128 // 64 * 35
    for f16, want in ((0.0, 1), (1.0, 0)):
        w = mask.build_mask(1, 2, 256, 64 * n_kt, 128, 64, 1, f16, 5, 2)
        bits = mask.unpack_bits(w, 128)
        assert (bits[..., :n_kt] == want).all()
        assert (bits[..., n_kt:] == 0).all()


def test_binomial_fraction():
    f16 = 0.25
    bits = mask.group_bits(2, 32, 16384, 16384, 128, 64, 4, f16, 2030)
    n = bits.size
    frac16 = 1 - bits.mean()
    sd = math.sqrt(f16 * (1 - f16) / n)
    assert abs(frac16 - f16) < 5 * sd


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2, (3, 4, 130)).astype(np.uint8)
    assert (mask.unpack_bits(mask.pack_bits(bits, 3), 130) == bits).all()
    with pytest.raises(ValueError):
        mask.pack_bits(bits, 2)


# ---------------------------------------------------------------------------
# structured static template: expected bit rows written out by hand from the
# definition (g < sink, or d < band, or d % stride == 0 with d = |gq - g|)
# ---------------------------------------------------------------------------

def _rows(strings):
    return np.array([[int(c) for c in r] for r in strings], dtype=np.uint8)


def test_template_hand_worked_square():
    # tile_m = tile_n = 64, G = 1, S = 512: 8 query tiles, 8 groups, gq = qt;
    # sink 1, band 2, stride 3.  Row qt lists bits g = 0..7 (0 = 16-bit).
    want = _rows(["00101101",    # qt 0: 16-bit {0, 1, 3, 6}
                  "00010110",    # qt 1: {0, 1, 2, 4, 7}
                  "00001011",    # qt 2: {0, 1, 2, 3, 5}
                  "01000101",    # qt 3: {0, 2, 3, 4, 6}
                  "00100010",    # qt 4: {0, 1, 3, 4, 5, 7}
                  "01010001",    # qt 5: {0, 2, 4, 5, 6}
                  "01101000",    # qt 6: {0, 3, 5, 6, 7}
                  "00110100"])   # qt 7: {0, 1, 4, 6, 7}
    got = mask.template_group_bits(1, 1, 512, 512, 64, 64, 1, 1, 2, 3)[0, 0]
    assert (got == want).all()


def test_template_hand_worked_tall_tiles():
    # tile_m = 128, tile_n = 64, G = 1, S = 512: gq = 2 qt + 1 (the group of
    # the tile's last row); band 3 only
    want = _rows(["00001111",    # gq 1: groups 0..3
                  "10000011",    # gq 3: groups 1..5
                  "11100000",    # gq 5: groups 3..7
                  "11111000"])   # gq 7: groups 5..7
    got = mask.template_group_bits(2, 3, 512, 512, 128, 64, 1, 0, 3, 0)
    assert got.shape == (2, 3, 4, 8)
    for b in range(2):
        for h in range(3):
            assert (got[b, h] == want).all()


def test_template_extremes_and_grouping():
    # no template part: everything 8-bit; a band covering every group or a
    # sink of n_g groups: everything 16-bit; stride 1: everything 16-bit
    assert mask.template_group_bits(1, 2, 1000, 1000, 128, 64, 4, 0, 0, 0).all()
    n_g = -(-(-(-1000 // 64)) // 4)
    for sink, band, stride in ((n_g, 0, 0), (0, n_g, 0), (0, 0, 1)):
        assert not mask.template_group_bits(1, 2, 1000, 1000, 128, 64, 4, sink, band, stride).any()
    # G = 4 groups of 256 keys, tile_m = 128: query tiles 2j and 2j+1 share gq = j
    bits = mask.template_group_bits(1, 1, 2048, 2048, 128, 64, 4, 0, 1, 0)[0, 0]
    for qt in range(16):
        assert bits[qt].tolist() == [0 if g == qt // 2 else 1 for g in range(8)]
    # keys beyond the queries (a chunk of 128 queries after 896 earlier
    # tokens): the tile's last row sits at key 1023, group 15
    bits = mask.template_group_bits(1, 1, 128, 1024, 128, 64, 1, 0, 1, 0)[0, 0]
    assert bits.tolist() == [[1] * 15 + [0]]
    # 300 queries after 212 tokens, tile_m 64, G 2 (128 keys per group):
    # tile ends at keys 275, 339, 403, 467, 531 -> groups 2, 2, 3, 3, 4 -> 3
    # (clamped: 4 groups)
    bits = mask.template_group_bits(1, 1, 300, 512, 64, 64, 2, 0, 1, 0)[0, 0]
    assert [int(np.argmin(r)) for r in bits] == [2, 2, 3, 3, 3] and (bits.sum(1) == 3).all()
    # queries beyond the keys: positions before key 0 clamp to group 0, the
    # others land on the last group
    bits = mask.template_group_bits(1, 1, 1024, 128, 128, 64, 1, 0, 1, 0)[0, 0]
    assert (bits[:7, 0] == 0).all() and (bits[:7, 1] == 1).all()
    assert bits[7].tolist() == [1, 0]


def test_template_packing_multiword():
    # 200 groups need 4 words; bit g sits in word g // 64 at g % 64
    B, Hq, S, tm, tn, G = 1, 1, 200 * 64, 128, 64, 1
    bits = mask.template_group_bits(B, Hq, S, S, tm, tn, G, 3, 4, 17)
    words = mask.build_mask_template(B, Hq, S, S, tm, tn, G, 3, 4, 17, 5)
    assert words.shape == (1, 1, 100, 5) and (words[..., 4] == 0).all()
    for qt in (0, 37, 99):
        for g in range(200):
            w, bit = divmod(g, 64)
            assert ((int(words[0, 0, qt, w]) >> bit) & 1) == bits[0, 0, qt, g]
