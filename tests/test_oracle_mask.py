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
    T = math.floor(f16 * 2 ** 32)
    out = np.zeros((B, Hq, n_qt, W), dtype=np.uint64)
    for b in range(B):
        for h in range(Hq):
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
