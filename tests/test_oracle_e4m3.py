"""Pins for oracle.e4m3 against the OCP E4M3 definition and torch's cast."""
import os

import numpy as np
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_constants.txt")


def test_spec_constants():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        c, val = line.split()
        got = e4m3.decode(np.array([int(c, 16)], np.uint8))[0]
        want = float(val)
        assert got == want and np.signbit(got) == val.startswith("-"), (c, got, want)


def test_nan_codes():
    assert np.isnan(e4m3.decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert (e4m3.encode(e4m3.decode(codes)) == codes).all()


def test_midpoints_round_to_even_and_neighbours():
    mags = e4m3.decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert (np.diff(mags) > 0).all()
    for c in range(0x7E):
        mid = 0.5 * (mags[c] + mags[c + 1])
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(np.array([mid]))[0] == even
        assert e4m3.encode(np.array([-mid]))[0] == (even | 0x80)
        eps = (mags[c + 1] - mags[c]) * 1e-6
        assert e4m3.encode(np.array([mid - eps]))[0] == c
        assert e4m3.encode(np.array([mid + eps]))[0] == c + 1


def test_saturation_and_signed_zero():
    x = np.array([448.0, 449.0, 1e6, -1e6, -0.0, -1e-9, 1e-9, 2.0 ** -10, 1.5 * 2.0 ** -10])
    c = e4m3.encode(x)
    assert list(c) == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x00, 0x01]


def test_matches_torch_float8_e4m3fn():
    # torch's cast is RNE but not saturating: clamp to +-448 first.
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(400_000) * 30,
        rng.uniform(-448, 448, 300_000),
        rng.standard_normal(300_000) * 0.01,
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(x.astype(np.float64))
    assert (ref == got).all()


def test_rounding_boundaries_are_midpoints():
    b = e4m3.rounding_boundaries()
    assert len(b) == 126
    codes_below = e4m3.encode(b * (1 - 1e-9))
    codes_above = e4m3.encode(b * (1 + 1e-9))
    assert (codes_above.astype(int) - codes_below.astype(int) == 1).all()
