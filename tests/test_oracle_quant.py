"""Pins for oracle.quant: closed-form invariants and a second, scalar
implementation whose fp32 rounding comes from struct packing."""
import struct

import numpy as np
import pytest
import torch

from oracle import e4m3, quant


def f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def scalar_quantize(block, code):
    """Direct formula, one element at a time, fp32 rounding via struct."""
    qmax = 127.0 if code == "i8" else 448.0
    a = max(abs(float(x)) for x in block.flat)
    if a == 0:
        return [0] * block.size, 0.0
    # python division is correctly rounded in fp64; rounding that to fp32 is
    # the correctly rounded fp32 quotient (53 >= 2*24 + 2, so the double
    # rounding is innocuous for division of fp32 operands)
    scale = f32(a / qmax)
    inv = f32(qmax / a)
    out = []
    for x in block.flat:
        y = f32(float(x) * inv)    # product of two fp32 is exact in fp64
        if code == "i8":
            c = int(round(y))      # python round: half to even
            c = max(-127, min(127, c))
            out.append(c & 0xFF)
        else:
            y = max(-448.0, min(448.0, y))
            t = torch.tensor([y], dtype=torch.float32).to(torch.float8_e4m3fn)
            out.append(int(t.view(torch.uint8)[0]))
    return out, scale


@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_matches_scalar_implementation(code):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 3, 37, 8)) * rng.choice([0.01, 1, 30], (2, 3, 1, 1)))
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    x[1, 2, 16:32] = 0.0                                  # an all-zero block
    codes, scales = quant.quantize_blocks(x, 16, code)
    assert scales.shape == (2, 3, 3)
    for b in range(2):
        for h in range(3):
            for blk in range(3):
                r0, r1 = blk * 16, min(37, blk * 16 + 16)
                want, s = scalar_quantize(x[b, h, r0:r1], code)
                assert scales[b, h, blk] == np.float32(s)
                assert list(codes[b, h, r0:r1].flat) == want


def test_int8_invariants():
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((1, 4, 200, 64))).to(torch.float16).float().numpy()
    codes, scales = quant.quantize_blocks(x, 64, "i8")
    vals = codes.view(np.int8).astype(np.float64)
    for h in range(4):
        for blk in range(4):
            r0, r1 = blk * 64, min(200, blk * 64 + 64)
            cb = vals[0, h, r0:r1]
            assert np.abs(cb).max() == 127
            s = float(scales[0, h, blk])
            err = np.abs(x[0, h, r0:r1] - cb * s)
            assert (err <= s * (0.5 + 2.0 ** -15)).all()
    assert codes.view(np.int8).min() >= -127


def test_e4m3_invariants():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((1, 2, 128, 128)) * 3).to(torch.bfloat16).float().numpy()
    codes, scales = quant.quantize_blocks(x, 64, "e4m3")
    vals = e4m3.decode(codes)
    for h in range(2):
        for blk in range(2):
            cb = vals[0, h, blk * 64:(blk + 1) * 64]
            assert np.abs(cb).max() == 448.0
            s = float(scales[0, h, blk])
            xb = x[0, h, blk * 64:(blk + 1) * 64]
            # relative error of a normal e4m3 value is at most 2^-4, plus the
            # absolute half-ulp of the subnormal range, plus fp32 slack
            err = np.abs(xb - cb * s)
            assert (err <= np.abs(xb) * 2.0 ** -4 * (1 + 1e-6) + s * 2.0 ** -10 * (1 + 1e-6)).all()


def test_zero_block_and_dequantize():
    x = np.zeros((1, 1, 10, 8), np.float32)
    x[0, 0, 0, 0] = -0.0
    for code in ("i8", "e4m3"):
        c, s = quant.quantize_blocks(x, 4, code)
        assert (c == 0).all() and (s == 0).all()
        assert (quant.dequantize(c, s, 4, code) == 0).all()
