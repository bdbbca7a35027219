"""Per-block absmax quantisation of Q or K (oracle; test infrastructure only).

Source: "TileMix: Mixed-Precision Attention for Faster LLM Prefill", section 2,
"The Dual-Path Engine": on the 8-bit path queries and keys are quantised and
the products are rescaled with per-block scale factors.  The LampAttention
abstract uses an 8-bit floating-point format for the same products.

Readings where the pages are silent (each listed in the design notes):
* a block is ``block_rows`` consecutive sequence rows times the full head dim,
  per (batch, head); the last block of a sequence may be short;
* symmetric absmax scaling, no zero point; QMAX = 127 for int8 (-128 unused),
  448 for e4m3;
* the arithmetic is fp32, as a kernel would do it:
  ``scale = fl32(a / QMAX)``, ``inv = fl32(QMAX / a)``, ``y = fl32(x * inv)``;
  int8 code = clamp(round-half-even(y), -127, 127); e4m3 code =
  E4M3(clamp(y, -448, 448)) with round-half-even;
* an all-zero block has scale 0 and all codes 0.

numpy float32 arithmetic is IEEE single precision with round-to-nearest-even,
so the expressions below are the fp32 operations themselves.
"""
import numpy as np

from . import e4m3

QMAX = {"i8": 127.0, "e4m3": 448.0}


def quantize_blocks(x, block_rows, code, lengths=None):
    """Quantise x[B, H, S, D] (values exactly representable in fp32).

    Returns (codes, scales): codes uint8 [B, H, S, D] (int8 two's complement or
    E4M3FN bits), scales float32 [B, H, ceil(S / block_rows)].

    ``lengths`` (variable-length batch, one length per b, 0 <= L[b] <= S):
    rows L[b] .. S-1 of sequence b are padding and count as zeros, so they do
    not enter a block's absmax and their codes are 0.
    """
    if code not in QMAX:
        raise ValueError(code)
    x = np.asarray(x, dtype=np.float32)
    B, H, S, D = x.shape
    if lengths is not None:
        lengths = np.asarray(lengths)
        if lengths.shape != (B,) or (lengths < 0).any() or (lengths > S).any():
            raise ValueError("lengths must hold one value in [0, S] per batch entry")
        x = x.copy()
        for b in range(B):
            x[b, :, int(lengths[b]):, :] = 0.0
    nb = -(-S // block_rows)
    qmax = np.float32(QMAX[code])
    codes = np.zeros((B, H, S, D), dtype=np.uint8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for blk in range(nb):
        r0, r1 = blk * block_rows, min(S, (blk + 1) * block_rows)
        xb = x[:, :, r0:r1, :]
        a = np.abs(xb).max(axis=(2, 3))                      # [B, H], exact
        nz = a > 0
        a_safe = np.where(nz, a, np.float32(1.0)).astype(np.float32)
        scale = np.where(nz, a_safe / qmax, np.float32(0.0)).astype(np.float32)
        inv = np.where(nz, qmax / a_safe, np.float32(0.0)).astype(np.float32)
        y = (xb * inv[:, :, None, None]).astype(np.float32)
        if code == "i8":
            q = np.clip(np.rint(y), -127, 127).astype(np.int8).view(np.uint8)
        else:
            q = e4m3.encode(np.clip(y.astype(np.float64), -448.0, 448.0))
            # an all-zero block encodes as +0 regardless of the sign of zero
            q = np.where(nz[:, :, None, None], q, np.uint8(0)).astype(np.uint8)
        codes[:, :, r0:r1, :] = q
        scales[:, :, blk] = scale
    return codes, scales


def code_values(codes, code):
    """Numeric value of each code as float64 (int8 integer or e4m3 value)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if code == "i8":
        return codes.view(np.int8).astype(np.float64)
    return e4m3.decode(codes)


def dequantize(codes, scales, block_rows, code):
    """code value times its block scale, float64 [B, H, S, D]."""
    vals = code_values(codes, code)
    S = vals.shape[2]
    rows = np.arange(S) // block_rows
    return vals * scales.astype(np.float64)[:, :, rows][..., None]
