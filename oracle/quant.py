"""Per-block quantisation of Q, K and V (oracle; test infrastructure only).

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

V (the optional 8-bit P V product) is quantised by ``quantize_v_tiles``:
e4m3 codes with one power-of-two scale per block (the scale a gfx950 scaled
matrix instruction applies exactly); see its docstring for the reading.

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


# ---------------------------------------------------------------------------
# V for the 8-bit P V product
# ---------------------------------------------------------------------------

V_EXP_MIN, V_EXP_MAX = -126, 126


def v_block_exponent(a):
    """Exponent e of a V block scale 2**e for block absmax a >= 0.

    e is the smallest integer with a <= 448 * 2**e, so that the scaled block
    fills the top binade of e4m3 without saturating: with a = f * 2**k,
    f in [0.5, 1) (frexp) and 448 = 0.875 * 2**9, that is k - 9, plus one when
    f > 0.875.  e is clamped to [-126, 126] (2**e stays a normal fp32 number);
    an all-zero block gets e = 0.
    """
    a = np.asarray(a, dtype=np.float64)
    f, k = np.frexp(a)
    e = k - 9 + (f > 0.875)
    e = np.where(a > 0, e, 0)
    return np.clip(e, V_EXP_MIN, V_EXP_MAX).astype(np.int64)


def quantize_v_tiles(v, block_rows, lengths=None):
    """Quantise V[B, H, S, D] to e4m3 with power-of-two block scales.

    Reading (the pages quantise only Q and K; this is the optional 8-bit P V
    variant): a block is ``block_rows`` keys times the head dim per (b, h),
    its scale is 2**e with e from ``v_block_exponent`` of the block absmax,
    and code = E4M3(v * 2**-e) with round-half-even.  The scaling is exact,
    so each value is rounded once and never saturates.  Padding keys of a
    variable-length batch count as zeros.

    Returns (codes uint8 [B, H, S, D], scales float32 [B, H, nb] = 2**e).
    """
    x = np.asarray(v, dtype=np.float64)
    B, H, S, D = x.shape
    if lengths is not None:
        lengths = np.asarray(lengths)
        if lengths.shape != (B,) or (lengths < 0).any() or (lengths > S).any():
            raise ValueError("lengths must hold one value in [0, S] per batch entry")
        x = x.copy()
        for b in range(B):
            x[b, :, int(lengths[b]):, :] = 0.0
    nb = -(-S // block_rows)
    codes = np.zeros((B, H, S, D), dtype=np.uint8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for blk in range(nb):
        r0, r1 = blk * block_rows, min(S, (blk + 1) * block_rows)
        xb = x[:, :, r0:r1, :]
        e = v_block_exponent(np.abs(xb).max(axis=(2, 3)))        # [B, H]
        y = np.ldexp(xb, -e[:, :, None, None])
        q = e4m3.encode(y)
        nz = (np.abs(xb).max(axis=(2, 3)) > 0)[:, :, None, None]
        codes[:, :, r0:r1, :] = np.where(nz, q, np.uint8(0))
        scales[:, :, blk] = np.ldexp(1.0, e).astype(np.float32)
    return codes, scales


def v_tile_key_order():
    """Key offset inside a 64-key tile held at each of the 64 byte positions
    of a row of the tile-packed V layout.

    Position 32 * c + p (c in {0, 1}, p in 0..31) holds key
    32 * (p // 16) + 8 * ((p % 16) // 4) + p % 4 + 4 * c: the order in which a
    32x32 matrix-instruction accumulator distributes one row's 64 scores over
    a lane pair, so that a lane's weights, in register order, meet the V codes
    of the same keys.
    """
    pos = np.arange(64)
    c, p = pos // 32, pos % 32
    return 32 * (p // 16) + 8 * ((p % 16) // 4) + p % 4 + 4 * c


def pack_v_tiles(codes, tile_n=64):
    """Tile-packed V codes: [B, H, S, D] -> [B, H, ceil(S / 64), D, 64].

    Tile t, row d, position j holds V code (t * 64 + v_tile_key_order()[j], d);
    keys past S are 0.
    """
    if tile_n != 64:
        raise ValueError("the tile-packed V layout has 64 keys per tile")
    codes = np.asarray(codes, dtype=np.uint8)
    B, H, S, D = codes.shape
    nt = -(-S // 64)
    padded = np.zeros((B, H, nt * 64, D), dtype=np.uint8)
    padded[:, :, :S] = codes
    tiles = padded.reshape(B, H, nt, 64, D)
    return np.ascontiguousarray(tiles[:, :, :, v_tile_key_order(), :].transpose(0, 1, 2, 4, 3))
