"""Random packed precision mask (oracle; test infrastructure only).

Source: "TileMix: Mixed-Precision Attention for Faster LLM Prefill", section 2,
"Packed Bitmasks": a packed bitmask per query row laid over the key tiles, a
0 bit selecting the 16-bit path and a 1 bit the 8-bit path, one bit governing
a group of adjacent key tiles so the mask stays a few bytes per row.

Readings (listed in the design notes):
* one mask row per query tile (tile_m rows): routing is decided per score tile;
* group g covers key tiles [g*G, (g+1)*G); n_g = ceil(n_kt / G); the row is
  W >= ceil(n_g / 64) little-endian uint64 words, bit g % 64 of word g // 64,
  unused bits 0;
* the random template draws each (b, h, qt, g) independently: r is output
  number idx = ((b*Hq + h)*n_qt + qt)*n_g + g of SplitMix64 seeded with
  ``seed``; with T = floor(f16 * 2**32) the group is 16-bit iff
  (r >> 32) < T, and its bit is 1 (8-bit) otherwise.

Structured static template (the pages' routing policy is "static, data-free
structured templates", TileMix section 4, with a "SpTrans75" configuration
named in section 3 but not defined; the reading taken, after the fixed
patterns of sparse transformers, is listed in the design notes): with the
query tile's own group gq = clamp((pos) // (G*tile_n), 0, n_g - 1), pos =
(qt + 1)*tile_m - 1 + S_k - S_q the key position of its last row (queries
aligned with the end of the keys, as for causal attention), and
d = |gq - g|, group g is 16-bit iff

    g < sink   or   d < band   or   (stride > 0 and d % stride == 0),

the same for every (b, h).

SplitMix64 is the generator of Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators" (OOPSLA 2014): the state advances by the
golden-ratio increment 0x9E3779B97F4A7C15 and each output is the state passed
through the variant-13 finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9,
xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).  Output number n
(counting from 0) is the finaliser applied to seed + (n + 1) * increment.
"""
import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1


def splitmix64_int(seed, n):
    """Output number n of SplitMix64 seeded with ``seed`` (Python ints)."""
    z = (seed + (n + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64(seed, n):
    """Vectorised SplitMix64 output number n (uint64 array) for a seed."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + (n + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def n_tiles(S, tile):
    return -(-S // tile)


def group_bits(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, seed):
    """bits[b, h, qt, g] (uint8, 1 = 8-bit path) of the random template.

    frac_16bit: one fraction for every head, or one per query head (a
    sequence of Hq values: per-head mix ratios; the draws are the same, only
    the threshold differs by head)."""
    f = np.asarray(frac_16bit, dtype=np.float64)
    if f.ndim == 0:
        f = np.full(Hq, float(f))
    if f.shape != (Hq,):
        raise ValueError("frac_16bit: one value, or one per query head")
    if not ((f >= 0.0) & (f <= 1.0)).all():
        raise ValueError("frac_16bit outside [0, 1]")
    n_qt = n_tiles(S_q, tile_m)
    n_kt = n_tiles(S_k, tile_n)
    n_g = n_tiles(n_kt, tiles_per_bit)
    # T = floor(f * 2^32) <= 2^32, compared with the upper 32 bits of the draw
    T = np.array([int(np.floor(x * 4294967296.0)) for x in f], dtype=np.uint64)
    idx = np.arange(B * Hq * n_qt * n_g, dtype=np.uint64)
    r = splitmix64(seed, idx).reshape(B, Hq, n_qt, n_g)
    is16 = (r >> np.uint64(32)) < T[None, :, None, None]
    return (~is16).astype(np.uint8)


def pack_bits(bits, words_per_row):
    """Pack bits[..., n_g] into uint64 words[..., words_per_row], LSB first."""
    n_g = bits.shape[-1]
    if words_per_row * 64 < n_g:
        raise ValueError("words_per_row too small")
    words = np.zeros(bits.shape[:-1] + (words_per_row,), dtype=np.uint64)
    for g in range(n_g):
        w, b = divmod(g, 64)
        words[..., w] |= bits[..., g].astype(np.uint64) << np.uint64(b)
    return words


def unpack_bits(words, n_g):
    """Inverse of pack_bits: bits[..., n_g] from uint64 words."""
    words = np.asarray(words, dtype=np.uint64)
    out = np.zeros(words.shape[:-1] + (n_g,), dtype=np.uint8)
    for g in range(n_g):
        w, b = divmod(g, 64)
        out[..., g] = ((words[..., w] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
    return out


def build_mask(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, seed,
               words_per_row):
    """Packed mask words [B, Hq, n_qt, words_per_row] (uint64)."""
    bits = group_bits(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, seed)
    return pack_bits(bits, words_per_row)


def template_group_bits(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, sink, band, stride):
    """bits[b, h, qt, g] (uint8, 1 = 8-bit path) of the structured template:
    the attention-sink groups, a local band around the query tile's own group
    and every stride-th group from it are 16-bit, everything else 8-bit."""
    if sink < 0 or band < 0 or stride < 0:
        raise ValueError("template parameters must be >= 0")
    n_qt = n_tiles(S_q, tile_m)
    n_kt = n_tiles(S_k, tile_n)
    n_g = n_tiles(n_kt, tiles_per_bit)
    bits = np.ones((n_qt, n_g), dtype=np.uint8)
    for qt in range(n_qt):
        pos = (qt + 1) * tile_m - 1 + S_k - S_q
        gq = min(n_g - 1, max(0, pos // (tiles_per_bit * tile_n)))
        for g in range(n_g):
            d = abs(gq - g)
            if g < sink or d < band or (stride > 0 and d % stride == 0):
                bits[qt, g] = 0
    return np.broadcast_to(bits, (B, Hq, n_qt, n_g)).copy()


def build_mask_template(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, sink, band, stride,
                        words_per_row):
    """Packed words [B, Hq, n_qt, words_per_row] (uint64) of the structured template."""
    bits = template_group_bits(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, sink, band, stride)
    return pack_bits(bits, words_per_row)
