"""Pins for the oracle's optional 8-bit P V product (V quantiser, tile-packed
layout, attention).

* the block exponent against its defining inequality a <= 448 * 2**e < 2a,
  evaluated with exact fp64 scaling instead of frexp;
* codes against a scalar brute force that rounds with torch's
  float8_e4m3fn table (not oracle.e4m3) and finds e by search;
* hand-derived values (all-ones block, 448 / 450 boundaries, zero block);
* the packed layout against hand-listed key positions and the 32x32
  accumulator layout;
* attention: V = 1 gives O = 1; V already on the e4m3 grid of its block gives
  the exp8 result without 8-bit P V; all tiles 16-bit gives the exp8 result;
  a scalar brute-force emulation of the tile loop.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import e4m3, quant

from test_oracle_attention import brute_logit, e4m3_torch, rand16, tiny_problem


# ---------------------------------------------------------------------------
# block exponent and codes
# ---------------------------------------------------------------------------

def test_exponent_hand_values():
    # 448 = 0.875 * 2**9 fits at e = 0; 224 fits at e = -1; 1 <= 1.75 at e = -8;
    # 450 > 448 needs e = 1; zero block e = 0; the clamp keeps 2**e normal.
    got = quant.v_block_exponent([448.0, 224.0, 1.0, 450.0, 0.0, 1e-40, 2.0 ** 100])
    assert list(got) == [0, -1, -8, 1, 0, -126, 92]


def test_exponent_defining_inequality():
    rng = np.random.default_rng(5)
    a = np.exp(rng.uniform(-60, 60, 20000)).astype(np.float32).astype(np.float64)
    a = np.concatenate([a, 448.0 * np.exp2(np.arange(-20, 20)), 448.0 * np.exp2(np.arange(-20, 20)) * (1 + 2 ** -20)])
    e = quant.v_block_exponent(a)
    assert (a <= np.ldexp(448.0, e)).all()
    assert (a > np.ldexp(448.0, e - 1)).all()


def _e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return codes.to(torch.float64).numpy()


def brute_v_codes(xb):
    """Scalar quantisation of one block: e by search, nearest e4m3 by scanning
    the 256 codes (ties to the even code; the sign of zero kept)."""
    table = _e4m3_table()
    a = max(abs(float(x)) for x in xb.ravel())
    if a == 0:
        return np.zeros(xb.shape, dtype=np.uint8), 1.0
    e = -126
    while not a <= 448.0 * 2.0 ** e:
        e += 1
    out = np.zeros(xb.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(xb):
        y = float(x) * 2.0 ** -e
        best = None
        for c in range(256):
            t = table[c]
            if math.isnan(t) or (c & 0x80) != (0x80 if math.copysign(1.0, y) < 0 else 0):
                continue
            d = abs(t - y)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        out[idx] = best[1]
    return out, 2.0 ** e


@pytest.mark.parametrize("seed,scale", [(1, 1.0), (2, 37.5), (3, 1e-3)])
def test_codes_brute_force(seed, scale):
    v = rand16((1, 2, 20, 4), seed, scale=scale)
    codes, scales = quant.quantize_v_tiles(v, 8)
    for h in range(2):
        for blk in range(3):
            r0, r1 = 8 * blk, min(20, 8 * blk + 8)
            c_b, s_b = brute_v_codes(v[0, h, r0:r1])
            assert scales[0, h, blk] == s_b
            assert (codes[0, h, r0:r1] == c_b).all()


def test_codes_hand_values():
    v = np.ones((1, 1, 64, 8))
    v[0, 0, 1::2] = -1.0
    codes, scales = quant.quantize_v_tiles(v, 64)
    # 1 * 2**8 = 256 = 1.0 * 2**8: exponent field 15, mantissa 0 -> 0x78
    assert scales[0, 0, 0] == 2.0 ** -8
    assert (codes[0, 0, 0::2] == 0x78).all() and (codes[0, 0, 1::2] == 0xF8).all()
    # block max 448: e = 0, value 1.0 is code 0x38; max 450: e = 1, 450 / 2 = 225
    # rounds to 224 = 1.75 * 2**7 (0x76), and 1.0 / 2 = 0.5 is code 0x30
    w = np.zeros((1, 1, 2, 2))
    w[0, 0, 0] = [448.0, 1.0]
    w[0, 0, 1] = [450.0, 1.0]
    c1, s1 = quant.quantize_v_tiles(w[:, :, :1], 1)
    c2, s2 = quant.quantize_v_tiles(w[:, :, 1:], 1)
    assert s1[0, 0, 0] == 1.0 and list(c1[0, 0, 0]) == [0x7E, 0x38]
    assert s2[0, 0, 0] == 2.0 and list(c2[0, 0, 0]) == [0x76, 0x30]
    z, sz = quant.quantize_v_tiles(np.zeros((1, 1, 5, 4)), 64)
    assert (z == 0).all() and sz[0, 0, 0] == 1.0


def test_top_binade_and_round_trip():
    v = rand16((2, 3, 300, 64), 9, scale=3.0)
    codes, scales = quant.quantize_v_tiles(v, 64)
    s = scales.astype(np.float64)
    m, _ = np.frexp(s)
    assert (m == 0.5).all()                                 # powers of two
    vals = e4m3.decode(codes)
    for blk in range(scales.shape[2]):
        mx = np.abs(vals[:, :, 64 * blk:64 * blk + 64]).max(axis=(2, 3))
        assert ((mx >= 224) & (mx <= 448)).all()      # (224, 448] before rounding
    deq = quant.dequantize(codes, scales, 64, "e4m3")
    rel = np.abs(deq - v) / np.maximum(np.abs(v), 2.0 ** -6 * s[:, :, np.arange(300) // 64][..., None])
    assert rel.max() <= 2.0 ** -4 + 1e-12                  # half an e4m3 ulp


def test_varlen_padding():
    v = rand16((2, 1, 100, 8), 4)
    codes, scales = quant.quantize_v_tiles(v, 64, lengths=[100, 70])
    assert (codes[1, :, 70:] == 0).all()
    c1, s1 = quant.quantize_v_tiles(v[1:, :, :70], 64)
    assert (codes[1, :, :70] == c1[0]).all() and (scales[1] == s1[0]).all()


# ---------------------------------------------------------------------------
# tile-packed layout
# ---------------------------------------------------------------------------

def test_key_order_hand_listed():
    o = quant.v_tile_key_order()
    for pos, key in [(0, 0), (3, 3), (4, 8), (15, 27), (16, 32), (31, 59), (32, 4), (36, 12), (63, 63)]:
        assert o[pos] == key
    assert sorted(o) == list(range(64))


def test_key_order_is_accumulator_layout():
    # S^T = K Q^T with two 32x32 blocks of keys: lane l, register i of block kb
    # holds key 32 kb + 8 (i // 4) + 4 (l // 32) + i % 4
    o = quant.v_tile_key_order()
    for half in range(2):
        for kb in range(2):
            for i in range(16):
                assert o[32 * half + 16 * kb + i] == 32 * kb + 8 * (i // 4) + 4 * half + i % 4


def test_pack_tiles():
    S, D = 100, 3
    codes = (np.arange(S)[:, None] * 3 + np.arange(D)[None, :]) % 251 + 1
    codes = codes.astype(np.uint8)[None, None]
    packed = quant.pack_v_tiles(codes)
    assert packed.shape == (1, 1, 2, D, 64)
    o = quant.v_tile_key_order()
    for t in range(2):
        for d in range(D):
            for j in range(64):
                key = 64 * t + o[j]
                want = codes[0, 0, key, d] if key < S else 0
                assert packed[0, 0, t, d, j] == want


# ---------------------------------------------------------------------------
# attention with 8-bit P V
# ---------------------------------------------------------------------------

def lamp_O(P, h=0, b=0):
    res, rows, _ = A.attn_lamp(P, b, h, np.arange(-(-P.S_q // P.sub_rows)))
    return res.O


def test_requires_exp8_and_mask_routing():
    with pytest.raises(ValueError):
        tiny_problem(seed=1, code="i8", S=8, pv8=True)
    with pytest.raises(ValueError):
        tiny_problem(seed=1, code="i8", S=8, pv8=True, exp8=True, adaptive=True)


@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_v_ones_gives_ones(code):
    q = rand16((1, 2, 40, 8), 1)
    k = rand16((1, 1, 40, 8), 2)
    v = np.ones((1, 1, 40, 8))
    P = A.make_problem(q, k, v, causal=True, code=code, tile_m=8, tile_n=8, tiles_per_bit=1,
                       frac_16bit=0.3, seed=7, exp8=True, pv8=True)
    for h in range(2):
        assert np.abs(lamp_O(P, h) - 1.0).max() < 1e-12


@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_v_on_grid_equals_exp8(code):
    q = rand16((1, 2, 48, 8), 3)
    k = rand16((1, 1, 48, 8), 4)
    v = rand16((1, 1, 48, 8), 5)
    vc, vs = quant.quantize_v_tiles(v, 8)
    vg = quant.dequantize(vc, vs, 8, "e4m3")               # already on the grid
    kw = dict(causal=True, code=code, tile_m=8, tile_n=8, tiles_per_bit=1, frac_16bit=0.4, seed=8,
              exp8=True)
    P8 = A.make_problem(q, k, vg, pv8=True, **kw)
    assert (P8.v_codes == vc).all()                         # requantisation is idempotent
    P = A.make_problem(q, k, vg, **kw)
    for h in range(2):
        assert np.abs(lamp_O(P8, h) - lamp_O(P, h)).max() < 1e-12


def test_all_16bit_ignores_v_codes():
    kw = dict(seed=6, code="e4m3", S=24, D=8, tm=8, tn=8, f16=1.0, exp8=True)
    P8 = tiny_problem(pv8=True, **kw)
    P = tiny_problem(**kw)
    assert np.abs(lamp_O(P8, 1) - lamp_O(P, 1)).max() == 0.0


def brute_lamp_pv8(P, b, h):
    """Scalar tile loop with exp8 weights and 8-bit V on 8-bit tiles; V codes
    from the scalar brute-force quantiser."""
    S, D, tn = P.S_q, P.D, P.tile_n
    kvh = P.kvh(h)
    v8 = np.zeros((P.S_k, D))
    for blk in range(-(-P.S_k // tn)):
        r0, r1 = blk * tn, min(P.S_k, (blk + 1) * tn)
        c_b, s_b = brute_v_codes(P.v[b, kvh, r0:r1])
        v8[r0:r1] = _e4m3_table()[c_b.astype(np.int64)] * s_b
    m = [-math.inf] * S
    l = [0.0] * S
    acc = [[0.0] * D for _ in range(S)]
    for kt in range(P.n_kt):
        cols = range(kt * tn, min(P.S_k, (kt + 1) * tn))
        for i in range(S):
            js = [j for j in cols if (not P.causal or j <= i)]
            if not js:
                continue
            sv = [brute_logit(P, b, h, i, j) for j in js]
            mn = max(m[i], max(x for x, _ in sv))
            alpha = 0.0 if m[i] == -math.inf else math.exp(m[i] - mn)
            ps = []
            for (x, r8), j in zip(sv, js):
                if r8:
                    ps.append((e4m3_torch(math.exp(e4m3_torch(x - mn))), v8[j]))
                else:
                    ps.append((math.exp(x - mn), P.v[b, kvh, j]))
            l[i] = alpha * l[i] + sum(p for p, _ in ps)
            for d in range(D):
                acc[i][d] = alpha * acc[i][d] + sum(p * vv[d] for p, vv in ps)
            m[i] = mn
    return np.array([[acc[i][d] / l[i] for d in range(D)] for i in range(S)])


@pytest.mark.parametrize("code,causal", [("i8", True), ("e4m3", False)])
def test_brute_force(code, causal):
    P = tiny_problem(seed=21, code=code, causal=causal, S=16, D=8, tm=4, tn=4, f16=0.4,
                     exp8=True, pv8=True)
    for h in range(P.Hq):
        assert np.abs(lamp_O(P, h) - brute_lamp_pv8(P, 0, h)).max() < 1e-12
