"""Pins for oracle.attention.

* brute-force scalar loops on tiny inputs (TileMix and Lamp, with e4m3
  rounding taken from torch's float8_e4m3fn cast rather than oracle.e4m3);
* special cases that reduce to torch's scaled_dot_product_attention in fp64:
  all-16-bit mask, all-8-bit mask on dequantised Q/K, adaptive with every
  sub-block flagged;
* the online-softmax identity (tile-by-tile emulation with nothing rounded
  equals the direct softmax);
* invariants: rows of P sum to 1, V = 1 gives O = 1, V = I exposes P,
  LSE = logsumexp of the routed logits;
* the 8-bit exponential table and its distance from rounding boundaries.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import e4m3, mask as omask, quant


def rand16(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(dtype).double().numpy()


def tiny_problem(seed=0, B=1, Hq=2, Hkv=1, S=16, D=8, tm=4, tn=4, G=1, f16=0.5,
                 code="i8", causal=True, **kw):
    q = rand16((B, Hq, S, D), seed)
    k = rand16((B, Hkv, S, D), seed + 1)
    v = rand16((B, Hkv, S, D), seed + 2)
    return A.make_problem(q, k, v, causal=causal, code=code, tile_m=tm, tile_n=tn,
                          tiles_per_bit=G, frac_16bit=f16, seed=seed + 100, **kw)


def e4m3_torch(x):
    """E4M3 RNE with saturation via torch's cast (clamped first)."""
    x = max(-448.0, min(448.0, x))
    t = torch.tensor([x], dtype=torch.float64).to(torch.float8_e4m3fn)
    return float(t.to(torch.float64)[0])


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def brute_logit(P, b, h, i, j):
    kvh = P.kvh(h)
    qt, kt = i // P.tile_m, j // P.tile_n
    route8 = P.bits[b, h, qt, kt // P.tiles_per_bit] == 1
    if route8:
        acc = sum(P.qv[b, h, i, d] * P.kv[b, kvh, j, d] for d in range(P.D))
        return acc * float(P.q_scales[b, h, qt]) * float(P.k_scales[b, kvh, kt]) * P.sm_scale, True
    return P.sm_scale * sum(P.q[b, h, i, d] * P.k[b, kvh, j, d] for d in range(P.D)), False


def brute_tilemix(P):
    O = np.zeros(P.q.shape)
    for b in range(P.B):
        for h in range(P.Hq):
            for i in range(P.S_q):
                js = [j for j in range(P.S_k) if (not P.causal or j <= i)]
                s = [brute_logit(P, b, h, i, j)[0] for j in js]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                l = sum(p)
                for d in range(P.D):
                    O[b, h, i, d] = sum(pj * P.v[b, P.kvh(h), j, d] for pj, j in zip(p, js)) / l
    return O


def brute_lamp(P, b, h):
    """Scalar emulation of the tile loop for every row of head (b, h)."""
    S, D, tn, sr = P.S_q, P.D, P.tile_n, P.sub_rows
    m = [-math.inf] * S
    l = [0.0] * S
    acc = [[0.0] * D for _ in range(S)]
    flags = {}
    for kt in range(P.n_kt):
        cols = range(kt * tn, min(P.S_k, (kt + 1) * tn))
        valid = {i: [j for j in cols if (not P.causal or j <= i)] for i in range(S)}
        s8 = {(i, j): brute_logit(P, b, h, i, j) for i in range(S) for j in valid[i]}
        use16 = {}
        for sb in range(-(-S // sr)):
            rows = range(sb * sr, min(S, (sb + 1) * sr))
            flagged = False
            if P.adaptive:
                for i in rows:
                    e8 = [s8[i, j][0] for j in valid[i] if s8[i, j][1]]
                    if e8:
                        mp = max(m[i], max(e8))
                        if max(e8) - mp >= -P.tau:
                            flagged = True
                flags[sb, kt] = flagged
            for i in rows:
                use16[i] = flagged
        for i in range(S):
            if not valid[i]:
                continue
            svals = []
            for j in valid[i]:
                sv, r8 = s8[i, j]
                if (not r8) or use16[i]:
                    svals.append((sum(P.q[b, h, i, d] * P.k[b, P.kvh(h), j, d] for d in range(D))
                                  * P.sm_scale, True, j))
                else:
                    svals.append((sv, False, j))
            mn = max(m[i], max(x for x, _, _ in svals))
            alpha = 0.0 if m[i] == -math.inf else math.exp(m[i] - mn)
            ps = []
            for x, is16, j in svals:
                if is16 or not P.exp8:
                    ps.append((math.exp(x - mn), j))
                else:
                    ps.append((e4m3_torch(math.exp(e4m3_torch(x - mn))), j))
            l[i] = alpha * l[i] + sum(p for p, _ in ps)
            for d in range(D):
                acc[i][d] = alpha * acc[i][d] + sum(p * P.v[b, P.kvh(h), j, d] for p, j in ps)
            m[i] = mn
    O = np.array([[acc[i][d] / l[i] for d in range(D)] for i in range(S)])
    return O, flags


@pytest.mark.parametrize("code", ["i8", "e4m3"])
@pytest.mark.parametrize("causal", [True, False])
def test_tilemix_brute_force(code, causal):
    P = tiny_problem(seed=3, code=code, causal=causal, Hq=2, Hkv=1, S=14, G=2)
    O = np.stack([np.stack([A.attn_tilemix(P, b, h, np.arange(P.S_q))[0]
                            for h in range(P.Hq)]) for b in range(P.B)])
    assert np.abs(O - brute_tilemix(P)).max() < 1e-12


@pytest.mark.parametrize("adaptive,exp8,tau", [
    (False, True, 4.0), (True, True, 2.0), (True, False, 1.0), (True, True, 0.5)])
def test_lamp_brute_force(adaptive, exp8, tau):
    P = tiny_problem(seed=11, code="e4m3", S=16, D=8, tm=4, tn=4, f16=0.3,
                     adaptive=adaptive, exp8=exp8, tau=tau, sub_rows=2)
    for h in range(P.Hq):
        res, rows, usb = A.attn_lamp(P, 0, h, np.arange(P.S_q // P.sub_rows))
        O_b, flags_b = brute_lamp(P, 0, h)
        assert np.abs(res.O - O_b).max() < 1e-12
        if adaptive:
            for (sb, kt), f in flags_b.items():
                assert res.flags[sb, kt] == f


# ---------------------------------------------------------------------------
# special cases against SDPA
# ---------------------------------------------------------------------------

def sdpa(q, k, v, causal, sm):
    rep = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(rep, dim=1)
    return F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=causal,
                                          scale=sm).numpy()


def full_tilemix(P):
    return np.stack([np.stack([A.attn_tilemix(P, b, h, np.arange(P.S_q))[0]
                               for h in range(P.Hq)]) for b in range(P.B)])


@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_all_16bit_is_sdpa(code):
    P = tiny_problem(seed=5, B=2, Hq=4, Hkv=2, S=200, D=32, tm=64, tn=32, f16=1.0, code=code)
    assert (P.bits == 0).all()
    assert np.abs(full_tilemix(P) - sdpa(P.q, P.k, P.v, True, P.sm_scale)).max() < 1e-12


@pytest.mark.parametrize("code,tm,tn", [("i8", 64, 32), ("e4m3", 128, 64), ("i8", 32, 64)])
def test_all_8bit_is_sdpa_on_dequantised(code, tm, tn):
    P = tiny_problem(seed=6, B=1, Hq=4, Hkv=2, S=260, D=32, tm=tm, tn=tn, f16=0.0, code=code)
    assert (P.bits[..., :P.n_g] == 1).all()
    qh = quant.dequantize(P.q_codes, P.q_scales, tm, code)
    kh = quant.dequantize(P.k_codes, P.k_scales, tn, code)
    assert np.abs(full_tilemix(P) - sdpa(qh, kh, P.v, True, P.sm_scale)).max() < 1e-12


def test_adaptive_all_flagged_is_16bit_sdpa():
    P = tiny_problem(seed=8, Hq=2, Hkv=1, S=96, D=16, tm=32, tn=16, f16=0.0, code="e4m3",
                     adaptive=True, exp8=True, tau=np.inf, sub_rows=16)
    ref = sdpa(P.q, P.k, P.v, True, P.sm_scale)
    for h in range(P.Hq):
        res, rows, _ = A.attn_lamp(P, 0, h, np.arange(6))
        # sub-block sb (rows 16sb..16sb+15) sees key tiles 0..sb; tiles above
        # the causal diagonal are never processed
        assert (res.flags == np.tril(np.ones((6, 6), bool))).all()
        assert np.abs(res.O - ref[0, h]).max() < 1e-12


@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_online_identity_nothing_flagged(code):
    # adaptive with tau = -inf flags nothing; without 8-bit exp the tile loop
    # must reproduce the direct softmax on the same routes.
    for adaptive in (False, True):
        P = tiny_problem(seed=9, Hq=2, Hkv=2, S=300, D=32, tm=64, tn=32, f16=0.4, code=code,
                         adaptive=adaptive, exp8=False, tau=-np.inf, sub_rows=32)
        for h in range(P.Hq):
            res, rows, _ = A.attn_lamp(P, 0, h, np.arange(-(-300 // 32)))
            O, lse = A.attn_tilemix(P, 0, h, rows)
            assert not res.flags.any()
            assert np.abs(res.O - O).max() < 1e-12
            assert np.abs(res.lse - lse).max() < 1e-11


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_probabilities_sum_to_one_and_lse():
    P = tiny_problem(seed=12, Hq=2, Hkv=1, S=150, D=16, tm=32, tn=16, G=2, f16=0.5)
    rows = np.arange(P.S_q)
    for h in range(P.Hq):
        s, _, ok = A.routed_logits(P, 0, h, rows)
        s = np.where(ok, s, -np.inf)
        p = torch.softmax(torch.from_numpy(s), dim=1).numpy()
        assert np.abs(p.sum(1) - 1).max() < 1e-12
        _, lse = A.attn_tilemix(P, 0, h, rows)
        assert np.abs(lse - torch.logsumexp(torch.from_numpy(s), 1).numpy()).max() < 1e-11


def test_v_identity_exposes_p():
    P = tiny_problem(seed=13, Hq=1, Hkv=1, S=32, D=32, tm=16, tn=16, f16=0.5)
    P.v = np.eye(32)[None, None]
    s, _, ok = A.routed_logits(P, 0, 0, np.arange(32))
    p = torch.softmax(torch.from_numpy(np.where(ok, s, -np.inf)), 1).numpy()
    O, _ = A.attn_tilemix(P, 0, 0, np.arange(32))
    assert np.abs(O - p).max() < 1e-13


@pytest.mark.parametrize("exp8,adaptive", [(True, False), (True, True), (False, False)])
def test_v_ones_gives_ones(exp8, adaptive):
    P = tiny_problem(seed=14, Hq=2, Hkv=1, S=130, D=16, tm=32, tn=16, f16=0.5, code="e4m3",
                     exp8=exp8, adaptive=adaptive, sub_rows=16)
    P.v = np.ones_like(P.v)
    for h in range(P.Hq):
        res, _, _ = A.attn_lamp(P, 0, h, np.arange(-(-130 // 16)))
        assert np.abs(res.O - 1).max() < 1e-13
        O, _ = A.attn_tilemix(P, 0, h, np.arange(130))
        assert np.abs(O - 1).max() < 1e-13


def test_int_accumulator_exact():
    P = tiny_problem(seed=15, Hq=2, Hkv=1, S=256, D=128, tm=128, tn=64, code="i8")
    rows, cols = np.arange(256), np.arange(256)
    ia = A.int_acc_exact(P, 0, 1, rows, cols)
    assert (ia.astype(np.float64) == A.acc8(P, 0, 1, rows, cols)).all()
    assert np.abs(ia).max() < 2 ** 31


def test_e4m3_products_exact_in_fp64():
    # the e4m3 dot product is computed exactly: compare with exact rationals
    from fractions import Fraction
    P = tiny_problem(seed=16, Hq=1, Hkv=1, S=4, D=256, tm=4, tn=4, code="e4m3")
    a = A.acc8(P, 0, 0, np.arange(4), np.arange(4))
    for i in range(4):
        for j in range(4):
            ex = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(P.qv[0, 0, i], P.kv[0, 0, j]))
            assert Fraction(float(a[i, j])) == ex


# ---------------------------------------------------------------------------
# Lamp flags and the 8-bit exponential
# ---------------------------------------------------------------------------

def test_flags_first_tile_and_monotone_in_tau():
    prev = None
    for tau in (0.0, 0.5, 2.0, 4.0, 8.0):
        P = tiny_problem(seed=17, Hq=1, Hkv=1, S=256, D=32, tm=64, tn=32, f16=0.0,
                         code="e4m3", adaptive=True, exp8=True, tau=tau, sub_rows=32)
        res, rows, usb = A.attn_lamp(P, 0, 0, np.arange(8))
        # tile 0 is every row's first processed tile
        assert res.flags[:, 0].all()
        if prev is not None:
            assert (res.flags | ~prev).all() or res.flag_dontcare.any()
        prev = res.flags


def test_flag_rowmax_form():
    # with sub-block width = one key tile, flagged iff some row has
    # rowmax8 >= m - tau (m = running max before the tile)
    P = tiny_problem(seed=18, Hq=1, Hkv=1, S=128, D=32, tm=32, tn=16, f16=0.0, code="i8",
                     adaptive=True, exp8=False, tau=1.5, sub_rows=16)
    res, rows, usb = A.attn_lamp(P, 0, 0, np.arange(8))
    for sb in range(8):
        rr = np.arange(sb * 16, sb * 16 + 16)
        m = np.full(16, -np.inf)
        for kt in range(P.n_kt):
            cols = np.arange(kt * 16, kt * 16 + 16)
            ok = P.valid(rr, cols)
            if not ok.any():
                continue
            s8 = np.where(ok, A.logits8(P, 0, 0, rr, cols), -np.inf)
            rm = s8.max(1)
            want = bool(((rm >= m - 1.5) & ok.any(1)).any())
            assert res.flags[sb, kt] == want
            s16 = np.where(ok, A.logits16(P, 0, 0, rr, cols), -np.inf)
            m = np.maximum(m, (s16 if want else s8).max(1))


def test_exp8_table_margins():
    # the 128 codes of non-positive logits: +0 and 0x80..0xFE
    codes = np.array([0x00] + list(range(0x80, 0xFF)), np.uint8)
    x = e4m3.decode(codes)
    ex = np.exp(x)
    p = A.exp8_of_code(codes)
    assert p[0] == 1.0 and p[1] == 1.0               # +0 and -0
    assert int((p > 0).sum()) == 79
    # every exp(x) lies far from an e4m3 rounding boundary (relative distance
    # well above fp32 exp error), so an fp32 exp reproduces this table
    b = e4m3.rounding_boundaries()
    nz = ex >= b[0] * 0.5
    rel = np.min(np.abs(ex[nz, None] - b[None, :]) / ex[nz, None], axis=1)
    assert rel.min() > 1e-4
    # torch's cast agrees on the table
    for xi, pi in zip(x, p):
        assert e4m3_torch(math.exp(xi)) == pi


def test_route_counts():
    P = tiny_problem(seed=19, B=2, Hq=3, Hkv=1, S=300, D=8, tm=64, tn=32, G=2, f16=0.3)
    c = A.route_counts(P)
    n8 = n16 = 0
    for b in range(2):
        for h in range(3):
            for i in range(300):
                for j in range(i + 1):
                    if P.bits[b, h, i // 64, (j // 32) // 2]:
                        n8 += 1
                    else:
                        n16 += 1
    assert c == dict(n8=n8, n16=n16, nvalid=n8 + n16)


def test_quadratic_arithmetic_claim():
    # TileMix page, section 1: a 32,000-token document has about 1e9 score
    # interactions
    assert 32_000 * 32_000 >= 1.0e9


# ---------------------------------------------------------------------------
# causal with fewer queries than keys: the queries are the last S_q positions
# ---------------------------------------------------------------------------

def sdpa_bottom_right(q, k, v, sm):
    """fp64 SDPA with an explicit mask: query i sees keys j <= i + S_k - S_q."""
    S_q, S_k = q.shape[2], k.shape[2]
    rep = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(rep, dim=1)
    keep = torch.arange(S_k)[None, :] <= torch.arange(S_q)[:, None] + (S_k - S_q)
    return F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=keep,
                                          scale=sm).numpy()


def chunk_problem(seed, S_q, S_k, f16, code="i8", **kw):
    q = rand16((1, 2, S_q, 16), seed)
    k = rand16((1, 1, S_k, 16), seed + 1)
    v = rand16((1, 1, S_k, 16), seed + 2)
    return A.make_problem(q, k, v, causal=True, code=code, tile_m=32, tile_n=16,
                          tiles_per_bit=1, frac_16bit=f16, seed=seed + 100, **kw)


@pytest.mark.parametrize("S_q,S_k", [(40, 100), (1, 77), (64, 64)])
def test_causal_chunk_all_16bit_is_sdpa(S_q, S_k):
    P = chunk_problem(21, S_q, S_k, 1.0)
    assert np.abs(full_tilemix(P) - sdpa_bottom_right(P.q, P.k, P.v, P.sm_scale)).max() < 1e-12


def test_causal_chunk_is_suffix_of_full_prefill():
    # the last S_q rows of a causal prefill over S_k tokens, computed as a
    # chunk (same keys, same per-row routes), equal the full prefill's rows
    S_k, S_q = 96, 40
    q = rand16((1, 2, S_k, 16), 31)
    k = rand16((1, 1, S_k, 16), 32)
    v = rand16((1, 1, S_k, 16), 33)
    full = A.make_problem(q, k, v, causal=True, code="i8", tile_m=8, tile_n=16,
                          tiles_per_bit=1, frac_16bit=1.0, seed=1)
    chunk = A.make_problem(q[:, :, S_k - S_q:].copy(), k, v, causal=True, code="i8", tile_m=8,
                           tile_n=16, tiles_per_bit=1, frac_16bit=1.0, seed=1)
    for h in range(2):
        of = A.attn_tilemix(full, 0, h, np.arange(S_k - S_q, S_k))[0]
        oc = A.attn_tilemix(chunk, 0, h, np.arange(S_q))[0]
        assert np.abs(of - oc).max() < 1e-12


def test_causal_chunk_brute_force():
    P = chunk_problem(41, 10, 23, 0.5)
    O = np.zeros(P.q.shape)
    off = P.S_k - P.S_q
    for h in range(P.Hq):
        for i in range(P.S_q):
            js = [j for j in range(P.S_k) if j <= i + off]
            s = [brute_logit(P, 0, h, i, j)[0] for j in js]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = sum(p)
            for d in range(P.D):
                O[0, h, i, d] = sum(pj * P.v[0, P.kvh(h), j, d] for pj, j in zip(p, js)) / l
    assert np.abs(full_tilemix(P) - O).max() < 1e-12


def test_causal_more_queries_than_keys_rejected():
    with pytest.raises(ValueError):
        chunk_problem(1, 50, 40, 0.5)


# ---------------------------------------------------------------------------
# variable-length batches: each sequence equals its own dense problem
# ---------------------------------------------------------------------------

def varlen_problem(seed, S_q, S_k, Lq, Lk, causal, f16, code="i8", **kw):
    B = len(Lq)
    q = rand16((B, 2, S_q, 16), seed)
    k = rand16((B, 1, S_k, 16), seed + 1)
    v = rand16((B, 1, S_k, 16), seed + 2)
    return A.make_problem(q, k, v, causal=causal, code=code, tile_m=32, tile_n=16,
                          tiles_per_bit=2, frac_16bit=f16, seed=seed + 100,
                          seqlens_q=np.array(Lq), seqlens_k=np.array(Lk), **kw)


def dense_slice(P, b, **kw):
    """Sequence b of a variable-length problem as a dense problem of its own
    lengths, with the same mask rows."""
    lq, lk = int(P.Lq[b]), int(P.Lk[b])
    n_qt = -(-lq // P.tile_m)
    return A.make_problem(P.q[b:b + 1, :, :lq], P.k[b:b + 1, :, :lk], P.v[b:b + 1, :, :lk],
                          causal=P.causal, code=P.code, tile_m=P.tile_m, tile_n=P.tile_n,
                          tiles_per_bit=P.tiles_per_bit, frac_16bit=0.0, seed=0,
                          mask_words=P.mask_words[b:b + 1, :, :n_qt], sm_scale=P.sm_scale, **kw)


@pytest.mark.parametrize("causal,Lq,Lk", [
    (True, [70, 1, 100, 33], [100, 9, 100, 64]),
    (False, [50, 100, 17], [3, 120, 120]),
])
@pytest.mark.parametrize("code", ["i8", "e4m3"])
def test_varlen_equals_dense_sequences(causal, Lq, Lk, code):
    P = varlen_problem(51, 100, 120, Lq, Lk, causal, 0.4, code)
    for b in range(P.B):
        lq = int(P.Lq[b])
        D = dense_slice(P, b)
        # quantiser: codes of valid rows and the scales of their blocks agree;
        # padding rows are code 0
        assert (P.q_codes[b, :, :lq] == D.q_codes[0]).all()
        assert (P.q_codes[b, :, lq:] == 0).all()
        nq = -(-lq // P.tile_m)
        assert (P.q_scales[b, :, :nq] == D.q_scales[0]).all()
        assert (P.q_scales[b, :, nq:] == 0).all()
        lk = int(P.Lk[b])
        assert (P.k_codes[b, :, :lk] == D.k_codes[0]).all() and (P.k_codes[b, :, lk:] == 0).all()
        for h in range(P.Hq):
            o1, l1 = A.attn_tilemix(P, b, h, np.arange(lq))
            o2, l2 = A.attn_tilemix(D, 0, h, np.arange(lq))
            assert np.abs(o1 - o2).max(initial=0) < 1e-12
            assert (np.isneginf(l1) == np.isneginf(l2)).all()
            fin = np.isfinite(l2)
            assert np.abs(l1[fin] - l2[fin]).max(initial=0) < 1e-12


def test_varlen_lamp_equals_dense_sequences():
    P = varlen_problem(61, 96, 96, [96, 40, 7], [96, 80, 50], True, 0.0, "e4m3",
                       adaptive=True, exp8=True, tau=2.0, sub_rows=16)
    for b in range(P.B):
        lq = int(P.Lq[b])
        D = dense_slice(P, b, adaptive=True, exp8=True, tau=2.0, sub_rows=16)
        nsb = -(-lq // 16)
        for h in range(P.Hq):
            r1, rows1, _ = A.attn_lamp(P, b, h, np.arange(nsb))
            r2, rows2, _ = A.attn_lamp(D, 0, h, np.arange(nsb))
            keep = rows1 < lq
            assert (rows1[keep] == rows2).all()
            assert np.abs(r1.O[keep] - r2.O).max() < 1e-12
            nk = r2.flags.shape[1]
            assert (r1.flags[:, :nk] == r2.flags).all() and not r1.flags[:, nk:].any()


def test_varlen_full_lengths_equal_dense():
    P = varlen_problem(71, 64, 64, [64, 64], [64, 64], True, 0.5)
    Q = A.make_problem(P.q, P.k, P.v, causal=True, code="i8", tile_m=32, tile_n=16,
                       tiles_per_bit=2, frac_16bit=0.5, seed=171)
    assert (P.q_codes == Q.q_codes).all() and (P.mask_words == Q.mask_words).all()
    for b in range(2):
        for h in range(2):
            assert np.abs(A.attn_tilemix(P, b, h, np.arange(64))[0] -
                          A.attn_tilemix(Q, b, h, np.arange(64))[0]).max() == 0


def test_varlen_rows_without_keys():
    P = varlen_problem(81, 40, 40, [40, 20], [0, 20], False, 0.5)
    O, lse = A.attn_tilemix(P, 0, 0, np.arange(40))
    assert (O == 0).all() and np.isneginf(lse).all()
    with pytest.raises(ValueError):
        varlen_problem(1, 40, 40, [30], [20], True, 0.5)        # causal needs Lq <= Lk
    with pytest.raises(ValueError):
        varlen_problem(1, 40, 40, [41], [40], False, 0.5)       # beyond the padded length
