"""Pins for oracle.decode (attention over an int8 key/value cache)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import decode, quant


def rand16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).double().numpy()


def test_decode_brute_force():
    # per-element loops over the codes and scales, written from the definition
    B, Hq, Hkv, S_q, S_k, D = 1, 4, 2, 3, 150, 8
    q, k, v = rand16((B, Hq, S_q, D), 1), rand16((B, Hkv, S_k, D), 2), rand16((B, Hkv, S_k, D), 3)
    P, (vc, vs) = decode.decode_problem(q, k, v, causal=True, tile_m=64)
    qc, qs = quant.quantize_blocks(q, 64, "i8")
    kc, ks = quant.quantize_blocks(k, 64, "i8")
    sm = 1.0 / math.sqrt(D)
    i8 = lambda c: int(np.uint8(c).view(np.int8))
    for h in range(Hq):
        kvh = h // 2
        O, lse = decode.decode_attention(P, 0, h, np.arange(S_q))
        for i in range(S_q):
            js = [j for j in range(S_k) if j <= i + S_k - S_q]
            s = [sum(i8(qc[0, h, i, d]) * i8(kc[0, kvh, j, d]) for d in range(D)) *
                 float(qs[0, h, 0]) * float(ks[0, kvh, j // 64]) * sm for j in js]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = sum(p)
            for d in range(D):
                ref = sum(pj * i8(vc[0, kvh, j, d]) * float(vs[0, kvh, j // 64])
                          for pj, j in zip(p, js)) / l
                assert abs(O[i, d] - ref) < 1e-12
            assert abs(lse[i] - (m + math.log(l))) < 1e-12


def test_decode_exact_cache_equals_sdpa_on_dequantised():
    # a cache whose values are exactly representable (V = code * scale) makes
    # the dequantised V equal to V itself; with K and Q likewise exact the
    # result is plain fp64 SDPA on those values
    rng = np.random.default_rng(5)
    B, Hq, Hkv, S_q, S_k, D = 2, 4, 1, 5, 200, 16
    sc = 2.0 ** -6
    # every block holds a +-127 entry so its scale is exactly sc
    def exact(shape, block):
        x = rng.integers(-127, 128, size=shape).astype(np.float64)
        x[:, :, ::block, 0] = 127.0
        return x * sc
    q, k, v = exact((B, Hq, S_q, D), 64), exact((B, Hkv, S_k, D), 64), exact((B, Hkv, S_k, D), 64)
    P, (vc, vs) = decode.decode_problem(q, k, v, causal=True, tile_m=64)
    assert (vs == np.float32(127 * sc / 127)).all()
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    keep = torch.arange(S_k)[None, :] <= torch.arange(S_q)[:, None] + (S_k - S_q)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=keep,
                                         scale=1.0 / math.sqrt(D)).numpy()
    for b in range(B):
        for h in range(Hq):
            O, _ = decode.decode_attention(P, b, h, np.arange(S_q))
            assert np.abs(O - ref[b, h]).max() < 1e-12


def test_decode_constant_values():
    # V constant along the keys: every output row equals that constant's
    # dequantised value whatever the weights
    B, Hq, Hkv, S_q, S_k, D = 1, 2, 1, 2, 130, 8
    q, k = rand16((B, Hq, S_q, D), 7), rand16((B, Hkv, S_k, D), 8)
    v = np.ones((B, Hkv, S_k, D)) * 0.75
    P, _ = decode.decode_problem(q, k, v, causal=False, tile_m=64)
    v_hat = 127.0 * float(np.float32(0.75) / np.float32(127.0))   # code 127 times the fp32 scale
    for h in range(Hq):
        O, _ = decode.decode_attention(P, 0, h, np.arange(S_q))
        assert np.abs(O - v_hat).max() < 1e-12
