"""Attention over an 8-bit key/value cache (oracle; test infrastructure only).

Source: "TileMix: Mixed-Precision Attention for Faster LLM Prefill", section
4 "Why It Matters": the method supports INT8 key/value caches, which matter
for the decode phase (few new queries against a long cached context).

Reading taken (listed in the design notes): the cache holds K and V as int8
codes with one fp32 scale per block of 64 keys of one (b, kv head), exactly
as the per-block quantiser writes them (quant.quantize_blocks with
block_rows = 64); the queries are 16-bit and quantised by the same quantiser
in blocks of `tile_m` rows, so the logits are those of the 8-bit path,

    s_ij = (cq_i . ck_j) * sQ[i] * sK[j] * sm,

and the output uses the dequantised values,

    O_i = sum_j p_ij * sV[j] * cv_j,   p_i = softmax over valid j of s_i.

Causal attention aligns the queries with the end of the cache (query i of
S_q sits at key position i + S_k - S_q).  In fp64 the integer dot products
are exact, so this is the definition written out.
"""
import numpy as np

from . import attention as A
from . import quant


def decode_problem(q, k, v, *, causal, tile_m, sm_scale=0.0):
    """(P, v_hat): the oracle problem of a decode step over the int8 cache
    built from 16-bit K and V.  P routes every key tile to the 8-bit path and
    carries the dequantised cache values as its V."""
    v = np.asarray(v, dtype=np.float64)
    vc, vs = quant.quantize_blocks(v, 64, "i8")
    v_hat = quant.dequantize(vc, vs, 64, "i8")
    B, Hq, S_q, _ = np.asarray(q).shape
    S_k = v.shape[2]
    n_g = -(-S_k // 64)
    words = np.full((B, Hq, -(-S_q // tile_m), max(1, -(-n_g // 64))), np.uint64(2 ** 64 - 1),
                    dtype=np.uint64)
    P = A.make_problem(q, k, v_hat, causal=causal, code="i8", tile_m=tile_m, tile_n=64,
                       tiles_per_bit=1, frac_16bit=0.0, seed=0, mask_words=words,
                       sm_scale=sm_scale)
    return P, (vc, vs)


def decode_attention(P, b, h, rows):
    """O[rows, D], LSE[rows] of head (b, h): softmax of the 8-bit-path logits
    times the dequantised cache values."""
    return A.attn_tilemix(P, b, h, rows)
