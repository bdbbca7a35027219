"""Seeded input generators (torch CPU RNG).

Recipe: torch.Generator('cpu').manual_seed(seed); fp32 standard normal draws
in the order Q [B,Hq,S,D], K [B,Hkv,S,D], V [B,Hkv,S,D]; cast to the 16-bit
dtype with round-to-nearest-even.

Outlier recipe (adaptive workload): after Q, K, V, draw 4 distinct channels
and a sign per channel from the same generator; Q's outlier channels become
20 * sign * |Q|, K's become 20 * K, and key 0 of every (batch, KV head) gets
40 * sign on the outlier channels (an attention sink every query sees).  The
scaling happens in fp32 before the cast.

Input scale (optional): Q and K are multiplied by a constant in fp32 after
the outlier step and before the cast, for cases with large logits.
"""
import torch

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def make_inputs(cfg, seed=None, S=None):
    """(q, k, v) CPU tensors of cfg's 16-bit dtype.  ``S`` overrides the
    sequence length (smaller parity cases of the same recipe)."""
    seed = cfg.input_seed if seed is None else seed
    S = cfg.S if S is None else S
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(cfg.B, cfg.Hq, S, cfg.D, generator=g, dtype=torch.float32)
    k = torch.randn(cfg.B, cfg.Hkv, S, cfg.D, generator=g, dtype=torch.float32)
    v = torch.randn(cfg.B, cfg.Hkv, S, cfg.D, generator=g, dtype=torch.float32)
    if cfg.outliers:
        ch = torch.randperm(cfg.D, generator=g)[:4]
        sign = torch.randint(0, 2, (4,), generator=g).float() * 2 - 1
        q[..., ch] = 20.0 * sign * q[..., ch].abs()
        k[..., ch] = 20.0 * k[..., ch]
        k[:, :, 0, ch] = 40.0 * sign
    if cfg.input_scale != 1.0:
        q = q * cfg.input_scale
        k = k * cfg.input_scale
    dt = _DT[cfg.dtype]
    return q.to(dt), k.to(dt), v.to(dt)
