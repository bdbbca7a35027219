"""CPU emulation of the int8 mask path's fp32 weight arithmetic.

The attention kernel's int8 tiles under mask routing with full-precision
exponentials keep each integer accumulator as the float 1.5 * 2^23 + acc and
take the weight as exp2(x * c - (m + 1.5 * 2^23 * c)) with a lazily moved
reference m (base-2 units).  This emulates that arithmetic in numpy float32
(one query tile of one head, key tiles of 64 in ascending order, weights
rounded to 16 bits for P V and the row sum) and compares O with the oracle's
exact softmax ("TileMix", section 2 "The Dual-Path Engine": INT8 products
rescaled with per-block scale factors, one shared online softmax).

* ``exact_fold``: the scale c rounded to 21 significant bits, the reference
  an integer, and m + 1.5 * 2^23 * c checked exact (TwoSum) before it is
  used, the offset subtracted from x first when it is not.  One fp32 rounding
  per exponent.
* ``rounded_fold``: m + 1.5 * 2^23 * c rounded in fp32 (two roundings whose
  error, up to about 1.5 accumulator units of logit, differs per key tile).

On inputs with outlier channels the rounded fold exceeds the output
tolerance while the exact fold stays well inside it.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import compare
from synthetic import Config, make_inputs

K0 = np.float32(12582912.0)          # 1.5 * 2^23
LOG2E = np.float32(1.4426950408889634)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def round_sig21(c):
    b = np.asarray(c, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(4)) & np.uint32(0xFFFFFFF8)).view(np.float32)


def fma32(a, b, c):
    """fp32 fma emulated in fp64 (exact product of two fp32 values, one
    fp64 rounding of the sum, then fp32)."""
    return f32(np.float64(a) * np.float64(b) + np.float64(c))


def bf16(x):
    b = f32(x).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def f16r(x):
    return f32(x).astype(np.float16).astype(np.float32)


def two_sum_err(a, b):
    a, b = f32(a), f32(b)
    s = f32(a + b)
    bb = f32(s - a)
    return f32(f32(a - f32(s - bb)) + f32(b - bb))


def emulate_int8_lazy(P, b, h, rows, mode, dtype="bf16"):
    """O of the given rows (all in one query tile) computed the kernel's way
    on tiles routed 8-bit; 16-bit tiles use fp32 logits sm*log2e*q.k."""
    R = len(rows)
    qt = rows[0] // P.tile_m
    sQ = f32(P.q_scales[b, h][qt])
    sm = f32(P.sm_scale)
    r8t = P.route8_tiles(b, h)[qt]
    vh = P.v[b, P.kvh(h)]
    m = np.full(R, -np.inf, dtype=np.float32)
    l = np.zeros(R, dtype=np.float32)
    O = np.zeros((R, P.D))
    waves = rows // 32
    for kt in range(P.n_kt):
        cols = np.arange(kt * P.tile_n, min(P.S_k, (kt + 1) * P.tile_n))
        ok = P.valid(rows, cols, b)
        if not ok.any():
            continue
        if r8t[kt]:
            acc = A.int_acc_exact(P, b, h, rows, cols)
            x = f32(K0 + acc.astype(np.float64))          # exact
            sK = f32(P.k_scales[b, P.kvh(h)][kt])
            c = f32(f32(f32(sQ * sK) * sm) * LOG2E)
            if mode == "exact_fold":
                c = round_sig21(c)
            xo = K0
        else:
            x = f32(P.q[b, h][rows] @ P.k[b, P.kvh(h)][cols].T)   # fp32 rounding of the dot
            c = f32(sm * LOG2E)
            xo = np.float32(0.0)
        lg = np.where(ok, f32(f32(x - xo) * c), -np.inf).astype(np.float32)
        mx = lg.max(axis=1)
        # lazy reference: moved per 32-row wave when a row max grows by > 8
        m_new = m.copy()
        for wv in np.unique(waves):
            sel = waves == wv
            if (mx[sel] > m[sel] + 8).any():
                mm = np.maximum(m[sel], mx[sel])
                m_new[sel] = np.ceil(mm) if mode == "exact_fold" else mm
        mr = np.where(np.isneginf(m_new), np.float32(0), m_new).astype(np.float32)
        if mode == "exact_fold":
            t = f32(xo * c)                                   # exact by construction
            msub = f32(mr + t)
            err = two_sum_err(mr, t)
            xx = x
            for wv in np.unique(waves):
                sel = waves == wv
                if (err[sel] != 0).any():
                    xx = xx.copy()
                    xx[sel] = f32(x[sel] - xo)
                    msub = msub.copy()
                    msub[sel] = mr[sel]
            y = fma32(xx, c, -msub[:, None])
        else:
            msub = f32(mr + f32(xo * c))
            y = fma32(x, c, -msub[:, None])
        p = np.where(ok, np.exp2(np.where(ok, y, -np.inf).astype(np.float64)), 0.0)
        p16 = bf16(f32(p)) if dtype == "bf16" else f16r(p)
        alpha = np.where(np.isneginf(m), 0.0, np.exp2((m - m_new).astype(np.float64)))
        alpha = np.where(m_new == m, 1.0, alpha)
        l = f32(alpha * l + p16.astype(np.float64).sum(axis=1))
        O = alpha[:, None] * O + p16.astype(np.float64) @ vh[cols]
        m = m_new
    return O / l[:, None].astype(np.float64)


def outlier_problem(D, dtype, f16, scale, S=2048):
    cfg = Config(f"emul_d{D}", B=1, Hq=1, Hkv=1, S=S, D=D, causal=True, dtype=dtype,
                 tile_m=128, tile_n=64, tiles_per_bit=4, frac_16bit=f16, code="i8", exp8=False,
                 outliers=True, input_scale=scale, input_seed=31, mask_seed=32)
    q, k, v = make_inputs(cfg)
    P = A.make_problem(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                       causal=True, code="i8", tile_m=128, tile_n=64, tiles_per_bit=4,
                       frac_16bit=f16, seed=cfg.mask_seed)
    return cfg, P


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (128, "f16"), (256, "bf16"), (256, "f16")])
def test_exact_fold_within_tolerance_rounded_fold_not(D, dtype):
    cfg, P = outlier_problem(D, dtype, 0.0, 1.0)
    rows = np.arange(cfg.S - 128, cfg.S)              # last (longest) query tile
    O_ref, _ = A.attn_tilemix(P, 0, 0, rows)
    with np.errstate(over="ignore"):
        e_new = np.abs(emulate_int8_lazy(P, 0, 0, rows, "exact_fold", dtype) - O_ref)
        e_old = np.abs(emulate_int8_lazy(P, 0, 0, rows, "rounded_fold", dtype) - O_ref)
    tol = compare.tolerance(O_ref, dtype)
    assert (e_new <= 0.75 * tol).all(), e_new.max()
    assert (e_old > tol).any(), e_old.max()
