"""Helpers for the GPU parity tests: run the HIP pipeline through the C ABI
binding and build the oracle's view of the same seeded inputs."""
import json
import os

import numpy as np
import torch

# LampAttention acceptance counts over the session (printed at the end of the
# run by conftest.py): sub-blocks checked, flag decisions within the error
# bound (evaluated both ways), sub-blocks whose GPU flags picked a non-primary
# branch, flag mismatches, branch-cap overflows, rows excluded (always 0) and
# the largest widening for e4m3 rounding flips.
LAMP_REPORT = {}


def record_lamp(st):
    path = os.environ.get("LAMP_REPORT_FILE")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                                **{k: v for k, v in st.items()}}) + "\n")
    for k in ("n_subblocks", "n_split", "n_branches", "n_nonprimary", "flag_mismatch",
              "unresolved", "excluded_rows", "lse_bad", "n_bad", "n_elems", "n_wide"):
        LAMP_REPORT[k] = LAMP_REPORT.get(k, 0) + int(st.get(k, 0))
    test = _current_test()
    for k in ("max_extra", "max_err"):
        v = float(st.get(k, 0.0))
        if v >= LAMP_REPORT.get(k, 0.0):
            LAMP_REPORT[k] = v
            LAMP_REPORT[k + "_test"] = test


def _current_test():
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0].split("::")[-1]


# Acceptance of the paths checked element by element against one oracle
# output (TileMix: the mask paths with fp32 exponentials; decode): elements
# compared, the largest error, how many exceed atol (accepted through one
# ulp of the output dtype or the widening for the exponents' error bounds),
# the largest widening, and the largest LSE deviation relative to its bound.
PATH_REPORT = {}


def record_path(path, st, O_gpu, O_ref, dtype, extra=None, lse_dev=None, lse_tol=None):
    from oracle import compare
    r = PATH_REPORT.setdefault(path, {})
    err = np.abs(np.asarray(O_gpu, dtype=np.float64) - np.asarray(O_ref, dtype=np.float64))
    r["n_elems"] = r.get("n_elems", 0) + int(err.size)
    r["n_over_atol"] = r.get("n_over_atol", 0) + int((err > compare.ATOL[dtype]).sum())
    test = _current_test()
    if err.size and float(err.max()) >= r.get("max_err", 0.0):
        r["max_err"], r["max_err_test"] = float(err.max()), test
    if extra is not None:
        e = np.broadcast_to(np.asarray(extra, dtype=np.float64), err.shape) if np.ndim(extra) == err.ndim \
            else np.broadcast_to(np.asarray(extra, dtype=np.float64)[..., None], err.shape)
        r["n_wide"] = r.get("n_wide", 0) + int((e > compare.ATOL[dtype]).sum())
        if e.size and float(e.max()) >= r.get("max_extra", 0.0):
            r["max_extra"], r["max_extra_test"] = float(e.max()), test
    if lse_dev is not None and np.size(lse_dev):
        ratio = float(np.max(np.asarray(lse_dev) / np.maximum(np.asarray(lse_tol), 1e-300)))
        r["max_lse_dev"] = max(r.get("max_lse_dev", 0.0), float(np.max(lse_dev)))
        r["max_lse_ratio"] = max(r.get("max_lse_ratio", 0.0), ratio)

from oracle import attention as A
from oracle import mask as omask


def device():
    return torch.device("cuda:0")


def u64(t):
    return t.cpu().numpy().view(np.uint64)


def gpu_run(cfg, q, k, v, *, lse=True, flags=None, dbg=False, mask_words=None, pv8=False):
    """Quantise, build the mask (unless given) and run attention on the GPU
    (pv8: V tiles quantised too, 8-bit P V on 8-bit tiles)."""
    import mixed_precision_tiled_amd as L
    dev = device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    S_q, S_k = q.shape[2], k.shape[2]
    q8, sq = L.lamp_quantize_blocks(qd, cfg.tile_m, cfg.code)
    k8, sk = L.lamp_quantize_blocks(kd, cfg.tile_n, cfg.code)
    n_g = -(-(-(-S_k // cfg.tile_n)) // cfg.tiles_per_bit)
    W = max(1, -(-n_g // 64))
    if mask_words is not None:
        mask = torch.from_numpy(np.ascontiguousarray(mask_words).view(np.int64)).to(dev)
    elif cfg.mask_all_ones:
        mask = L.lamp_build_mask(cfg.B, cfg.Hq, S_q, S_k, cfg.tile_m, cfg.tile_n,
                                 cfg.tiles_per_bit, 0.0, cfg.mask_seed, W, device=dev)
    else:
        mask = L.lamp_build_mask(cfg.B, cfg.Hq, S_q, S_k, cfg.tile_m, cfg.tile_n,
                                 cfg.tiles_per_bit, cfg.frac_16bit, cfg.mask_seed, W, device=dev)
    lse_t = torch.full((cfg.B, cfg.Hq, S_q), float("nan"), device=dev) if lse else None
    flags_t = None
    if cfg.adaptive and flags is not False:
        flags_t = torch.full(L.lamp.flags_shape(cfg.B, cfg.Hq, S_q, S_k), -1, dtype=torch.int64,
                             device=dev)
    dbg_t = None
    if dbg:
        dbg_t = torch.full((cfg.B, cfg.Hq, S_q, S_k), -(2 ** 31), dtype=torch.int32, device=dev)
    v8 = vs = None
    if pv8:
        v8, vs = L.lamp_quantize_v_tiles(vd)
    out = L.lamp_attn_fwd(qd, kd, vd, q8, k8, sq, sk, mask, code=cfg.code, causal=cfg.causal,
                          tile_m=cfg.tile_m, tiles_per_bit=cfg.tiles_per_bit,
                          mode=L.LAMP_MODE_ADAPTIVE if cfg.adaptive else L.LAMP_MODE_MASK,
                          exp8=cfg.exp8, tau=cfg.tau, sub_rows=cfg.sub_rows,
                          sm_scale=cfg.sm_scale, lse=lse_t, flags_out=flags_t, dbg_qk_acc=dbg_t,
                          v8=v8, v_scale=vs)
    torch.cuda.synchronize()
    return dict(q8=q8.cpu().numpy(), sq=sq.cpu().numpy(), k8=k8.cpu().numpy(),
                sk=sk.cpu().numpy(), mask=u64(mask), out=out.float().cpu().numpy(),
                lse=None if lse_t is None else lse_t.cpu().numpy(),
                flags=None if flags_t is None else u64(flags_t),
                dbg=None if dbg_t is None else dbg_t.cpu().numpy(),
                v8=None if v8 is None else v8.cpu().numpy(),
                vs=None if vs is None else vs.cpu().numpy())


def oracle_mask(cfg, S_q, S_k):
    n_g = -(-(-(-S_k // cfg.tile_n)) // cfg.tiles_per_bit)
    W = max(1, -(-n_g // 64))
    f16 = 0.0 if cfg.mask_all_ones else cfg.frac_16bit
    return omask.build_mask(cfg.B, cfg.Hq, S_q, S_k, cfg.tile_m, cfg.tile_n, cfg.tiles_per_bit,
                            f16, cfg.mask_seed, W)


def oracle_problem(cfg, q, k, v, b=None, h=None, mask_words=None, pv8=False):
    """Oracle Problem for all heads, or for the single query head (b, h) and
    its KV head (quantisation blocks never cross heads, so this is exact)."""
    S_q, S_k = q.shape[2], k.shape[2]
    mw = oracle_mask(cfg, S_q, S_k) if mask_words is None else mask_words
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    if b is not None:
        kvh = h // (cfg.Hq // cfg.Hkv)
        qn = qn[b:b + 1, h:h + 1]
        kn, vn = kn[b:b + 1, kvh:kvh + 1], vn[b:b + 1, kvh:kvh + 1]
        mw = mw[b:b + 1, h:h + 1]
    return A.make_problem(qn, kn, vn, causal=cfg.causal, code=cfg.code, tile_m=cfg.tile_m,
                          tile_n=cfg.tile_n, tiles_per_bit=cfg.tiles_per_bit,
                          frac_16bit=cfg.frac_16bit, seed=cfg.mask_seed, mask_words=mw,
                          sm_scale=cfg.sm_scale, adaptive=cfg.adaptive, exp8=cfg.exp8,
                          tau=cfg.tau, sub_rows=cfg.sub_rows, pv8=pv8)
