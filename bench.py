#!/usr/bin/env python3
"""Benchmark of the mixed-precision tiled attention prefill hot path on one
MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: per-block quantisation of Q and K, the packed
precision mask, and the dual-path attention forward.  Default workload: the
Qwen3-8B-shaped prefill (batch 2, 32 query / 8 KV heads, head dim 128, 16k
tokens, causal, bf16) with 25% of the mask groups on the bf16 path and int8
elsewhere.

Prints ONE JSON line on stdout.  `value` is the step's algorithmic TFLOP/s
(QK^T 2d flops per valid score element on its path, plus 2d for each
adaptively recomputed element, plus P V 2d per valid element); `roofline`
describes the attention kernel alone against the mix-weighted MFMA roofline
T_roof = 2d N8 / P8 + 2d (N16 + Nflag) / P16 + 2d Nvalid / P16 with MI355X's
published dense peaks P8 = 5.0e15 (int8 / fp8) and P16 = 2.5e15 (bf16 /
fp16); `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.  `roofline.sustained` repeats the roofline against the dense MFMA
rates this GPU sustains under a full-chip matrix load (measured live by a
probe kernel, with the shader clock they ran at).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK8 = 5.0e15      # MI355X dense int8 / fp8 MFMA, ops/s
PEAK16 = 2.5e15     # MI355X dense bf16 / fp16 MFMA, flop/s
KERNEL_SOURCES = ["mixed_precision_tiled_amd/csrc/attn_kernel.h",
                  "mixed_precision_tiled_amd/csrc/lamp_device.h",
                  "mixed_precision_tiled_amd/csrc/attn_dispatch.h",
                  "mixed_precision_tiled_amd/csrc/attn_d64.hip",
                  "mixed_precision_tiled_amd/csrc/attn_d128.hip",
                  "mixed_precision_tiled_amd/csrc/attn_d256.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# valid-element counts per path (roofline input), from the mask the GPU built
# ---------------------------------------------------------------------------

def tile_valid_counts(S_q, S_k, tile_m, tile_n, causal):
    """[n_qt, n_kt] number of valid (query, key) pairs in each score tile."""
    n_qt, n_kt = -(-S_q // tile_m), -(-S_k // tile_n)
    r0 = np.arange(n_qt) * tile_m
    r1 = np.minimum(S_q, r0 + tile_m)                 # rows [r0, r1)
    c0 = np.arange(n_kt) * tile_n
    c1 = np.minimum(S_k, c0 + tile_n)                 # cols [c0, c1)
    if not causal:
        return np.outer(r1 - r0, c1 - c0).astype(np.int64)
    cnt = np.zeros((n_qt, n_kt), dtype=np.int64)
    off = S_k - S_q                   # causal: query i sees keys j <= i + off
    for a in range(n_qt):
        rows = np.arange(r0[a], r1[a])
        # valid keys per row within the tile: clip(row + off + 1, c0, c1) - c0
        cnt[a] = (np.clip(rows[:, None] + off + 1, c0[None, :], c1[None, :]) - c0[None, :]).sum(0)
    return cnt


def route_counts(mask_words, S_q, S_k, tile_m, tile_n, tiles_per_bit, causal, flags=None,
                 seqlens_q=None, seqlens_k=None):
    """dict(n8, n16, nflag, nvalid) from packed mask words [B, Hq, n_qt, W]
    (optionally a variable-length batch: per-sequence lengths [B])."""
    mw = np.asarray(mask_words, dtype=np.uint64)
    B = mw.shape[0]
    n_qt, n_kt = -(-S_q // tile_m), -(-S_k // tile_n)
    n_sb = -(-S_q // 32)
    g = np.arange(n_kt) // tiles_per_bit
    bits = ((mw[..., g // 64] >> (g % 64).astype(np.uint64)) & np.uint64(1)).astype(np.int64)
    Lq = [S_q] * B if seqlens_q is None else [int(x) for x in seqlens_q]
    Lk = [S_k] * B if seqlens_k is None else [int(x) for x in seqlens_k]

    def counts(lq, lk, rows):
        # [ceil(S_q/rows), n_kt] valid pairs per tile of a sequence of lengths lq, lk
        c = np.zeros((-(-S_q // rows), n_kt), dtype=np.int64)
        if lq > 0 and lk > 0:
            t = tile_valid_counts(lq, lk, rows, tile_n, causal)
            c[:t.shape[0], :t.shape[1]] = t
        return c

    cnt = np.stack([counts(Lq[b], Lk[b], tile_m) for b in range(B)])     # [B, n_qt, n_kt]
    n8 = int((bits * cnt[:, None]).sum())
    nvalid = int(cnt.sum()) * mw.shape[1]
    nflag = 0
    if flags is not None:
        # flags [B, Hq, n_sb, FW]: sub-block of 32 rows x key tile
        fw = np.asarray(flags, dtype=np.uint64)
        kt = np.arange(n_kt)
        fb = ((fw[..., kt // 64] >> (kt % 64).astype(np.uint64)) & np.uint64(1)).astype(np.int64)
        sub = np.stack([counts(Lq[b], Lk[b], 32) for b in range(B)])    # [B, n_sb, n_kt]
        nflag = int((fb[:, :, :n_sb] * sub[:, None]).sum())
    return dict(n8=n8, n16=nvalid - n8, nflag=nflag, nvalid=nvalid)


def algorithmic_flops(c, D):
    return 2.0 * D * (c["n8"] + c["n16"] + c["nflag"]) + 2.0 * D * c["nvalid"]


def roofline_time(c, D):
    return 2.0 * D * c["n8"] / PEAK8 + 2.0 * D * (c["n16"] + c["nflag"]) / PEAK16 + \
        2.0 * D * c["nvalid"] / PEAK16


def roofline_time_pv8(c, D):
    """Roofline with the 8-bit P V product: P V of 8-bit-routed elements at the
    8-bit rate too."""
    return 2.0 * D * c["n8"] / PEAK8 + 2.0 * D * (c["n16"] + c["nflag"]) / PEAK16 + \
        2.0 * D * c["n8"] / PEAK8 + 2.0 * D * c["n16"] / PEAK16


def roofline_time_at(c, D, p8, p16):
    return 2.0 * D * c["n8"] / p8 + 2.0 * D * (c["n16"] + c["nflag"]) / p16 + \
        2.0 * D * c["nvalid"] / p16


# ---------------------------------------------------------------------------
# sustained MFMA rates of this GPU (the published peaks assume the top engine
# clock, which a full-chip matrix load does not hold)
# ---------------------------------------------------------------------------

def sustained_mfma_peaks(torch, iters=100000, reps=3):
    """Dense bf16 and int8 MFMA rates with every SIMD's matrix pipe busy on
    pseudo-random operands, and the shader clock meanwhile, from the probe
    library built beside liblamp.so.  The int8 rate also stands for fp8 (the
    same published dense rate).  None if the probe library is missing."""
    import ctypes
    path = os.path.join(ROOT, "mixed_precision_tiled_amd", "libmfma_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mfma_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_probe_launch.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    nblk = 2 * torch.cuda.get_device_properties(0).multi_processor_count  # 2 waves per SIMD
    sink = torch.empty(nblk * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * nblk, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for kind, name, per_mfma in ((0, "bf16_fp16", 32768.0), (1, "int8_fp8", 65536.0)):
        for r in range(reps):          # the last repetition is reported
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = lib.mfma_probe_launch(kind, nblk, iters, 12345 + r, sink.data_ptr(),
                                       clk.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"mfma probe launch failed ({rc})")
        t = e0.elapsed_time(e1) * 1e-3
        ticks = clk.cpu().numpy().reshape(-1, 2).astype(np.float64)
        out[name] = {"ops_per_s": nblk * 4 * iters * 4 * per_mfma / t,
                     "clock_ghz": round(float(ticks[:, 0].sum() / ticks[:, 1].sum() * 0.1), 3)}
    return out


# ---------------------------------------------------------------------------
# decode over an int8 key/value cache (HBM-bound)
# ---------------------------------------------------------------------------

HBM_PEAK = 8.0e12    # MI355X HBM3E, bytes/s


def decode_measurement(torch, L, iters=20, warmup=3):
    """One new token per sequence over a 32768-token int8 cache, Qwen3-8B
    heads (32 query / 8 KV, head dim 128), batch 8; synthetic seeded bf16
    inputs quantised once.  Algorithmic bytes per launch: the cache codes
    (2 D bytes per key per KV head) and scales, the query codes and scales,
    and the 16-bit output."""
    B, Hq, Hkv, S_q, S_k, D = 8, 32, 8, 1, 32768, 128
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(4242)
    q = torch.randn((B, Hq, S_q, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_k, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_k, D), generator=g, device=dev).to(torch.bfloat16)
    q8, sq = L.lamp_quantize_blocks(q, 64, "i8")
    k8, sk = L.lamp_quantize_blocks(k, 64, "i8")
    v8, sv = L.lamp_quantize_blocks(v, 64, "i8")
    del k, v
    out = torch.empty((B, Hq, S_q, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(L.lamp_decode_workspace_bytes(B, Hkv, S_k, D), dtype=torch.uint8, device=dev)
    run = lambda: L.lamp_decode_fwd(q8, sq, k8, sk, v8, sv, causal=True, tile_m=64,
                                    dtype=torch.bfloat16, out=out, workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b_ in ev:
        a.record()
        run()
        b_.record()
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b_) for a, b_ in ev])) * 1e-3
    n_kt = -(-S_k // 64)
    nbytes = (2 * B * Hkv * S_k * D + 2 * B * Hkv * n_kt * 4 + B * Hq * S_q * D + B * Hq * 4 +
              2 * B * Hq * S_q * D)
    return {"workload": "qwen3_8b_decode_b8_q1_k32768_int8_kv", "batch": B, "q_heads": Hq,
            "kv_heads": Hkv, "new_tokens": S_q, "cache_tokens": S_k, "head_dim": D,
            "ms_mean": round(t * 1e3, 4), "algorithmic_bytes": nbytes,
            "achieved_gbs": round(nbytes / t / 1e9, 1), "peak_gbs": HBM_PEAK / 1e9,
            "frac_hbm": round(nbytes / t / HBM_PEAK, 4),
            "workspace_bytes": int(ws.numel())}


def copy_calibration(torch, mib):
    """One device-to-device copy of mib MiB: the reference dispatch that
    scales the HBM byte counters of a counter pass."""
    if mib <= 0:
        return
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=torch.device("cuda:0"))
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {n} bytes read + {n} bytes written")


def profile_suite(torch, L, steps, warmup):
    """Each benchmarked configuration's step (quantisers, mask builder,
    attention) run warmup + steps times, in a fixed order, then the decode
    step: one process whose kernel dispatches a profiler can attribute by
    order.  Returns the per-configuration mean attention time."""
    from synthetic import get_config, make_inputs
    dev = torch.device("cuda:0")
    out = {}
    runs = [("C5", 0.25, "i8", False), ("C5", 0.25, "e4m3", False), ("C5", 0.25, "e4m3", True),
            ("C4", None, None, False), ("C3", None, None, False)]
    cache = {}
    for name, f, code, pv8 in runs:
        cfg = get_config(name, f, code)
        if name not in cache:
            cache.clear()
            q, k, v = make_inputs(cfg)
            cache[name] = tuple(t.to(dev) for t in (q, k, v))
            del q, k, v
        qd, kd, vd = cache[name]
        pipe = Pipeline(L, cfg, qd, kd, vd, torch, pv8=pv8)
        ts = time_attn(torch, pipe, iters=steps, warmup=warmup, prep_each=True)
        key = cfg.name + ("_pv8" if pv8 else "")
        out[key] = round(float(np.mean(ts)) * 1e3, 4)
        log(f"[bench] profile suite: {key} attention {out[key]} ms")
        del pipe
    cache.clear()
    out["decode"] = decode_measurement(torch, L, iters=steps, warmup=warmup)["ms_mean"]
    return out


# ---------------------------------------------------------------------------
# traffic from the committed rocprofv3 counter summary of this kernel
# ---------------------------------------------------------------------------

def committed_traffic(workload):
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# ---------------------------------------------------------------------------

def host_description():
    """CPU model (from /proc/cpuinfo) and the BLAS library numpy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}".strip()
    except Exception:
        pass
    return model, blas


def cpu_baseline(cfg, q, k, v, budget_s=12.0):
    from oracle import attention as A
    from oracle import mask as omask
    cores = len(os.sched_getaffinity(0))
    cpu_model, blas = host_description()
    t_prep = 0.0
    dt = 0.0
    flops = 0.0
    tiles = 0
    heads = 0
    t0 = time.perf_counter()
    mw_all = omask.build_mask(cfg.B, cfg.Hq, cfg.S, cfg.S, cfg.tile_m, cfg.tile_n, cfg.tiles_per_bit,
                              cfg.frac_16bit, cfg.mask_seed, cfg.words_per_row)
    t_prep += time.perf_counter() - t0
    # query tiles of head (0, 0) from the last (longest) downwards, then of
    # the next heads, until the budget is spent
    for bh in range(cfg.B * cfg.Hq):
        if dt > budget_s:
            break
        b, h = divmod(bh, cfg.Hq)
        kvh = h // (cfg.Hq // cfg.Hkv)
        t0 = time.perf_counter()
        qn = q[b:b + 1, h:h + 1].double().numpy()
        kn = k[b:b + 1, kvh:kvh + 1].double().numpy()
        vn = v[b:b + 1, kvh:kvh + 1].double().numpy()
        mw = mw_all[b:b + 1, h:h + 1]
        P = A.make_problem(qn, kn, vn, causal=cfg.causal, code=cfg.code, tile_m=cfg.tile_m,
                           tile_n=cfg.tile_n, tiles_per_bit=cfg.tiles_per_bit,
                           frac_16bit=cfg.frac_16bit, seed=cfg.mask_seed, mask_words=mw,
                           adaptive=cfg.adaptive, exp8=cfg.exp8, tau=cfg.tau, sub_rows=cfg.sub_rows)
        t_prep += time.perf_counter() - t0
        heads += 1
        t1 = time.perf_counter()
        for qt in range(cfg.n_qt - 1, -1, -1):
            rows = np.arange(qt * cfg.tile_m, min(cfg.S, (qt + 1) * cfg.tile_m))
            if A.uses_lamp(P):
                per = cfg.tile_m // cfg.sub_rows
                A.attn_lamp(P, 0, 0, np.arange(qt * per, (qt + 1) * per))
            else:
                A.attn_tilemix(P, 0, 0, rows)
            nvalid = int(((np.arange(cfg.S)[None, :] <= rows[:, None]) if cfg.causal
                          else np.ones((len(rows), cfg.S), bool)).sum())
            flops += 4.0 * cfg.D * nvalid
            tiles += 1
            if dt + (time.perf_counter() - t1) > budget_s:
                break
        dt += time.perf_counter() - t1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": (f"numpy fp64 oracle, {tiles} query tiles of {cfg.tile_m} rows over {heads} "
                       f"head(s) from (b=0, h=0), each head's tiles from the longest down "
                       f"({tiles * cfg.tile_m} of {cfg.B * cfg.Hq * cfg.S} query rows of the "
                       f"workload), {dt:.1f} s; per-head quantisation + mask prep {t_prep:.1f} s "
                       f"excluded"),
            "seconds": round(dt, 2)}


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------

class Pipeline:
    """Preallocated buffers for one configuration; run() enqueues one step."""

    def __init__(self, L, cfg, qd, kd, vd, torch, template=None, seqlens=None, pv8=False):
        self.L, self.cfg, self.torch = L, cfg, torch
        self.pv8 = pv8                 # 8-bit P V on 8-bit tiles (V quantised too)
        self.template = template       # (sink, band, stride) groups, or the random mask
        # variable-length batch: one length per sequence (queries = keys)
        self.seqlens = None if seqlens is None else \
            torch.tensor(list(seqlens), dtype=torch.int32, device=qd.device)
        self.qd, self.kd, self.vd = qd, kd, vd
        dev = qd.device
        B, Hq, Hkv, S, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D
        self.q8 = torch.empty((B, Hq, S, D), dtype=torch.uint8, device=dev)
        self.k8 = torch.empty((B, Hkv, S, D), dtype=torch.uint8, device=dev)
        self.sq = torch.empty((B, Hq, cfg.n_qt), dtype=torch.float32, device=dev)
        self.sk = torch.empty((B, Hkv, cfg.n_kt), dtype=torch.float32, device=dev)
        self.mask = torch.empty((B, Hq, cfg.n_qt, cfg.words_per_row), dtype=torch.int64, device=dev)
        self.out = torch.empty_like(qd)
        self.flags = None
        if cfg.adaptive:
            self.flags = torch.empty(L.lamp.flags_shape(B, Hq, S, S), dtype=torch.int64, device=dev)
        self.f16 = 0.0 if cfg.mask_all_ones else cfg.frac_16bit
        self.v8 = self.vs = None
        if pv8:
            self.v8 = torch.empty((B, Hkv, cfg.n_kt, D, 64), dtype=torch.uint8, device=dev)
            self.vs = torch.empty((B, Hkv, cfg.n_kt), dtype=torch.float32, device=dev)

    def prep(self):
        L, c = self.L, self.cfg
        L.lamp_quantize_blocks(self.qd, c.tile_m, c.code, codes=self.q8, scales=self.sq,
                               seqlens=self.seqlens)
        L.lamp_quantize_blocks(self.kd, c.tile_n, c.code, codes=self.k8, scales=self.sk,
                               seqlens=self.seqlens)
        if self.pv8:
            L.lamp_quantize_v_tiles(self.vd, codes=self.v8, scales=self.vs, seqlens=self.seqlens)
        if self.template is not None:
            L.lamp_build_mask_template(c.B, c.Hq, c.S, c.S, c.tile_m, c.tile_n, c.tiles_per_bit,
                                       *self.template, c.words_per_row, mask=self.mask)
        else:
            L.lamp_build_mask(c.B, c.Hq, c.S, c.S, c.tile_m, c.tile_n, c.tiles_per_bit, self.f16,
                              c.mask_seed, c.words_per_row, mask=self.mask)

    def attn(self):
        L, c = self.L, self.cfg
        L.lamp_attn_fwd(self.qd, self.kd, self.vd, self.q8, self.k8, self.sq, self.sk, self.mask,
                        code=c.code, causal=c.causal, tile_m=c.tile_m,
                        tiles_per_bit=c.tiles_per_bit, words_per_row=c.words_per_row,
                        mode=L.LAMP_MODE_ADAPTIVE if c.adaptive else L.LAMP_MODE_MASK,
                        exp8=c.exp8, tau=c.tau, sub_rows=c.sub_rows, out=self.out,
                        flags_out=self.flags, seqlens_q=self.seqlens, seqlens_k=self.seqlens,
                        v8=self.v8, v_scale=self.vs)

    def counts(self):
        mw = self.mask.cpu().numpy().view(np.uint64)
        fl = None if self.flags is None else self.flags.cpu().numpy().view(np.uint64)
        ls = None if self.seqlens is None else self.seqlens.cpu().tolist()
        return route_counts(mw, self.cfg.S, self.cfg.S, self.cfg.tile_m, self.cfg.tile_n,
                            self.cfg.tiles_per_bit, self.cfg.causal, fl, ls, ls)


def other_workloads(torch, L):
    """Attention alone on the 32k-token int8 workload (f = 0.10) and on the
    adaptive e4m3 workload with 8-bit exponentials (head dim 256, outlier
    channels and a sink key), each against its mix-weighted roofline (the
    adaptive one counting its flagged recompute)."""
    from synthetic import get_config, make_inputs
    dev = torch.device("cuda:0")
    out = {}
    for name in ("C4", "C3"):
        cfg = get_config(name)
        q, k, v = make_inputs(cfg)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        del q, k, v
        sp = Pipeline(L, cfg, qd, kd, vd, torch)
        sp.prep()
        ts = time_attn(torch, sp, iters=10, warmup=2, prep_each=True)
        cc = sp.counts()
        tr = roofline_time(cc, cfg.D)
        med = float(np.median(ts))
        rec = {"workload": cfg.name, "attn_ms": round(med * 1e3, 4),
               "tflops": round(algorithmic_flops(cc, cfg.D) / med / 1e12, 1),
               "roofline_frac": round(tr / med, 4), "t_roof_ms": round(tr * 1e3, 4),
               "fa_convention_tflops": round(cfg.fa_flops() / med / 1e12, 1)}
        if cfg.adaptive:
            rec["flagged_frac_of_8bit"] = round(cc["nflag"] / max(1, cc["n8"]), 4)
        out[name] = rec
        del sp, qd, kd, vd
        torch.cuda.empty_cache()
    return out


def component_times(torch, pipe, iters=20):
    """Each enqueued part of a step timed alone with HIP events on the current
    stream: the Q and K quantisers (HBM-bound; bytes read + written against
    8 TB/s), the mask builder and the attention kernel."""
    L, c = pipe.L, pipe.cfg
    parts = {
        "quantize_q": (lambda: L.lamp_quantize_blocks(pipe.qd, c.tile_m, c.code, codes=pipe.q8,
                                                      scales=pipe.sq, seqlens=pipe.seqlens),
                       3 * pipe.qd.numel() + 4 * pipe.sq.numel()),
        "quantize_k": (lambda: L.lamp_quantize_blocks(pipe.kd, c.tile_n, c.code, codes=pipe.k8,
                                                      scales=pipe.sk, seqlens=pipe.seqlens),
                       3 * pipe.kd.numel() + 4 * pipe.sk.numel()),
        "build_mask": (lambda: L.lamp_build_mask(c.B, c.Hq, c.S, c.S, c.tile_m, c.tile_n,
                                                 c.tiles_per_bit, pipe.f16, c.mask_seed,
                                                 c.words_per_row, mask=pipe.mask), None),
        "attention": (pipe.attn, None),
    }
    out = {}
    for name, (fn, nbytes) in parts.items():
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        rec = {"ms": round(ms, 4)}
        if nbytes is not None:
            rec["bytes"] = int(nbytes)
            rec["gbs"] = round(nbytes / ms / 1e6, 1)
            rec["frac_hbm"] = round(nbytes / ms / 1e6 / (HBM_PEAK / 1e9), 4)
        out[name] = rec
    return out


def time_attn(torch, pipe, iters, warmup, prep_each=False):
    """Attention launch times (HIP events around each launch); prep_each:
    the quantisers and the mask builder run before every launch as well
    (outside the events)."""
    if not prep_each:
        pipe.prep()
    for _ in range(warmup):
        if prep_each:
            pipe.prep()
        pipe.attn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        if prep_each:
            pipe.prep()
        a.record()
        pipe.attn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C5", choices=["C1", "C2", "C3", "C4", "C5"])
    ap.add_argument("--frac", type=float, default=None, help="C5: 16-bit fraction")
    ap.add_argument("--code", default=None, choices=["i8", "e4m3"], help="C5: 8-bit code")
    ap.add_argument("--no-sweep", action="store_true", help="skip the C5 precision-mix sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device-to-device once (reference "
                         "dispatch for scaling the HBM byte counters)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode measurement over an int8 K/V cache (for profiling)")
    ap.add_argument("--profile-suite", action="store_true",
                    help="only run --steps steps of every benchmarked kernel configuration, one "
                         "after the other (for rocprofv3 counter passes)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(each (batch, KV head) group is independent: the path would shard by KV head "
              f"with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixed_precision_tiled_amd as L
    from synthetic import C5_FRACS, get_config, make_inputs

    if args.decode_only:
        print(json.dumps({"decode_int8_kv": decode_measurement(torch, L)}), flush=True)
        return
    if args.profile_suite:
        res = profile_suite(torch, L, args.steps, args.warmup)
        copy_calibration(torch, args.copy_calibration)
        print(json.dumps({"profile_suite": res}), flush=True)
        return

    cfg = get_config(args.config, args.frac, args.code)
    if args.config == "C5" and args.frac is None and args.code is None:
        cfg = get_config("C5", 0.25, "i8")
    dev = torch.device("cuda:0")
    log(f"[bench] workload {cfg.name}: generating inputs")
    q, k, v = make_inputs(cfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    pipe = Pipeline(L, cfg, qd, kd, vd, torch)

    # ---- warmup, then exactly K timed steps ----
    for _ in range(args.warmup):
        pipe.prep()
        pipe.attn()
    torch.cuda.synchronize()
    attn_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        pipe.prep()
        attn_ev[i][0].record()
        pipe.attn()
        attn_ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_s = t_start.elapsed_time(t_end) * 1e-3 / args.steps
    attn_s = np.array([a.elapsed_time(b) for a, b in attn_ev]) * 1e-3
    log(f"[bench] {args.steps} steps: {step_s * 1e3:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}),"
        f" attention mean {attn_s.mean() * 1e3:.3f} ms min {attn_s.min() * 1e3:.3f}")

    c = pipe.counts()
    F = algorithmic_flops(c, cfg.D)
    T_roof = roofline_time(c, cfg.D)
    attn_mean = float(attn_s.mean())
    achieved = F / attn_mean / 1e12
    peak = F / T_roof / 1e12
    traffic = committed_traffic(cfg.name)
    result = {
        "metric": "mixed-precision attn prefill TFLOP/s & % of mix-weighted MFMA roofline",
        "value": round(F / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("i8" if cfg.code == "i8" else "e4m3") + "+bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "seq_len": cfg.S, "head_dim": cfg.D, "causal": cfg.causal,
                   "tile_m": cfg.tile_m, "tile_n": cfg.tile_n,
                   "tiles_per_bit": cfg.tiles_per_bit, "frac_16bit": cfg.frac_16bit,
                   "code": cfg.code, "exp8": cfg.exp8, "adaptive": cfg.adaptive,
                   "input_dtype": cfg.dtype},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 2),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": "attn_fwd_kernel", "attn_ms_mean": round(attn_mean * 1e3, 4),
                     "attn_ms_min": round(float(attn_s.min()) * 1e3, 4),
                     "t_roof_ms": round(T_roof * 1e3, 4),
                     "counts": c, "fa_convention_tflops": round(cfg.fa_flops() / attn_mean / 1e12, 2),
                     "peaks": {"int8_fp8": PEAK8, "bf16_fp16": PEAK16},
                     "kernel_source_sha256": kernel_source_hash()},
    }
    result["components"] = component_times(torch, pipe)
    log(f"[bench] components: {json.dumps(result['components'])}")
    sus = sustained_mfma_peaks(torch)
    if sus is not None:
        p8s, p16s = sus["int8_fp8"]["ops_per_s"], sus["bf16_fp16"]["ops_per_s"]
        t_sus = roofline_time_at(c, cfg.D, p8s, p16s)
        result["roofline"]["sustained"] = {
            "peaks": {"int8_fp8": round(p8s, -9), "bf16_fp16": round(p16s, -9)},
            "clock_ghz": {"int8_fp8": sus["int8_fp8"]["clock_ghz"],
                          "bf16_fp16": sus["bf16_fp16"]["clock_ghz"]},
            "t_roof_ms": round(t_sus * 1e3, 4), "frac": round(t_sus / attn_mean, 4)}
        log(f"[bench] sustained MFMA: {json.dumps(result['roofline']['sustained'])}")
    if args.config == "C5" and not args.no_sweep:
        sweep = {}
        for code in ("i8", "e4m3"):
            for f in C5_FRACS:
                sc = get_config("C5", f, code)
                sp = Pipeline(L, sc, qd, kd, vd, torch)
                sp.prep()
                ts = time_attn(torch, sp, iters=10, warmup=2, prep_each=True)
                cc = sp.counts()
                tr = roofline_time(cc, sc.D)
                sweep[f"{code}_f{int(round(100 * f)):02d}"] = {
                    "attn_ms": round(float(np.median(ts)) * 1e3, 4),
                    "tflops": round(algorithmic_flops(cc, sc.D) / float(np.median(ts)) / 1e12, 1),
                    "roofline_frac": round(tr / float(np.median(ts)), 4),
                    "t_roof_ms": round(tr * 1e3, 4)}
                del sp
        # a structured static template with about a quarter of the valid
        # elements on the 16-bit path (sink group, band of 2, every 5th group)
        tpl = (1, 2, 5)
        sc = get_config("C5", 0.25, "i8")
        sp = Pipeline(L, sc, qd, kd, vd, torch, template=tpl)
        sp.prep()
        ts = time_attn(torch, sp, iters=10, warmup=2, prep_each=True)
        cc = sp.counts()
        tr = roofline_time(cc, sc.D)
        sweep["i8_template_sink1_band2_stride5"] = {
            "attn_ms": round(float(np.median(ts)) * 1e3, 4),
            "tflops": round(algorithmic_flops(cc, sc.D) / float(np.median(ts)) / 1e12, 1),
            "roofline_frac": round(tr / float(np.median(ts)), 4),
            "t_roof_ms": round(tr * 1e3, 4),
            "frac_16bit_elements": round(cc["n16"] / cc["nvalid"], 4)}
        del sp
        # a variable-length batch in the same padded tensors: 16384 and 6000
        # tokens
        lens = (16384, 6000)
        sp = Pipeline(L, sc, qd, kd, vd, torch, seqlens=lens)
        sp.prep()
        ts = time_attn(torch, sp, iters=10, warmup=2, prep_each=True)
        cc = sp.counts()
        tr = roofline_time(cc, sc.D)
        sweep["i8_f25_varlen_16384_6000"] = {
            "attn_ms": round(float(np.median(ts)) * 1e3, 4),
            "tflops": round(algorithmic_flops(cc, sc.D) / float(np.median(ts)) / 1e12, 1),
            "roofline_frac": round(tr / float(np.median(ts)), 4),
            "t_roof_ms": round(tr * 1e3, 4)}
        del sp
        # the 8-bit P V product on 8-bit tiles (e4m3 path with 8-bit
        # exponentials), all tiles 8-bit and a quarter of the groups 16-bit
        for f in (0.0, 0.25):
            sc = get_config("C5", f, "e4m3")
            sp = Pipeline(L, sc, qd, kd, vd, torch, pv8=True)
            sp.prep()
            ts = time_attn(torch, sp, iters=10, warmup=2, prep_each=True)
            cc = sp.counts()
            tr = roofline_time_pv8(cc, sc.D)
            sweep[f"e4m3_f{int(round(100 * f)):02d}_pv8"] = {
                "attn_ms": round(float(np.median(ts)) * 1e3, 4),
                "tflops": round(algorithmic_flops(cc, sc.D) / float(np.median(ts)) / 1e12, 1),
                "roofline_frac": round(tr / float(np.median(ts)), 4),
                "t_roof_ms": round(tr * 1e3, 4)}
            del sp
        result["sweep_c5_attention"] = sweep
        log(f"[bench] sweep {json.dumps(sweep)}")
    if not args.no_sweep:
        dm = decode_measurement(torch, L)
        result["decode_int8_kv"] = dm
        log(f"[bench] decode over an int8 K/V cache: {json.dumps(dm)}")
        ow = other_workloads(torch, L)
        result["other_workloads"] = ow
        log(f"[bench] other workloads: {json.dumps(ow)}")
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, q, k, v, budget_s=args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    copy_calibration(torch, args.copy_calibration)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
