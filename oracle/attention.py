"""Mixed-precision attention prefill forward (oracle; test infrastructure only).

Sources:
* "TileMix: Mixed-Precision Attention for Faster LLM Prefill", section 2
  "How It Works": the score matrix is cut into tiles ("The Tile
  Architecture"); the inner loop reads the mask bit of the current key-tile
  group and sends the tile down a 16-bit floating-point product or an INT8
  product rescaled by per-block scale factors ("The Dual-Path Engine"); both
  paths update the same online-softmax running maximum and normaliser, so the
  full dense attention graph is kept.
* "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
  Accelerators", Abstract: products and exponentials evaluated in 8-bit
  formats, sensitive sub-blocks identified adaptively and recomputed in 16-bit.

Two definitions are implemented:

``tilemix``  (mask routing, exponentials in full precision).  Because the
    online softmax is an exact rewrite of softmax, the result is plain softmax
    attention over per-element routed logits, written out directly:
    s_ij = s8_ij if the tile of (i, j) is routed 8-bit else s16_ij,
    O_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i) over valid j.

``lamp``  (8-bit exponentials and/or adaptive routing).  Rounding to 8 bits
    depends on the running maximum at the time a tile is processed, so the
    online softmax is emulated tile by tile in ascending key-tile order, with
    the state (m, l, acc) updated after each key tile of tile_n columns.

Logits (fp64):
    16-bit: s16 = sm * q . k
    int8:   s8  = (cq . ck) * sQ[qt] * sK[kt] * sm, the integer dot exact
    e4m3:   s8  = (val(cq) . val(ck)) * sQ * sK * sm, exact in fp64 (every
            product is a multiple of 2**-18 below 2**18 and at most 256 terms
            are summed)

Readings where the pages are silent (listed in the design notes): causal
aligns the queries with the end of the keys, as for a chunk of S_q new
queries after S_k - S_q earlier tokens: query i sits at key position
i + S_k - S_q and sees keys j <= i + S_k - S_q (so S_q <= S_k; S_q == S_k is
the plain lower triangle); a variable-length batch gives each sequence b its
own lengths Lq[b] <= S_q and Lk[b] <= S_k inside the padded tensors, rows and
keys beyond them are padding (quantised as zeros, never attended, their
outputs undefined), and causal alignment uses Lk[b] - Lq[b]; a row with no
valid key has O = 0 and LSE = -inf; GQA maps query head h to KV head
h // (Hq / Hkv); sm defaults to 1 / sqrt(D); the 8-bit logit that is rounded
is the max-shifted x = s - m_new, then exp(x) is rounded again, both to E4M3
with round-to-nearest-even and saturation; alpha = exp(m - m_new) is full
precision; a sub-block is sub_rows query rows by one key tile, flagged when
some valid 8-bit-routed logit lies within tau of the look-ahead running
maximum m' = max(m, rowmax of the tile's 8-bit logits); flagged sub-blocks use
16-bit logits for the whole sub-block.

Optional 8-bit P V (``pv8``, with exp8 and mask routing; a variant the pages
do not specify): on 8-bit tiles the e4m3 weights multiply V quantised to e4m3
with one power-of-two scale per tile_n-key block (``quant.quantize_v_tiles``);
16-bit tiles keep the 16-bit V.  The normaliser still sums the weights.
"""
from dataclasses import dataclass, field

import numpy as np

from . import e4m3, mask as omask, quant

U32 = 2.0 ** -24          # unit roundoff of fp32, for the fragility bounds


@dataclass
class Problem:
    q: np.ndarray                 # [B, Hq, S_q, D] float64 (exact upcast of 16-bit)
    k: np.ndarray                 # [B, Hkv, S_k, D]
    v: np.ndarray                 # [B, Hkv, S_k, D]
    causal: bool
    code: str                     # "i8" | "e4m3"
    tile_m: int
    tile_n: int
    tiles_per_bit: int
    mask_words: np.ndarray        # [B, Hq, n_qt, W] uint64
    q_codes: np.ndarray
    q_scales: np.ndarray
    k_codes: np.ndarray
    k_scales: np.ndarray
    sm_scale: float = 0.0
    adaptive: bool = False
    exp8: bool = False
    tau: float = 4.0
    sub_rows: int = 32
    seqlens_q: np.ndarray = None  # [B] lengths of a variable-length batch (None: S_q)
    seqlens_k: np.ndarray = None  # [B] (None: S_k)
    pv8: bool = False             # 8-bit P V on 8-bit tiles (needs exp8, mask routing)
    v_codes: np.ndarray = None    # [B, Hkv, S_k, D] e4m3 codes of V (pv8)
    v_scales: np.ndarray = None   # [B, Hkv, n_kt] power-of-two block scales (pv8)

    def __post_init__(self):
        B, Hq, S_q, D = self.q.shape
        _, Hkv, S_k, _ = self.k.shape
        if Hq % Hkv:
            raise ValueError("Hq must be a multiple of Hkv")
        if self.causal and S_q > S_k:
            raise ValueError("causal needs S_q <= S_k")
        if self.sm_scale <= 0:
            self.sm_scale = 1.0 / np.sqrt(D)
        self.B, self.Hq, self.Hkv, self.S_q, self.S_k, self.D = B, Hq, Hkv, S_q, S_k, D
        self.Lq = np.full(B, S_q) if self.seqlens_q is None else np.asarray(self.seqlens_q)
        self.Lk = np.full(B, S_k) if self.seqlens_k is None else np.asarray(self.seqlens_k)
        if self.Lq.shape != (B,) or self.Lk.shape != (B,):
            raise ValueError("one length per batch entry")
        if (self.Lq < 0).any() or (self.Lq > S_q).any() or (self.Lk < 0).any() or (self.Lk > S_k).any():
            raise ValueError("lengths outside [0, S]")
        if self.causal and (self.Lq > self.Lk).any():
            raise ValueError("causal needs Lq[b] <= Lk[b]")
        self.n_qt = omask.n_tiles(S_q, self.tile_m)
        self.n_kt = omask.n_tiles(S_k, self.tile_n)
        self.n_g = omask.n_tiles(self.n_kt, self.tiles_per_bit)
        self.qv = quant.code_values(self.q_codes, self.code)
        self.kv = quant.code_values(self.k_codes, self.code)
        self.bits = omask.unpack_bits(self.mask_words, self.n_g)   # [B,Hq,n_qt,n_g]
        if self.pv8:
            if not self.exp8 or self.adaptive:
                raise ValueError("the 8-bit P V product needs exp8 and mask routing")
            if self.v_codes is None or self.v_scales is None:
                raise ValueError("pv8 needs V codes and scales")
            self.v8 = quant.dequantize(self.v_codes, self.v_scales, self.tile_n, "e4m3")

    def kvh(self, h):
        return h // (self.Hq // self.Hkv)

    def route8_tiles(self, b, h):
        """[n_qt, n_kt] bool: tile routed to the 8-bit path by the mask."""
        g = np.arange(self.n_kt) // self.tiles_per_bit
        return self.bits[b, h][:, g].astype(bool)

    def valid(self, rows, cols, b=0):
        lq, lk = int(self.Lq[b]), int(self.Lk[b])
        ok = (cols[None, :] < lk) & (rows[:, None] < lq)
        if self.causal:
            ok &= cols[None, :] <= rows[:, None] + (lk - lq)
        return ok


def make_problem(q, k, v, *, causal, code, tile_m, tile_n, tiles_per_bit, frac_16bit,
                 seed, words_per_row=None, mask_words=None, **kw):
    """Build a Problem from 16-bit inputs (given as float arrays) end to end:
    oracle quantisation of Q (blocks of tile_m rows) and K (tile_n rows), and
    the random mask template unless ``mask_words`` is given."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qc, qs = quant.quantize_blocks(q, tile_m, code, kw.get("seqlens_q"))
    kc, ks = quant.quantize_blocks(k, tile_n, code, kw.get("seqlens_k"))
    if kw.get("pv8") and "v_codes" not in kw:
        kw["v_codes"], kw["v_scales"] = quant.quantize_v_tiles(v, tile_n, kw.get("seqlens_k"))
    B, Hq, S_q, _ = q.shape
    S_k = k.shape[2]
    if mask_words is None:
        n_g = omask.n_tiles(omask.n_tiles(S_k, tile_n), tiles_per_bit)
        W = words_per_row or omask.n_tiles(n_g, 64)
        mask_words = omask.build_mask(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit,
                                      frac_16bit, seed, W)
    return Problem(q=q, k=k, v=v, causal=causal, code=code, tile_m=tile_m, tile_n=tile_n,
                   tiles_per_bit=tiles_per_bit, mask_words=mask_words, q_codes=qc,
                   q_scales=qs, k_codes=kc, k_scales=ks, **kw)


# ---------------------------------------------------------------------------
# logits
# ---------------------------------------------------------------------------

def logits16(P, b, h, rows, cols):
    return P.sm_scale * (P.q[b, h][rows] @ P.k[b, P.kvh(h)][cols].T)


def acc8(P, b, h, rows, cols):
    """Exact 8-bit dot products (integer-valued for int8)."""
    return P.qv[b, h][rows] @ P.kv[b, P.kvh(h)][cols].T


def logits8(P, b, h, rows, cols):
    sq = P.q_scales[b, h].astype(np.float64)[rows // P.tile_m]
    sk = P.k_scales[b, P.kvh(h)].astype(np.float64)[cols // P.tile_n]
    return acc8(P, b, h, rows, cols) * sq[:, None] * sk[None, :] * P.sm_scale


def int_acc_exact(P, b, h, rows, cols):
    """int8 path only: the integer accumulator as int64, computed with integer
    arithmetic (used to pin acc8 and to compare the GPU's int32 dump)."""
    if P.code != "i8":
        raise ValueError("integer accumulator exists on the int8 path only")
    qi = P.q_codes[b, h][rows].view(np.int8).astype(np.int64)
    ki = P.k_codes[b, P.kvh(h)][cols].view(np.int8).astype(np.int64)
    return np.einsum("id,jd->ij", qi, ki)


def routed_logits(P, b, h, rows):
    """Per-element routed logits s[rows, S_k], the 8-bit mask, the valid mask."""
    cols = np.arange(P.S_k)
    r8 = P.route8_tiles(b, h)[(rows // P.tile_m)][:, cols // P.tile_n]
    s = np.where(r8, logits8(P, b, h, rows, cols), logits16(P, b, h, rows, cols))
    return s, r8, P.valid(rows, cols, b)


# ---------------------------------------------------------------------------
# TileMix: exact softmax over routed logits
# ---------------------------------------------------------------------------

def attn_tilemix(P, b, h, rows):
    """O[rows, D], LSE[rows] of head (b, h) under mask routing, full-precision exp."""
    rows = np.asarray(rows)
    s, _, ok = routed_logits(P, b, h, rows)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    none = ~ok.any(axis=1)               # rows with no valid key: O = 0, LSE = -inf
    m = np.where(none, 0.0, m)
    p = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    l_safe = np.where(none, 1.0, l)
    O = (p @ P.v[b, P.kvh(h)]) / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(none, -np.inf, m + np.log(l_safe))
    return O, lse


# ---------------------------------------------------------------------------
# LampAttention: tile-by-tile emulation
# ---------------------------------------------------------------------------

_P8_CACHE = {}


def exp8_of_code(codes):
    """p = E4M3(exp(val(code))) for e4m3 codes of non-positive logits."""
    return e4m3.round_to_e4m3(np.exp(e4m3.decode(codes)))


def exp8(x):
    """E4M3(exp(E4M3(x))) for x <= 0 (saturating at -448)."""
    return exp8_of_code(e4m3.encode(x))


@dataclass
class LampResult:
    O: np.ndarray
    lse: np.ndarray
    flags: np.ndarray             # [n_sb_rows, n_kt] bool, sub-block recomputed in 16-bit
    flag_dontcare: np.ndarray     # [n_sb_rows, n_kt] bool, decision within the GPU error bound
    fragile_rows: np.ndarray      # [R] bool, rows excluded from pass/fail
    extra_tol: np.ndarray         # [R] widening of the per-row tolerance (exp8 flips)
    counts: dict = field(default_factory=dict)


def _err_logits(P, b, h, rows, cols, s, use16):
    """Bound on the GPU's fp32 error in each logit (see design notes).

    8-bit int8: the accumulator is exact; the scale product and the final
    multiply add at most 3 roundings -> 4u|s|.  8-bit e4m3 and 16-bit: exact
    products summed in fp32 -> gamma_D * sum|products| * scale, plus 4u|s|.
    """
    D = P.D
    gam = D * U32 / (1 - D * U32)
    sm = P.sm_scale
    qa16, ka16 = np.abs(P.q[b, h][rows]), np.abs(P.k[b, P.kvh(h)][cols])
    e16 = gam * sm * (qa16 @ ka16.T)
    if P.code == "i8":
        e8 = np.zeros_like(s)
    else:
        sq = P.q_scales[b, h].astype(np.float64)[rows // P.tile_m]
        sk = P.k_scales[b, P.kvh(h)].astype(np.float64)[cols // P.tile_n]
        e8 = gam * (np.abs(P.qv[b, h][rows]) @ np.abs(P.kv[b, P.kvh(h)][cols]).T) \
            * sq[:, None] * sk[None, :] * sm
    return np.where(use16, e16, e8) + 4 * U32 * np.abs(s)


def attn_lamp(P, b, h, sub_blocks):
    """Emulate the online softmax for the given sub-blocks (indices of
    sub_rows-row blocks of head (b, h)); rows processed together, key tiles in
    ascending order."""
    sr = P.sub_rows
    sub_blocks = np.asarray(sub_blocks, dtype=np.int64)
    rows = (sub_blocks[:, None] * sr + np.arange(sr)[None, :]).reshape(-1)
    rows = rows[rows < P.S_q]
    sbid = rows // sr                                   # sub-block of each row
    usb, sb_idx = np.unique(sbid, return_inverse=True)  # local sub-block index per row
    R, D = len(rows), P.D
    vh = P.v[b, P.kvh(h)]
    r8_tiles = P.route8_tiles(b, h)
    qt = rows // P.tile_m

    m = np.full(R, -np.inf)
    em = np.zeros(R)                      # bound on |m_gpu - m_ref|
    l = np.zeros(R)
    acc = np.zeros((R, D))
    flags = np.zeros((len(usb), P.n_kt), dtype=bool)
    dontcare = np.zeros((len(usb), P.n_kt), dtype=bool)
    diverged = np.zeros(len(usb), dtype=bool)
    frag_p = np.zeros(R)                  # sum of possible p flips
    frag_pv = np.zeros(R)                 # sum of p flips times max|v_j|
    vmax = np.abs(vh).max(axis=1)
    n8 = n16 = nflag = nvalid = 0

    for kt in range(P.n_kt):
        cols = np.arange(kt * P.tile_n, min(P.S_k, (kt + 1) * P.tile_n))
        ok = P.valid(rows, cols, b)
        if not ok.any():
            continue
        r8 = r8_tiles[qt, kt][:, None] & ok             # valid and 8-bit routed
        s8 = logits8(P, b, h, rows, cols)
        s16 = logits16(P, b, h, rows, cols)
        flag_row = np.zeros(R, dtype=bool)
        if P.adaptive:
            s8v = np.where(r8, s8, -np.inf)
            rowmax8 = s8v.max(axis=1)
            e8 = _err_logits(P, b, h, rows, cols, s8, np.zeros_like(ok))
            has8 = r8.any(axis=1)
            mprime = np.maximum(m, rowmax8)
            with np.errstate(invalid="ignore"):
                d_row = np.where(has8, rowmax8 - mprime, -np.inf)
            e_row = np.where(has8, np.where(r8, e8, 0).max(axis=1, initial=0) + em, 0.0)
            for i_sb in range(len(usb)):
                sel = (sb_idx == i_sb) & has8
                if not sel.any():
                    continue
                dmax = d_row[sel].max() + P.tau
                flagged = dmax >= 0
                flags[i_sb, kt] = flagged
                if abs(dmax) <= 2 * e_row[sel].max() + 4 * U32 * (abs(P.tau) + 1):
                    dontcare[i_sb, kt] = True
                    diverged[i_sb] = True
                if diverged[i_sb]:
                    dontcare[i_sb, kt] = True
                if flagged:
                    flag_row |= (sb_idx == i_sb)
        use16 = (~r8_tiles[qt, kt])[:, None] | flag_row[:, None]
        use16 = np.broadcast_to(use16, ok.shape)
        s = np.where(use16, s16, s8)
        sv = np.where(ok, s, -np.inf)
        m_new = np.maximum(m, sv.max(axis=1))
        es = _err_logits(P, b, h, rows, cols, s, use16)
        em = np.where(np.isfinite(m_new), np.maximum(em, np.where(ok, es, 0).max(axis=1)), em)
        with np.errstate(invalid="ignore"):
            x = np.where(ok, s - m_new[:, None], -np.inf)
        p16 = np.exp(x)
        if P.exp8:
            xc = np.maximum(np.where(ok, x, -448.0), -448.0)
            p8 = exp8(xc)
            ex = es + em[:, None] + 2 * U32 * (np.abs(xc) + np.abs(s))
            lo = exp8(np.maximum(xc - ex, -448.0))
            hi = exp8(np.minimum(xc + ex, 0.0))
            dp = np.where(ok & ~use16, hi - lo, 0.0)
            frag_p += dp.sum(axis=1)
            frag_pv += (dp * vmax[cols][None, :]).sum(axis=1)
        else:
            p8 = p16
        p = np.where(ok, np.where(use16, p16, p8), 0.0)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        alpha = np.where(np.isfinite(m_new), alpha, 1.0)
        l = alpha * l + p.sum(axis=1)
        if P.pv8:
            # 8-bit weights meet the e4m3 V codes of their tile (products exact)
            p8v = np.where(use16, 0.0, p)
            acc = alpha[:, None] * acc + (p - p8v) @ vh[cols] + p8v @ P.v8[b, P.kvh(h)][cols]
        else:
            acc = alpha[:, None] * acc + p @ vh[cols]
        m = np.where(np.isfinite(m_new), m_new, m)
        n8 += int((ok & r8).sum())
        n16 += int((ok & ~np.broadcast_to(r8_tiles[qt, kt][:, None], ok.shape)).sum())
        nflag += int((ok & r8 & flag_row[:, None]).sum())
        nvalid += int(ok.sum())

    none = l == 0                        # rows with no valid key: O = 0, LSE = -inf
    l_safe = np.where(none, 1.0, l)
    O = acc / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(none, -np.inf, m + np.log(l_safe))
    fragile_rows = diverged[sb_idx]
    extra = (frag_pv + frag_p * np.abs(O).max(axis=1)) / l_safe
    counts = dict(n8=n8, n16=n16, nflag=nflag, nvalid=nvalid)
    return LampResult(O=O, lse=lse, flags=flags, flag_dontcare=dontcare,
                      fragile_rows=fragile_rows, extra_tol=extra, counts=counts), rows, usb


def uses_lamp(P):
    return P.adaptive or P.exp8


# ---------------------------------------------------------------------------
# route counts (roofline input)
# ---------------------------------------------------------------------------

def route_counts(P):
    """Valid score elements per path under the mask: dict(n8, n16, nvalid).

    Tiles above the causal diagonal are not counted; diagonal and ragged
    tiles are counted per element.
    """
    n8 = n16 = 0
    rows_all = np.arange(P.S_q)
    for b in range(P.B):
        for qt in range(P.n_qt):
            rows = rows_all[qt * P.tile_m:(qt + 1) * P.tile_m]
            for kt in range(P.n_kt):
                cols = np.arange(kt * P.tile_n, min(P.S_k, (kt + 1) * P.tile_n))
                nv = int(P.valid(rows, cols, b).sum())
                if nv == 0:
                    continue
                g = kt // P.tiles_per_bit
                n8b = int(P.bits[b, :, qt, g].sum())
                n8 += nv * n8b
                n16 += nv * (P.Hq - n8b)
    return dict(n8=n8, n16=n16, nvalid=n8 + n16)
