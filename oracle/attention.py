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

Tolerances (for the comparison with an fp32 evaluation): every logit carries
a rigorous bound on its evaluation error (fp32 sums of the exact products in
any order, the gfx950 matrix cores' cut of e4m3 products, the fp32 scale
roundings).  ``attn_lamp`` takes every flag decision whose margin lies within
its bound both ways (one branch per outcome), and widens each output element
by the exact effect of moving every weight as far as its logit's bound
allows: the e4m3 rounding flips one by one, the relative weight errors through
Cauchy-Schwarz on running moments of V, all in the frame of the final running
maximum.  The LSE bound adds the maximum's, the exponents' and the flips'
shares to the rounding of the sum and the logarithm.

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
# e4m3 products on the gfx950 matrix cores (the pages fix no accuracy for the
# 8-bit products; this is what the hardware was measured to do): within each
# group of 8 consecutive head-dim indices every product is cut toward zero to
# a multiple of 2^(e + 1 - 14), e the largest exponent sum ea + eb of the
# group's operand pairs, before the group sums are added in fp32.
F8_GROUP = 8
F8_WINDOW = 14


def _e4m3_exp(v):
    """Exponent by which the matrix cores align an e4m3 value: floor(log2|v|)
    for normal values, -6 for subnormal values and zero (the exponent field's
    minimum)."""
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -6, e, -6.0)


def _f8_cut_err(qv, kv):
    """Bound [R, C] on how far the matrix cores' cut (above) moves the dot
    products of the rows of qv [R, D] with the rows of kv [C, D] (e4m3
    values): cut toward zero to
    a multiple of its group's granule 2^(e + 1 - F8_WINDOW), a product p
    loses its remainder r = p - trunc(p / granule) * granule (all of it below
    a granule; nothing within 7 binades of the group's largest, as an e4m3
    product has at most 8 significant bits).  The positive products can only
    lower the sum and the negative ones only raise it, so the error is at
    most the larger of the two losses, (sum |r| + |sum r|) / 2.  Products,
    granules and remainders are exact in fp32 (8 significant bits, exponents
    within [-18, 18]); the sums are taken in fp64."""
    R, D = qv.shape
    C, G = kv.shape[0], D // F8_GROUP
    # [index in group, row, group], one contiguous slice per index in group
    qj = np.ascontiguousarray(qv.reshape(R, G, F8_GROUP).transpose(2, 0, 1)).astype(np.float32)
    kj = np.ascontiguousarray(kv.reshape(C, G, F8_GROUP).transpose(2, 0, 1)).astype(np.float32)
    pq = np.ldexp(np.float32(1), _e4m3_exp(qj).astype(np.int32)).astype(np.float32)
    pk = np.ldexp(np.float32(1), _e4m3_exp(kj).astype(np.int32)).astype(np.float32)
    err = np.zeros((R, C))
    step = max(1, (1 << 18) // max(1, C * G))         # rows per chunk
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        top = pq[0, r0:r1, None] * pk[0, None]         # 2^e of each group, [r, C, G]
        for j in range(1, F8_GROUP):
            np.maximum(top, pq[j, r0:r1, None] * pk[j, None], out=top)
        gran = top * np.float32(2.0 ** (1 - F8_WINDOW))
        inv = np.float32(2.0 ** (F8_WINDOW - 1)) / top
        tot, sgn = np.zeros(top.shape), np.zeros(top.shape)
        for j in range(F8_GROUP):
            prod = qj[j, r0:r1, None] * kj[j, None]
            cut = np.trunc(prod * inv) * gran
            rem = prod - cut
            sgn += rem
            tot += np.abs(rem)
        err[r0:r1] = 0.5 * (tot.sum(axis=2) + np.abs(sgn.sum(axis=2)))
    return err


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


def _err_logits_tilemix(P, b, h, rows, cols, s, r8, m_row):
    """Bound on the error of an fp32 evaluation of the max-shifted exponent
    s - m under mask routing (natural-log units), for any reference m the
    evaluation chooses: exact 8-bit integer products (int8) or exact products
    summed in fp32 in any order (16-bit: gamma_D * sum|products| * scale,
    Higham eq. (3.5); e4m3: the same plus the matrix cores' cut of each
    group's products), a scale product of a few fp32 roundings that
    may be cut to 21 significant bits, and one rounding of the shifted
    exponent: 20u(|s| + |m|) covers the latter two with room."""
    D = P.D
    gam = D * U32 / (1 - D * U32)
    sm = P.sm_scale
    e = gam * sm * (np.abs(P.q[b, h][rows]) @ np.abs(P.k[b, P.kvh(h)][cols]).T)
    if P.code == "i8":
        e8 = np.zeros_like(s)
    else:
        sq = P.q_scales[b, h].astype(np.float64)[rows // P.tile_m]
        sk = P.k_scales[b, P.kvh(h)].astype(np.float64)[cols // P.tile_n]
        qv, kv = P.qv[b, h][rows], P.kv[b, P.kvh(h)][cols]
        e8 = (gam * (np.abs(qv) @ np.abs(kv).T) + _f8_cut_err(qv, kv)) \
            * sq[:, None] * sk[None, :] * sm
    return np.where(r8, e8, e) + 20 * U32 * (np.abs(s) + np.abs(m_row)[:, None])


def tilemix_bounds(P, b, h, rows, dtype="bf16"):
    """``attn_tilemix`` with bounds for an fp32 evaluation whose exponents
    carry errors within ``_err_logits_tilemix`` (E).

    The evaluation's weights share one reference (a common factor O does not
    see), so weight k is p_k exp(d_k) with |d_k| <= E_k, and O moves by
    sum_k p_k (exp(d_k) - 1) (v_k - O) / sum_k p_k exp(d_k): at most
    sqrt(sum p eps^2) sqrt(sum p (v - O)^2) / (l - sum p eps) per element
    (eps = expm1(E), Cauchy-Schwarz), the widening.  The LSE moves by at most
    max_j E_j, plus half an ulp of the 16-bit weights that the normaliser
    sums, fp16 subnormal weights (2^-25 each against l >= 1) and fp32
    rounding of the sum and the logarithm.  Returns (O [R, D], LSE [R],
    lse_tol [R], widening [R, D])."""
    rows = np.asarray(rows)
    s, r8, ok = routed_logits(P, b, h, rows)
    none = ~ok.any(axis=1)
    m = np.where(none, 0.0, np.where(ok, s, -np.inf).max(axis=1))
    sf = np.where(ok, s, 0.0)
    E = np.where(ok, _err_logits_tilemix(P, b, h, rows, np.arange(P.S_k), sf, r8, m), 0.0)
    O, lse = attn_tilemix(P, b, h, rows)
    sub16 = 0.0 if dtype == "bf16" else ok.sum(axis=1) * 2.0 ** -25
    lse_tol = (E.max(axis=1, initial=0.0) + np.log1p(_sum16_rel(dtype)) + sub16
               + (P.n_kt + 64) * U32 + 4 * U32 * np.abs(np.where(none, 0.0, lse)))
    p = np.where(ok, np.exp(sf - m[:, None]), 0.0)
    eps = np.expm1(E)
    pe = p * eps
    vh = P.v[b, P.kvh(h)]
    l = p.sum(axis=1)
    dev2 = p @ (vh * vh) - 2.0 * O * (p @ vh) + O * O * l[:, None]
    num = np.sqrt((pe * eps).sum(axis=1))[:, None] * np.sqrt(np.maximum(dev2, 0.0))
    denom = np.maximum(l - pe.sum(axis=1), 1e-300)
    extra = np.where(none[:, None], 0.0, num / denom[:, None])
    return O, lse, lse_tol, extra


# ---------------------------------------------------------------------------
# LampAttention: tile-by-tile emulation
# ---------------------------------------------------------------------------

def exp8_of_code(codes):
    """p = E4M3(exp(val(code))) for e4m3 codes of non-positive logits."""
    return e4m3.round_to_e4m3(np.exp(e4m3.decode(codes)))


def exp8(x):
    """E4M3(exp(E4M3(x))) for x <= 0 (saturating at -448)."""
    return exp8_of_code(e4m3.encode(x))


@dataclass
class LampBranch:
    """One sequence of outcomes of a sub-block's adaptive flag decisions.

    A decision whose margin lies within the bound on the GPU's fp32 error is
    evaluated both ways; each leaf of that tree is one branch, identified by
    its flags (two branches differ in the flag of the tile where they split).
    """
    flags: np.ndarray             # [n_kt] bool: sub-block recomputed in 16-bit at key tile kt
    dontcare: np.ndarray          # [n_kt] bool: decision at kt within the error bound (split)
    margin: np.ndarray            # [n_kt] max(s8 - m') + tau of the decision (nan: none)
    bound: np.ndarray             # [n_kt] error bound of that margin
    O: np.ndarray                 # [r, D]
    lse: np.ndarray               # [r]
    extra_tol: np.ndarray         # [r, D] widening for what the weights may move by
    lse_tol: np.ndarray           # [r] bound on |LSE_gpu - LSE|
    counts: dict = field(default_factory=dict)


@dataclass
class LampResult:
    O: np.ndarray                 # [R, D] of the primary branch (the oracle's own decisions)
    lse: np.ndarray               # [R]
    flags: np.ndarray             # [n_sb, n_kt] bool, primary branch
    flag_dontcare: np.ndarray     # [n_sb, n_kt] bool, primary branch's decisions within the bound
    extra_tol: np.ndarray         # [R, D]
    lse_tol: np.ndarray           # [R]
    branches: list                # per sub-block (sorted order): [LampBranch], [0] = primary
    row_branch: list              # per sub-block: indices (into the R rows) of its rows
    unresolved: np.ndarray        # [n_sb] bool: more branches than the cap (the rest dropped)
    counts: dict = field(default_factory=dict)


def _err_logits(P, b, h, rows, cols, s, use16):
    """Bound on the GPU's fp32 error in each logit s (natural-log units).

    8-bit int8: the accumulator is exact; the scale product and the final
    multiply add at most 3 roundings -> 4u|s|.  16-bit: exact products summed
    in fp32 in any order -> gamma_D * sum|products| * scale (Higham, "Accuracy
    and Stability of Numerical Algorithms", 2nd ed., eq. (3.5)); 8-bit e4m3:
    the same plus the matrix cores' cut of each group's products
    (``_f8_cut_err``); plus 4u|s| for the scale roundings and the product.
    """
    D = P.D
    gam = D * U32 / (1 - D * U32)
    sm = P.sm_scale
    qa16, ka16 = np.abs(P.q[b, h][rows]), np.abs(P.k[b, P.kvh(h)][cols])
    e16 = gam * sm * (qa16 @ ka16.T)
    if P.code == "i8" or np.all(use16):
        e8 = np.zeros_like(s)
    else:
        sq = P.q_scales[b, h].astype(np.float64)[rows // P.tile_m]
        sk = P.k_scales[b, P.kvh(h)].astype(np.float64)[cols // P.tile_n]
        qv, kv = P.qv[b, h][rows], P.kv[b, P.kvh(h)][cols]
        e8 = (gam * (np.abs(qv) @ np.abs(kv).T) + _f8_cut_err(qv, kv)) \
            * sq[:, None] * sk[None, :] * sm
    return np.where(use16, e16, e8) + 4 * U32 * np.abs(s)


def _sum16_rel(dtype):
    """Relative rounding of one weight to the 16-bit P operand (half an ulp)."""
    return 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11


class _State:
    """Online-softmax state of a group of rows along one branch."""

    def __init__(self, R, D, n_kt):
        self.m = np.full(R, -np.inf)
        self.em = np.zeros(R)             # bound on |m_gpu - m_ref|
        self.l = np.zeros(R)
        self.acc = np.zeros((R, D))
        self.fp = np.zeros(R)             # sum of possible weight flips (alpha-scaled)
        # the flips one by one: rows, global keys, log of the weight change
        # minus the log of the rows' accumulated rescale (logc) at the tile
        self.fe_rows, self.fe_keys, self.fe_logw = [], [], []
        self.logc = np.zeros(R)
        # weights of measure mu (p for fp32 weights, the upper end of the
        # range for e4m3 ones) with relative error bounds eps: sums of
        # mu * eps, mu * eps^2, and the moments mu, mu v, mu v^2 of the V
        # rows they meet
        self.fq = np.zeros(R)
        self.qe2 = np.zeros(R)
        self.q0 = np.zeros(R)
        self.q1 = np.zeros((R, D))
        self.q2 = np.zeros((R, D))
        self.xerr = np.zeros(R)           # largest exponent error bound of an fp32 weight
        self.nvalid_row = np.zeros(R)
        self.flags = np.zeros(n_kt, dtype=bool)
        self.dontcare = np.zeros(n_kt, dtype=bool)
        self.margin = np.full(n_kt, np.nan)
        self.bound = np.full(n_kt, np.nan)
        self.counts = dict(n8=0, n16=0, nflag=0, nvalid=0)

    def copy(self):
        c = _State.__new__(_State)
        for k, v in self.__dict__.items():
            c.__dict__[k] = dict(v) if isinstance(v, dict) else v.copy()
        return c


def _lamp_group(P, b, h, rows, perturb, max_branches, dtype):
    """Branches of one group of rows (one sub-block in the adaptive mode,
    every requested row otherwise)."""
    R, D = len(rows), P.D
    vh = P.v[b, P.kvh(h)]
    vflip = P.v8[b, P.kvh(h)] if P.pv8 else vh   # the V rows an 8-bit weight meets
    r8_tiles = P.route8_tiles(b, h)
    qt = rows // P.tile_m
    states = [_State(R, D, P.n_kt)]
    unresolved = False
    for kt in range(P.n_kt):
        cols = np.arange(kt * P.tile_n, min(P.S_k, (kt + 1) * P.tile_n))
        ok = P.valid(rows, cols, b)
        if not ok.any():
            continue
        r8 = r8_tiles[qt, kt][:, None] & ok             # valid and 8-bit routed
        s8 = logits8(P, b, h, rows, cols)
        s16 = logits16(P, b, h, rows, cols)
        e8 = _err_logits(P, b, h, rows, cols, s8, np.zeros(ok.shape, dtype=bool))
        e16 = _err_logits(P, b, h, rows, cols, s16, np.ones(ok.shape, dtype=bool))
        if perturb is not None:
            s8 = s8 + perturb(e8)
            s16 = s16 + perturb(e16)
        has8 = r8.any(axis=1)
        nxt = []
        for st in states:
            outcomes, split = [False], False
            if P.adaptive and has8.any():
                rowmax8 = np.where(r8, s8, -np.inf).max(axis=1)
                mprime = np.maximum(st.m, rowmax8)
                with np.errstate(invalid="ignore"):
                    d_row = rowmax8 - mprime
                e_row = np.where(r8, e8, 0).max(axis=1) + st.em
                dmax = d_row[has8].max() + P.tau
                bnd = 2 * e_row[has8].max() + 4 * U32 * (abs(P.tau) + 1)
                flagged = bool(dmax >= 0)
                outcomes = [flagged]
                st.margin[kt], st.bound[kt] = dmax, bnd
                if abs(dmax) <= bnd:
                    outcomes, split = [flagged, not flagged], True
            for i, fl in enumerate(outcomes):
                c = st if i == len(outcomes) - 1 else st.copy()
                c.dontcare[kt] = split
                _lamp_tile(P, c, kt, cols, ok, r8, r8_tiles[qt, kt], s8, s16, e8, e16, fl,
                           vh, b, h)
                nxt.append(c)
        if len(nxt) > max_branches:
            unresolved = True
            nxt = nxt[:max_branches]
        states = nxt

    u16 = _sum16_rel(dtype)
    branches = []
    for st in states:
        none = st.l == 0                 # rows with no valid key: O = 0, LSE = -inf
        l_safe = np.where(none, 1.0, st.l)
        O = st.acc / l_safe[:, None]
        with np.errstate(divide="ignore"):
            lse = np.where(none, -np.inf, st.m + np.log(l_safe))
        denom = np.maximum(l_safe - st.fp - st.fq, 1e-300)
        extra = (_flip_widening(st, O, vflip, R) + _rel_widening(st, O)) / denom[:, None]
        sub16 = 0.0 if dtype == "bf16" else st.nvalid_row * 2.0 ** -25
        # LSE = m + ln l: the GPU's m is off by at most em, an fp32 weight
        # by its exponent's error (xerr), the e4m3 weights by the flips
        # summed in fp (relative to l - fp); plus the 16-bit rounding of fp32
        # weights (exp8 weights are exact in 16 bits), fp16 subnormal
        # weights, and fp32 rounding of the sum and the log
        lse_tol = (st.em + st.xerr + np.log1p(st.fp / denom) + np.log1p(u16) + sub16
                   + 4 * U32 * np.abs(np.where(none, 0.0, lse)) + (P.n_kt + 64) * U32)
        branches.append(LampBranch(flags=st.flags, dontcare=st.dontcare, margin=st.margin,
                                   bound=st.bound, O=O, lse=lse,
                                   extra_tol=extra, lse_tol=lse_tol, counts=st.counts))
    return branches, unresolved


def _flip_widening(st, O, w, R, chunk=1 << 15):
    """Bound on |O_gpu - O| * (l - fp) from the e4m3 weights alone.

    Moving weight k by d_k changes the normalised output by exactly
    sum_k d_k (w_k - O) / (l + sum_k d_k), w_k the V row the weight meets;
    with |d_k| at most its flip range (rescaled to the final running
    maximum), the numerator is at most sum_k |d_k| |w_k - O|."""
    out = np.zeros((R, O.shape[1]))
    if not st.fe_rows:
        return out
    rows = np.concatenate(st.fe_rows)
    keys = np.concatenate(st.fe_keys)
    lw = np.concatenate(st.fe_logw)
    for i in range(0, rows.size, chunk):
        r, k = rows[i:i + chunk], keys[i:i + chunk]
        c = np.exp(lw[i:i + chunk] + st.logc[r])[:, None] * np.abs(w[k] - O[r])
        np.add.at(out, r, c)
    return out


def _rel_widening(st, O):
    """Bound on |O_gpu - O| * (l - changes) from the relative weight errors:
    by the same identity, sum_k mu_k eps_k |v_k - O|, at most
    sqrt(sum_k mu_k eps_k^2) * sqrt(sum_k mu_k (v_k - O)^2) (Cauchy-Schwarz),
    the second factor from the moments of the V rows the weights meet."""
    dev2 = st.q2 - 2.0 * O * st.q1 + O * O * st.q0[:, None]
    return np.sqrt(st.qe2)[:, None] * np.sqrt(np.maximum(dev2, 0.0))


def _lamp_tile(P, st, kt, cols, ok, r8, tile_is8, s8, s16, e8, e16, flag, vh, b, h):
    """Update one branch's state with key tile kt (flag: its sub-block is
    recomputed in 16-bit)."""
    use16 = np.broadcast_to((~tile_is8)[:, None] | flag, ok.shape)
    s = np.where(use16, s16, s8)
    es = np.where(use16, e16, e8)
    sv = np.where(ok, s, -np.inf)
    m_new = np.maximum(st.m, sv.max(axis=1))
    fin = np.isfinite(m_new)
    st.em = np.where(fin, np.maximum(st.em, np.where(ok, es, 0).max(axis=1)), st.em)
    with np.errstate(invalid="ignore"):
        x = np.where(ok, s - m_new[:, None], -np.inf)
    p16 = np.exp(x)
    if P.exp8:
        xc = np.maximum(np.where(ok, x, -448.0), -448.0)
        p8 = exp8(xc)
        ex = es + st.em[:, None] + 2 * U32 * (np.abs(xc) + np.abs(s))
        lo = exp8(np.maximum(xc - ex, -448.0))
        hi = exp8(np.minimum(xc + ex, 0.0))
        dp = np.where(ok & ~use16, hi - lo, 0.0)
        hi8 = np.where(ok & ~use16, hi, 0.0)
        fp32w = ok & use16
    else:
        p8 = p16
        dp = np.zeros(ok.shape)
        hi8 = np.zeros(ok.shape)
        fp32w = ok
    e32 = es + 2 * U32 * (np.abs(np.where(ok, x, 0)) + np.abs(s))
    st.xerr = np.maximum(st.xerr, np.where(fp32w, e32, 0).max(axis=1))
    p = np.where(ok, np.where(use16, p16, p8), 0.0)
    with np.errstate(invalid="ignore"):
        alpha = np.where(np.isfinite(st.m), np.exp(st.m - m_new), 0.0)
    alpha = np.where(fin, alpha, 1.0)
    # The GPU's weights, times the one constant exp(m_gpu - m) of their
    # final running maxima (which O does not see): an fp32 weight is p times
    # exp(its logit's error), at most p * eps with eps = expm1(e32); an e4m3
    # weight lies in [lo, hi] at the GPU's running maximum of this tile,
    # which is off by at most em, so in [lo e^-em, hi e^em]: the flip range
    # dp plus at most hi * expm1(em).  mu * eps bounds every such change.
    eps = np.where(fp32w, np.expm1(np.where(fp32w, e32, 0.0)), np.expm1(st.em)[:, None])
    pq = np.where(fp32w, p, 0.0)
    mu = pq + hi8
    vc = vh[cols]
    vc8 = P.v8[b, P.kvh(h)][cols] if P.pv8 else vc
    st.fq = alpha * st.fq + (mu * eps).sum(axis=1)
    st.qe2 = alpha * st.qe2 + (mu * eps * eps).sum(axis=1)
    st.q0 = alpha * st.q0 + mu.sum(axis=1)
    st.q1 = alpha[:, None] * st.q1 + pq @ vc + hi8 @ vc8
    st.q2 = alpha[:, None] * st.q2 + pq @ (vc * vc) + hi8 @ (vc8 * vc8)
    st.l = alpha * st.l + p.sum(axis=1)
    st.fp = alpha * st.fp + dp.sum(axis=1)
    st.logc = st.logc + np.where(alpha > 0, np.log(np.where(alpha > 0, alpha, 1.0)), 0.0)
    fr, fc = np.nonzero(dp)
    if fr.size:
        st.fe_rows.append(fr)
        st.fe_keys.append(cols[fc])
        st.fe_logw.append(np.log(dp[fr, fc]) - st.logc[fr])
    if P.pv8:
        # 8-bit weights meet the e4m3 V codes of their tile (products exact)
        p8v = np.where(use16, 0.0, p)
        st.acc = alpha[:, None] * st.acc + (p - p8v) @ vh[cols] + p8v @ P.v8[b, P.kvh(h)][cols]
    else:
        st.acc = alpha[:, None] * st.acc + p @ vh[cols]
    st.m = np.where(fin, m_new, st.m)
    st.nvalid_row += ok.sum(axis=1)
    st.flags[kt] = flag
    st.counts["n8"] += int(r8.sum())
    st.counts["n16"] += int((ok & ~np.broadcast_to(tile_is8[:, None], ok.shape)).sum())
    st.counts["nflag"] += int(r8.sum()) if flag else 0
    st.counts["nvalid"] += int(ok.sum())


def attn_lamp(P, b, h, sub_blocks, *, perturb=None, max_branches=64, dtype="bf16"):
    """Emulate the online softmax for the given sub-blocks (indices of
    sub_rows-row blocks of head (b, h)), key tiles in ascending order.

    In the adaptive mode every sub-block is emulated on its own, and a flag
    decision within the GPU error bound of the threshold is taken both ways
    (at most ``max_branches`` branches per sub-block).  ``perturb`` (tests
    only) maps the error bound of each logit to an offset added to it, to
    emulate a GPU within the bound.  ``dtype`` is the 16-bit type of the
    weights fed to P V (for the LSE bound).

    Returns (LampResult, rows, sorted sub-block indices)."""
    sr = P.sub_rows
    sub_blocks = np.asarray(sub_blocks, dtype=np.int64)
    rows = (sub_blocks[:, None] * sr + np.arange(sr)[None, :]).reshape(-1)
    rows = rows[rows < P.S_q]
    rows = np.unique(rows)
    sbid = rows // sr
    usb, sb_idx = np.unique(sbid, return_inverse=True)
    R, D = len(rows), P.D
    if P.adaptive:
        groups = [np.flatnonzero(sb_idx == i) for i in range(len(usb))]
    else:
        groups = [np.arange(R)]
    O = np.zeros((R, D))
    lse = np.zeros(R)
    extra = np.zeros((R, D))
    lse_tol = np.zeros(R)
    flags = np.zeros((len(usb), P.n_kt), dtype=bool)
    dontcare = np.zeros((len(usb), P.n_kt), dtype=bool)
    branches, row_branch = [], []
    unresolved = np.zeros(len(usb), dtype=bool)
    counts = dict(n8=0, n16=0, nflag=0, nvalid=0)
    for gi, idx in enumerate(groups):
        brs, unres = _lamp_group(P, b, h, rows[idx], perturb, max_branches, dtype)
        pr = brs[0]
        O[idx], lse[idx], extra[idx], lse_tol[idx] = pr.O, pr.lse, pr.extra_tol, pr.lse_tol
        for k in counts:
            counts[k] += pr.counts[k]
        if P.adaptive:
            flags[gi], dontcare[gi] = pr.flags, pr.dontcare
            branches.append(brs)
            row_branch.append(idx)
            unresolved[gi] = unres
        else:
            # one branch for all rows: split it per sub-block
            for i in range(len(usb)):
                sel = np.flatnonzero(sb_idx[idx] == i)
                branches.append([LampBranch(flags=pr.flags, dontcare=pr.dontcare, margin=pr.margin,
                                            bound=pr.bound, O=pr.O[sel],
                                            lse=pr.lse[sel], extra_tol=pr.extra_tol[sel],
                                            lse_tol=pr.lse_tol[sel], counts={})])
                row_branch.append(idx[sel])
    return LampResult(O=O, lse=lse, flags=flags, flag_dontcare=dontcare, extra_tol=extra,
                      lse_tol=lse_tol, branches=branches, row_branch=row_branch,
                      unresolved=unresolved, counts=counts), rows, usb


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
