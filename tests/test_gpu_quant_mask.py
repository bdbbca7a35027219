"""GPU parity: quantiser codes/scales and packed masks, bit-exact against the
oracle (through the C ABI binding)."""
import numpy as np
import pytest
import torch

from oracle import e4m3 as oe
from oracle import mask as omask
from oracle import quant as oq
from synthetic import CONFIGS, c5_variant, make_inputs

pytestmark = pytest.mark.gpu


def L():
    import mixed_precision_tiled_amd as lamp
    return lamp


def dev():
    return torch.device("cuda:0")


def gpu_quant(x, rows, code):
    c, s = L().lamp_quantize_blocks(x.to(dev()), rows, code)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def assert_quant_equal(x, rows, code):
    gc, gs = gpu_quant(x, rows, code)
    oc, os_ = oq.quantize_blocks(x.float().numpy(), rows, code)
    assert (gs == os_).all(), f"scales differ at {np.argwhere(gs != os_)[:5]}"
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5]}: gpu {gc[tuple(bad[0])]} oracle {oc[tuple(bad[0])]}"


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_quant_configs_full(name):
    cfg = CONFIGS[name]
    q, k, _ = make_inputs(cfg)
    print(f"[quant] {name} Q{tuple(q.shape)} K{tuple(k.shape)} {cfg.code}", flush=True)
    assert_quant_equal(q, cfg.tile_m, cfg.code)
    assert_quant_equal(k, cfg.tile_n, cfg.code)


@pytest.mark.parametrize("name,code", [("C4", "i8"), ("C5", "i8"), ("C5", "e4m3")])
def test_quant_configs_large_sampled_heads(name, code):
    cfg = CONFIGS[name] if name == "C4" else c5_variant(0.25, code)
    q, k, _ = make_inputs(cfg)
    print(f"[quant] {cfg.name} Q{tuple(q.shape)} {code}", flush=True)
    gq, gqs = gpu_quant(q, cfg.tile_m, code)
    gk, gks = gpu_quant(k, cfg.tile_n, code)
    for b, h in [(0, 0), (cfg.B - 1, cfg.Hq - 1), (0, 13)]:
        oc, os_ = oq.quantize_blocks(q[b:b + 1, h:h + 1].float().numpy(), cfg.tile_m, code)
        assert (gq[b:b + 1, h:h + 1] == oc).all() and (gqs[b:b + 1, h:h + 1] == os_).all()
    for b, h in [(0, 0), (cfg.B - 1, cfg.Hkv - 1)]:
        oc, os_ = oq.quantize_blocks(k[b:b + 1, h:h + 1].float().numpy(), cfg.tile_n, code)
        assert (gk[b:b + 1, h:h + 1] == oc).all() and (gks[b:b + 1, h:h + 1] == os_).all()


def crafted_e4m3_rows():
    """Values at which RNE to e4m3 must pick the even neighbour, exact e4m3
    values, tiny negatives (signed zero), with block absmax 448 so that
    inv = 1 and y = x exactly."""
    mags = oe.decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = 0.5 * (mags[1:] + mags[:-1])
    vals = np.concatenate([mids, -mids, mags, -mags, [-2.0 ** -12, -2.0 ** -11, 2.0 ** -11,
                                                      -3 * 2.0 ** -11, 448.0]])
    return vals


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_quant_e4m3_rounding_midpoints(dtype):
    vals = crafted_e4m3_rows()
    t = torch.tensor(vals, dtype=torch.float64).to(dtype)
    # keep only the values the 16-bit dtype represents exactly
    keep = t.double().numpy() == vals
    vals = vals[keep]
    n = len(vals)
    D = 64
    per = D - 1                      # last column holds the block absmax
    rows = -(-n // per)
    flat = np.zeros(rows * per)
    flat[:n] = vals
    x = np.zeros((rows, D))
    x[:, :per] = flat.reshape(rows, per)
    x[:, -1] = 448.0                 # every row has absmax 448 -> inv = 1, y = x
    xt = torch.from_numpy(x.reshape(1, 1, rows, D)).to(dtype)
    assert_quant_equal(xt, 1, "e4m3")
    assert_quant_equal(xt, rows, "e4m3")
    gc, _ = gpu_quant(xt, 1, "e4m3")
    got = gc.reshape(rows, D)[:, :per].reshape(-1)[:n]
    assert (got == oe.encode(vals)).all()


def test_quant_int8_half_integers():
    vals = np.arange(-126.5, 127.0, 1.0)           # k + 0.5: RNE picks the even k
    D = 128
    per = D - 1                                     # last column holds the absmax 127
    rows = -(-len(vals) // per)
    flat = np.zeros(rows * per)
    flat[:len(vals)] = vals
    x = np.zeros((rows, D))
    x[:, :per] = flat.reshape(rows, per)
    x[:, -1] = 127.0                                # absmax 127 -> inv = 1, y = x
    xt = torch.from_numpy(x.reshape(1, 1, rows, D)).to(torch.bfloat16)
    assert_quant_equal(xt, 1, "i8")
    gc, _ = gpu_quant(xt, 1, "i8")
    got = gc.reshape(rows, D)[:, :per].reshape(-1)[:len(vals)].view(np.int8).astype(int)
    assert (got == np.rint(vals)).all()


@pytest.mark.parametrize("code", ["i8", "e4m3"])
@pytest.mark.parametrize("D,rows", [(64, 64), (128, 128), (256, 64), (128, 37)])
def test_quant_ragged_strided_zero(code, D, rows):
    g = torch.Generator().manual_seed(D + rows)
    big = torch.randn(2, 5, 300, D + 64, generator=g) * 3
    big[1, 2, 64:128] = 0.0                           # an all-zero block (rows = 64)
    big = big.to(torch.bfloat16)
    xd = big.to(dev())[:, 1:4, :200, :D]              # strided view on the device
    assert xd.stride(2) == D + 64 and not xd.is_contiguous()
    c, s = L().lamp_quantize_blocks(xd, rows, code)
    torch.cuda.synchronize()
    oc, os_ = oq.quantize_blocks(big[:, 1:4, :200, :D].float().numpy(), rows, code)
    assert (c.cpu().numpy() == oc).all() and (s.cpu().numpy() == os_).all()


def test_quant_empty():
    x = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=dev())
    c, s = L().lamp_quantize_blocks(x, 64, "i8")
    assert c.numel() == 0 and s.numel() == 0


@pytest.mark.parametrize("shape", [
    (1, 1, 256, 256, 64, 64, 1, 0.5, 2001),
    (1, 32, 4096, 4096, 128, 64, 4, 0.25, 2002),
    (1, 16, 8192, 8192, 128, 64, 1, 0.0, 2003),
    (1, 32, 32768, 32768, 128, 64, 8, 0.10, 2004),
    (2, 32, 16384, 16384, 128, 64, 4, 0.0, 2005),
    (2, 32, 16384, 16384, 128, 64, 4, 0.10, 2015),
    (2, 32, 16384, 16384, 128, 64, 4, 0.50, 2055),
    (2, 32, 16384, 16384, 128, 64, 4, 1.0, 2105),
    (3, 5, 1000, 777, 64, 64, 3, 0.37, 99),
    (1, 2, 4096, 70000, 128, 64, 1, 0.3, 7),
])
def test_mask_bit_exact(shape):
    B, Hq, S_q, S_k, tm, tn, G, f16, seed = shape
    n_g = -(-(-(-S_k // tn)) // G)
    W = max(1, -(-n_g // 64))
    for w in (W, W + 1):
        m = L().lamp_build_mask(B, Hq, S_q, S_k, tm, tn, G, f16, seed, w, device=dev())
        torch.cuda.synchronize()
        ref = omask.build_mask(B, Hq, S_q, S_k, tm, tn, G, f16, seed, w)
        assert (m.cpu().numpy().view(np.uint64) == ref).all()


@pytest.mark.parametrize("shape", [
    (1, 4, 512, 512, 64, 64, 1, [0.0, 0.3, 0.7, 1.0], 31),
    (2, 32, 16384, 16384, 128, 64, 4, [0.05 * (h % 8) for h in range(32)], 2025),
    (1, 3, 8192, 8192, 128, 64, 1, [0.2, 0.5, 0.25], 41),        # two words
])
def test_mask_per_head_bit_exact(shape):
    B, Hq, S_q, S_k, tm, tn, G, fr, seed = shape
    n_g = -(-(-(-S_k // tn)) // G)
    W = max(1, -(-n_g // 64))
    m = L().lamp_build_mask_per_head(B, Hq, S_q, S_k, tm, tn, G, fr, seed, W, device=dev())
    torch.cuda.synchronize()
    ref = omask.build_mask(B, Hq, S_q, S_k, tm, tn, G, fr, seed, W)
    assert (m.cpu().numpy().view(np.uint64) == ref).all()


@pytest.mark.parametrize("shape", [
    (1, 1, 512, 512, 64, 64, 1, 1, 2, 3),
    (2, 32, 16384, 16384, 128, 64, 4, 1, 2, 8),
    (1, 4, 8192, 8192, 128, 64, 1, 2, 3, 16),      # 128 groups: two words
    (3, 5, 1000, 777, 64, 64, 3, 0, 1, 0),
    (1, 2, 4096, 70000, 128, 64, 1, 4, 5, 33),     # keys beyond the queries
    (1, 1, 70000, 4096, 128, 64, 2, 0, 3, 5),      # queries beyond the keys
    (1, 3, 2048, 2048, 128, 64, 4, 0, 0, 0),       # no template part: all 8-bit
])
def test_mask_template_bit_exact(shape):
    B, Hq, S_q, S_k, tm, tn, G, sink, band, stride = shape
    n_g = -(-(-(-S_k // tn)) // G)
    W = max(1, -(-n_g // 64))
    for w in (W, W + 1):
        m = L().lamp_build_mask_template(B, Hq, S_q, S_k, tm, tn, G, sink, band, stride, w,
                                         device=dev())
        torch.cuda.synchronize()
        ref = omask.build_mask_template(B, Hq, S_q, S_k, tm, tn, G, sink, band, stride, w)
        assert (m.cpu().numpy().view(np.uint64) == ref).all()


# ---------------------------------------------------------------------------
# V tiles for the 8-bit P V product
# ---------------------------------------------------------------------------

def assert_v_tiles_equal(v, seqlens=None):
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device=dev())
    gc, gs = L().lamp_quantize_v_tiles(v.to(dev()), seqlens=sl)
    torch.cuda.synchronize()
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    oc, os_ = oq.quantize_v_tiles(v.float().numpy(), 64, seqlens)
    assert (gs == os_).all(), f"scales differ at {np.argwhere(gs != os_)[:5]}"
    packed = oq.pack_v_tiles(oc)
    bad = np.argwhere(gc != packed)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5]}"


@pytest.mark.parametrize("D,S,dtype,scale", [
    (64, 200, torch.bfloat16, 1.0), (128, 320, torch.float16, 3.0), (256, 130, torch.bfloat16, 0.01),
    (128, 64, torch.bfloat16, 1e4), (128, 1, torch.float16, 1.0)])
def test_quant_v_tiles(D, S, dtype, scale):
    g = torch.Generator().manual_seed(D + S)
    v = (torch.randn(2, 3, S, D, generator=g) * scale).to(dtype)
    v[1, 2, :40] = 0.0                                # an all-zero first tile (S >= 64 cases)
    print(f"[quant v] D{D} S{S} {dtype} x{scale}", flush=True)
    assert_v_tiles_equal(v)


def test_quant_v_tiles_strided_and_varlen():
    g = torch.Generator().manual_seed(5)
    base = torch.randn(2, 300, 4, 128, generator=g).to(torch.bfloat16)
    v = base.transpose(1, 2)                           # [2, 4, 300, 128], non-contiguous
    print("[quant v] strided, varlen", flush=True)
    assert_v_tiles_equal(v)
    assert_v_tiles_equal(v, seqlens=[300, 97])
    assert_v_tiles_equal(v, seqlens=[0, 64])


def test_quant_v_tiles_rounding_midpoints():
    # block absmax 448 -> scale 1, so the codes are the e4m3 rounding of the
    # values themselves: midpoints must go to the even code
    vals = crafted_e4m3_rows()
    t = torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16)
    vals = vals[t.double().numpy() == vals]
    n = len(vals) // 64 * 64
    v = torch.tensor(vals[:n], dtype=torch.float64).to(torch.bfloat16).reshape(1, 1, n // 64, 64)
    v = v.transpose(2, 3).contiguous()                 # [1, 1, 64, n/64]: pad D to 64
    v = torch.nn.functional.pad(v, (0, 64 - v.shape[-1]))
    v[0, 0, 0, 0] = 448.0
    print("[quant v] midpoints", flush=True)
    assert_v_tiles_equal(v)


def test_exp8_table_exhaustive():
    """The attention kernel's 8-bit exponential table against the oracle's
    E4M3(exp(value)) on all 128 codes of non-positive logits (+0 and
    0x80..0xFE); 0xFF, the conversion's code for logits below -464, -inf and
    NaN, must weigh what a logit clamped to -448 weighs (0)."""
    from oracle import attention as oa
    t = L().lamp_exp8_table(device=dev()).cpu().numpy()
    codes = np.array([0x00] + list(range(0x80, 0xFF)), np.uint8)
    got = oe.decode(t[codes])
    want = oa.exp8_of_code(codes)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(codes[i]), got[i], want[i]) for i in bad[:8]]
    assert t[0xFF] == 0 and oa.exp8(np.array([-1000.0, -np.inf]))[0] == 0.0
    assert int((got > 0).sum()) == 79
