"""ctypes binding of liblamp.so (see include/lamp.h).

Argument marshalling only: tensors are turned into device pointers, sizes
and strides, outputs are allocated with torch when the caller passes none,
and every call goes to the HIP library on torch's current stream.  There is
no other implementation behind these functions: if the library is missing
the import fails.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblamp.so")

LAMP_OK, LAMP_ERR_NULL, LAMP_ERR_SHAPE, LAMP_ERR_UNSUPPORTED, LAMP_ERR_ALIGN, LAMP_ERR_HIP = range(6)
LAMP_F16, LAMP_BF16, LAMP_I8, LAMP_E4M3 = range(4)
LAMP_MODE_MASK, LAMP_MODE_ADAPTIVE = 0, 1

_DT16 = {torch.float16: LAMP_F16, torch.bfloat16: LAMP_BF16}
_CODE = {"i8": LAMP_I8, "e4m3": LAMP_E4M3, LAMP_I8: LAMP_I8, LAMP_E4M3: LAMP_E4M3}


class LampError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


def library_path():
    return _LIB_PATH


if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                      f"g.build()'` (hipcc, gfx950) first")
_lib = ctypes.CDLL(_LIB_PATH)

_i64, _i32, _u32, _u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
_vp, _fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)


class lamp_attn_params(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("mode", _i32), ("causal", _i32), ("sm_scale", ctypes.c_float),
        ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("S_q", _i64), ("S_k", _i64), ("D", _i64),
        ("q", _vp), ("k", _vp), ("v", _vp), ("in_dtype", _i32), ("code_dtype", _i32),
        ("q_str", _i64 * 3), ("k_str", _i64 * 3), ("v_str", _i64 * 3), ("o_str", _i64 * 3),
        ("q8", _vp), ("k8", _vp), ("q_scale", _vp), ("k_scale", _vp), ("mask", _vp),
        ("words_per_row", _i32), ("tile_m", _i32), ("tile_n", _i32), ("tiles_per_bit", _i32),
        ("exp8", _i32), ("tau", ctypes.c_float), ("sub_rows", _i32),
        ("out", _vp), ("lse", _vp), ("flags_out", _vp), ("dbg_qk_acc", _vp),
        ("seqlens_q", _vp), ("seqlens_k", _vp),
        ("pv8", _i32), ("v8", _vp), ("v_scale", _vp),
    ]


_lib.lamp_quantize_blocks.restype = _i32
_lib.lamp_quantize_blocks.argtypes = [_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32,
                                      _i32, _vp, _vp, _vp]
_lib.lamp_quantize_blocks_varlen.restype = _i32
_lib.lamp_quantize_blocks_varlen.argtypes = [_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                             _vp, _i32, _i32, _vp, _vp, _vp]
_lib.lamp_quantize_v_tiles.restype = _i32
_lib.lamp_quantize_v_tiles.argtypes = [_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp,
                                       _vp, _vp, _vp]
_lib.lamp_build_mask.restype = _i32
_lib.lamp_build_mask.argtypes = [_i64, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_double, _u64,
                                 _vp, _i32, _vp]
_lib.lamp_build_mask_per_head.restype = _i32
_lib.lamp_build_mask_per_head.argtypes = [_i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                          ctypes.POINTER(ctypes.c_double), _u64, _vp, _i32, _vp]
_lib.lamp_attn_fwd.restype = _i32
_lib.lamp_build_mask_template.restype = _i32
_lib.lamp_build_mask_template.argtypes = [_i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _vp, _i32, _vp]
_lib.lamp_attn_fwd.argtypes = [ctypes.POINTER(lamp_attn_params), _vp]
_lib.lamp_exp8_table.restype = _i32
_lib.lamp_exp8_table.argtypes = [_vp, _vp]
_lib.lamp_status_string.restype = ctypes.c_char_p
_lib.lamp_status_string.argtypes = [_i32]
_lib.lamp_last_error.restype = ctypes.c_char_p
_lib.lamp_last_error.argtypes = []
_lib.lamp_abi_version.restype = _i32
_lib.lamp_abi_version.argtypes = []


def _status_name(s):
    return _lib.lamp_status_string(s).decode()


def lamp_status_string(s):
    return _status_name(s)


def lamp_last_error():
    return _lib.lamp_last_error().decode()


def lamp_abi_version():
    return int(_lib.lamp_abi_version())


def exported_symbols(names):
    """The subset of ``names`` that the loaded library exports."""
    out = []
    for n in names:
        try:
            getattr(_lib, n)
            out.append(n)
        except AttributeError:
            pass
    return out


def _check(status):
    if status != LAMP_OK:
        raise LampError(status, lamp_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _strides3(t):
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    return (_i64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def cdiv(a, b):
    return -(-a // b)


def lamp_quantize_blocks(x, block_rows, code, codes=None, scales=None, seqlens=None):
    """Per-block quantisation of x [B, H, S, D] (fp16/bf16 CUDA tensor).

    Returns (codes uint8 [B, H, S, D], scales float32 [B, H, ceil(S/block_rows)]).
    seqlens: optional int32 tensor [B] (variable-length batch; rows past a
    sequence's length are padding, quantised as zeros).
    """
    B, H, S, D = x.shape
    nb = cdiv(S, block_rows)
    if codes is None:
        codes = torch.empty((B, H, S, D), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    if x.dtype not in _DT16:
        raise TypeError("x must be float16 or bfloat16")
    if x.stride(3) != 1 or not codes.is_contiguous() or not scales.is_contiguous():
        raise ValueError("x needs a contiguous head dim; codes and scales must be contiguous")
    if seqlens is not None and (seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,)
                                or not seqlens.is_contiguous()):
        raise ValueError("seqlens must be a contiguous int32 tensor [B]")
    _check(_lib.lamp_quantize_blocks_varlen(_ptr(x), _DT16[x.dtype], B, H, S, D, x.stride(0),
                                            x.stride(1), x.stride(2), _ptr(seqlens), block_rows,
                                            _CODE[code], _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def lamp_quantize_v_tiles(v, codes=None, scales=None, seqlens=None):
    """V [B, H, S, D] (fp16/bf16 CUDA tensor) as e4m3 codes for the 8-bit P V
    product.  Returns (codes uint8 [B, H, ceil(S/64), D, 64] tile-packed,
    scales float32 [B, H, ceil(S/64)], each a power of two)."""
    B, H, S, D = v.shape
    nt = cdiv(S, 64)
    if codes is None:
        codes = torch.empty((B, H, nt, D, 64), dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty((B, H, nt), dtype=torch.float32, device=v.device)
    if v.dtype not in _DT16:
        raise TypeError("v must be float16 or bfloat16")
    if v.stride(3) != 1 or not codes.is_contiguous() or not scales.is_contiguous():
        raise ValueError("v needs a contiguous head dim; codes and scales must be contiguous")
    if seqlens is not None and (seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,)
                                or not seqlens.is_contiguous()):
        raise ValueError("seqlens must be a contiguous int32 tensor [B]")
    _check(_lib.lamp_quantize_v_tiles(_ptr(v), _DT16[v.dtype], B, H, S, D, v.stride(0), v.stride(1),
                                      v.stride(2), _ptr(seqlens), _ptr(codes), _ptr(scales),
                                      _stream(v)))
    return codes, scales


def lamp_build_mask(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, seed,
                    words_per_row=None, mask=None, device="cuda"):
    """Random packed mask, int64 tensor [B, Hq, n_qt, W] holding the uint64 words."""
    n_qt = cdiv(S_q, tile_m)
    n_g = cdiv(cdiv(S_k, tile_n), tiles_per_bit)
    W = words_per_row or max(1, cdiv(n_g, 64))
    if mask is None:
        mask = torch.empty((B, Hq, n_qt, W), dtype=torch.int64, device=device)
    if not mask.is_contiguous():
        raise ValueError("mask must be contiguous")
    _check(_lib.lamp_build_mask(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, float(frac_16bit),
                                seed & ((1 << 64) - 1), _ptr(mask), W, _stream(mask)))
    return mask


def lamp_build_mask_per_head(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, seed,
                             words_per_row=None, mask=None, device="cuda"):
    """Random packed mask with one 16-bit fraction per query head
    (frac_16bit: Hq floats), int64 tensor [B, Hq, n_qt, W]."""
    n_qt = cdiv(S_q, tile_m)
    n_g = cdiv(cdiv(S_k, tile_n), tiles_per_bit)
    W = words_per_row or max(1, cdiv(n_g, 64))
    fr = [float(x) for x in frac_16bit]
    if len(fr) != Hq:
        raise ValueError("one fraction per query head")
    if mask is None:
        mask = torch.empty((B, Hq, n_qt, W), dtype=torch.int64, device=device)
    if not mask.is_contiguous():
        raise ValueError("mask must be contiguous")
    arr = (ctypes.c_double * max(1, Hq))(*fr)
    _check(_lib.lamp_build_mask_per_head(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, arr,
                                         seed & ((1 << 64) - 1), _ptr(mask), W, _stream(mask)))
    return mask


def lamp_build_mask_template(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, sink_groups,
                             band_groups, stride_groups, words_per_row=None, mask=None,
                             device="cuda"):
    """Structured static packed mask (sink groups, local band, strided
    groups), int64 tensor [B, Hq, n_qt, W] holding the uint64 words."""
    n_qt = cdiv(S_q, tile_m)
    n_g = cdiv(cdiv(S_k, tile_n), tiles_per_bit)
    W = words_per_row or max(1, cdiv(n_g, 64))
    if mask is None:
        mask = torch.empty((B, Hq, n_qt, W), dtype=torch.int64, device=device)
    if not mask.is_contiguous():
        raise ValueError("mask must be contiguous")
    _check(_lib.lamp_build_mask_template(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit,
                                         sink_groups, band_groups, stride_groups, _ptr(mask), W,
                                         _stream(mask)))
    return mask


def lamp_exp8_table(device="cuda"):
    """The attention kernel's 8-bit exponential of every e4m3 code: uint8
    tensor [256] on `device` (entry 0xFF is 0)."""
    table = torch.empty((256,), dtype=torch.uint8, device=device)
    _check(_lib.lamp_exp8_table(_ptr(table), _stream(table)))
    return table


def lamp_attn_fwd(q, k, v, q8, k8, q_scale, k_scale, mask, *, code, causal, tile_m,
                  tiles_per_bit, tile_n=64, words_per_row=None, mode=LAMP_MODE_MASK, exp8=False,
                  tau=4.0, sub_rows=32, sm_scale=0.0, out=None, lse=None, flags_out=None,
                  dbg_qk_acc=None, seqlens_q=None, seqlens_k=None, v8=None, v_scale=None):
    """Dual-path attention forward.  q [B,Hq,S_q,D], k/v [B,Hkv,S_k,D] 16-bit,
    q8/k8 codes and q_scale/k_scale from lamp_quantize_blocks, mask from
    lamp_build_mask.  Returns out [B,Hq,S_q,D] (q's dtype).  seqlens_q /
    seqlens_k: optional int32 tensors [B] of a variable-length batch.
    v8 / v_scale (from lamp_quantize_v_tiles) select the 8-bit P V product
    on 8-bit tiles (with exp8 and mask routing)."""
    B, Hq, S_q, D = q.shape
    _, Hkv, S_k, _ = k.shape
    if q.dtype not in _DT16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share float16 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, S_q, D), dtype=q.dtype, device=q.device)
    W = words_per_row or mask.shape[-1]
    if (v8 is None) != (v_scale is None):
        raise ValueError("v8 and v_scale go together")
    for t in (q8, k8, q_scale, k_scale, mask, lse, flags_out, dbg_qk_acc, seqlens_q, seqlens_k,
              v8, v_scale):
        if t is not None and not t.is_contiguous():
            raise ValueError("codes, scales, mask and optional outputs must be contiguous")
    for t in (seqlens_q, seqlens_k):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B,)):
            raise ValueError("seqlens must be int32 tensors [B]")
    # shapes and dtypes of everything the kernel reads or writes (a
    # mismatch would read or write out of bounds on the device)
    n_qt, n_kt = cdiv(S_q, tile_m), cdiv(S_k, tile_n)

    def need(name, t, shape, dtypes):
        if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes:
            raise ValueError(f"{name}: expected shape {tuple(shape)} and dtype in "
                             f"{[str(d) for d in dtypes]}, got {tuple(t.shape)} {t.dtype}")
    codes = (torch.uint8, torch.int8)
    need("q8", q8, (B, Hq, S_q, D), codes)
    need("k8", k8, (B, Hkv, S_k, D), codes)
    need("out", out, (B, Hq, S_q, D), (q.dtype,))
    if tile_m in (64, 128) and tile_n == 64:
        # (other tilings are refused by the library before any launch)
        need("q_scale", q_scale, (B, Hq, n_qt), (torch.float32,))
        need("k_scale", k_scale, (B, Hkv, n_kt), (torch.float32,))
        need("mask", mask, (B, Hq, n_qt, W), (torch.int64, torch.uint64))
    if lse is not None:
        need("lse", lse, (B, Hq, S_q), (torch.float32,))
    if flags_out is not None:
        need("flags_out", flags_out, flags_shape(B, Hq, S_q, S_k, tile_n, sub_rows),
             (torch.int64, torch.uint64))
    if dbg_qk_acc is not None:
        need("dbg_qk_acc", dbg_qk_acc, (B, Hq, S_q, S_k), (torch.int32,))
    if v8 is not None:
        need("v8", v8, (B, Hkv, n_kt, D, 64), codes)
        need("v_scale", v_scale, (B, Hkv, n_kt), (torch.float32,))
    p = lamp_attn_params()
    p.struct_size = ctypes.sizeof(lamp_attn_params)
    p.mode = mode
    p.causal = int(bool(causal))
    p.sm_scale = sm_scale
    p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = B, Hq, Hkv, S_q, S_k, D
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    p.in_dtype = _DT16[q.dtype]
    p.code_dtype = _CODE[code]
    p.q_str, p.k_str, p.v_str, p.o_str = _strides3(q), _strides3(k), _strides3(v), _strides3(out)
    p.q8, p.k8 = q8.data_ptr(), k8.data_ptr()
    p.q_scale, p.k_scale = q_scale.data_ptr(), k_scale.data_ptr()
    p.mask = mask.data_ptr()
    p.words_per_row = W
    p.tile_m, p.tile_n, p.tiles_per_bit = tile_m, tile_n, tiles_per_bit
    p.exp8 = int(bool(exp8))
    p.tau = tau
    p.sub_rows = sub_rows
    p.out = out.data_ptr()
    p.lse = None if lse is None else lse.data_ptr()
    p.flags_out = None if flags_out is None else flags_out.data_ptr()
    p.dbg_qk_acc = None if dbg_qk_acc is None else dbg_qk_acc.data_ptr()
    p.seqlens_q = None if seqlens_q is None else seqlens_q.data_ptr()
    p.seqlens_k = None if seqlens_k is None else seqlens_k.data_ptr()
    p.pv8 = int(v8 is not None)
    p.v8 = None if v8 is None else v8.data_ptr()
    p.v_scale = None if v_scale is None else v_scale.data_ptr()
    _check(_lib.lamp_attn_fwd(ctypes.byref(p), _stream(q)))
    return out


class lamp_decode_params(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("causal", _i32), ("sm_scale", ctypes.c_float), ("out_dtype", _i32),
        ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("S_q", _i64), ("S_k", _i64), ("D", _i64),
        ("q8", _vp), ("q_scale", _vp), ("tile_m", _i32), ("k8", _vp), ("k_scale", _vp),
        ("v8", _vp), ("v_scale", _vp), ("out", _vp), ("o_str", _i64 * 3), ("lse", _vp),
    ]


_lib.lamp_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.lamp_decode_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
_lib.lamp_decode_fwd.restype = _i32
_lib.lamp_decode_fwd.argtypes = [ctypes.POINTER(lamp_decode_params), _vp, ctypes.c_size_t, _vp]


def lamp_decode_workspace_bytes(B, Hkv, S_k, D):
    return int(_lib.lamp_decode_workspace_bytes(B, Hkv, S_k, D))


def lamp_decode_fwd(q8, q_scale, k8, k_scale, v8, v_scale, *, causal, tile_m, dtype,
                    sm_scale=0.0, out=None, lse=None, workspace=None):
    """Attention of q8 [B,Hq,S_q,D] over the int8 cache k8/v8 [B,Hkv,S_k,D]
    (codes and scales from lamp_quantize_blocks; K/V in 64-key blocks).
    Returns out [B,Hq,S_q,D] of torch dtype `dtype` (float16/bfloat16)."""
    B, Hq, S_q, D = q8.shape
    _, Hkv, S_k, _ = k8.shape
    if dtype not in _DT16:
        raise TypeError("dtype must be float16 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, S_q, D), dtype=dtype, device=q8.device)
    need = lamp_decode_workspace_bytes(B, Hkv, S_k, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q8.device)
    for t in (q8, q_scale, k8, k_scale, v8, v_scale, lse, workspace):
        if t is not None and not t.is_contiguous():
            raise ValueError("codes, scales, lse and workspace must be contiguous")
    p = lamp_decode_params()
    p.struct_size = ctypes.sizeof(lamp_decode_params)
    p.causal = int(bool(causal))
    p.sm_scale = sm_scale
    p.out_dtype = _DT16[dtype]
    p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = B, Hq, Hkv, S_q, S_k, D
    p.q8, p.q_scale, p.tile_m = q8.data_ptr(), q_scale.data_ptr(), tile_m
    p.k8, p.k_scale, p.v8, p.v_scale = k8.data_ptr(), k_scale.data_ptr(), v8.data_ptr(), v_scale.data_ptr()
    p.out = out.data_ptr()
    p.o_str = _strides3(out)
    p.lse = None if lse is None else lse.data_ptr()
    _check(_lib.lamp_decode_fwd(ctypes.byref(p), _ptr(workspace), workspace.numel(), _stream(q8)))
    return out


_lib.lamp_decode_fwd_noalloc.restype = _i32
_lib.lamp_decode_fwd_noalloc.argtypes = [ctypes.POINTER(lamp_decode_params), _vp]
LAMP_DECODE_SCRATCH_BYTES = 32 << 20


def lamp_decode_fwd_noalloc(q8, q_scale, k8, k_scale, v8, v_scale, *, causal, tile_m, out,
                            sm_scale=0.0, lse=None):
    """lamp_decode_fwd with the split partials in the library's fixed
    per-GPU scratch: no device memory is allocated (``out`` is required)."""
    B, Hq, S_q, D = q8.shape
    _, Hkv, S_k, _ = k8.shape
    if out.dtype not in _DT16 or tuple(out.shape) != (B, Hq, S_q, D):
        raise ValueError("out must be float16/bfloat16 [B, Hq, S_q, D]")
    for t in (q8, q_scale, k8, k_scale, v8, v_scale, lse):
        if t is not None and not t.is_contiguous():
            raise ValueError("codes, scales and lse must be contiguous")
    p = lamp_decode_params()
    p.struct_size = ctypes.sizeof(lamp_decode_params)
    p.causal = int(bool(causal))
    p.sm_scale = sm_scale
    p.out_dtype = _DT16[out.dtype]
    p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = B, Hq, Hkv, S_q, S_k, D
    p.q8, p.q_scale, p.tile_m = q8.data_ptr(), q_scale.data_ptr(), tile_m
    p.k8, p.k_scale, p.v8, p.v_scale = k8.data_ptr(), k_scale.data_ptr(), v8.data_ptr(), v_scale.data_ptr()
    p.out = out.data_ptr()
    p.o_str = _strides3(out)
    p.lse = None if lse is None else lse.data_ptr()
    _check(_lib.lamp_decode_fwd_noalloc(ctypes.byref(p), _stream(q8)))
    return out


def flags_shape(B, Hq, S_q, S_k, tile_n=64, sub_rows=32):
    return (B, Hq, cdiv(S_q, sub_rows), max(1, cdiv(cdiv(S_k, tile_n), 64)))


def fa_flops(B, Hq, S, D, causal):
    f = 4.0 * B * Hq * S * S * D
    return f / 2 if causal else f


__all__ = [n for n in dir() if n.startswith("lamp_") or n.startswith("LAMP_")] + [
    "LampError", "library_path", "exported_symbols", "flags_shape", "fa_flops"]
