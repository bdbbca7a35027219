"""C ABI checks that need no GPU: the header is valid C99, the binding's
struct layout equals the C layout, the built library exports every function
the header declares, and argument validation rejects bad calls (nothing is
launched on those paths)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lamp.h")
LIB = os.path.join(ROOT, "mixed_precision_tiled_amd", "liblamp.so")


def build_module():
    """build.py loaded by path (importing the package needs a built library)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_lamp_build", os.path.join(ROOT, "mixed_precision_tiled_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="session")
def lamp():
    if not os.path.exists(LIB):
        build_module().build()
    import mixed_precision_tiled_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lamp_\w+)\s*\(", src, flags=re.M)))


def test_header_is_c99(tmp_path):
    c = tmp_path / "t.c"
    c.write_text('#include "lamp.h"\nint main(void){return (int)sizeof(lamp_attn_params) > 0 ? 0 : 1;}\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.dirname(HEADER), "-c", str(c), "-o", str(tmp_path / "t.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layout_matches_binding(tmp_path, lamp):
    from mixed_precision_tiled_amd.lamp import lamp_attn_params as P
    fields = [f[0] for f in P._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lamp.h"', "int main(void){",
             'printf("size %zu\\n", sizeof(lamp_attn_params));']
    for f in fields:
        lines.append(f'printf("{f} %zu\\n", offsetof(lamp_attn_params, {f}));')
    lines.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)],
                   check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(P)
    for f in fields:
        assert int(out[f]) == getattr(P, f).offset, f


def test_decode_struct_layout_matches_binding(tmp_path, lamp):
    from mixed_precision_tiled_amd.lamp import lamp_decode_params as P
    fields = [f[0] for f in P._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lamp.h"', "int main(void){",
             'printf("size %zu\\n", sizeof(lamp_decode_params));']
    for f in fields:
        lines.append(f'printf("{f} %zu\\n", offsetof(lamp_decode_params, {f}));')
    lines.append("return 0;}")
    c = tmp_path / "dlayout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "dlayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)],
                   check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(P)
    for f in fields:
        assert int(out[f]) == getattr(P, f).offset, f


def test_decode_validation(lamp):
    from mixed_precision_tiled_amd.lamp import lamp_decode_params as P
    f = _lib(lamp).lamp_decode_fwd
    ws = ctypes.c_void_p(1 << 20)

    def params(**kw):
        p = P()
        p.struct_size = ctypes.sizeof(P)
        p.causal, p.out_dtype = 1, 1
        p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = 1, 8, 2, 1, 1000, 128
        p.q8 = p.q_scale = p.k8 = p.k_scale = p.v8 = p.v_scale = p.out = 4096
        p.tile_m = 64
        p.o_str[:] = [8 * 128, 128, 128]
        for key, val in kw.items():
            setattr(p, key, val)
        return p
    need = lamp.lamp_decode_workspace_bytes(1, 2, 1000, 128)
    # splits of 8..32 tiles aiming at 1024 waves: 16 tiles x 2 KV heads -> 8-tile splits, 2 of them
    assert need == 1 * 2 * 2 * 32 * 130 * 4
    cases = [(dict(struct_size=4), 3), (dict(D=256), 3), (dict(out_dtype=2), 3), (dict(Hkv=3), 3),
             (dict(S_q=9), 3),                   # 4 heads x 9 rows > 32 columns
             (dict(causal=2), 2), (dict(S_q=2, S_k=1), 3), (dict(tile_m=0), 2),
             (dict(k8=None), 1), (dict(q8=4100), 4), (dict(out=4097), 4), (dict(B=-1), 2),
             (dict(B=0), 0), (dict(S_k=0, causal=0), 2)]
    for kw, st in cases:
        p = params(**kw)
        assert f(ctypes.byref(p), ws, need, None) == st, kw
    p = params()
    assert f(ctypes.byref(p), ws, need - 1, None) == 2            # workspace too small
    assert f(ctypes.byref(p), None, need, None) == 1
    assert f(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 8), need, None) == 4
    assert f(None, ws, need, None) == 1


def test_decode_noalloc_validation(lamp):
    # the entry point without a workspace validates like lamp_decode_fwd and
    # refuses sizes whose partials exceed its fixed scratch, before it looks
    # up the scratch or launches anything (no GPU needed here)
    from mixed_precision_tiled_amd.lamp import lamp_decode_params as P
    f = _lib(lamp).lamp_decode_fwd_noalloc

    def params(**kw):
        p = P()
        p.struct_size = ctypes.sizeof(P)
        p.causal, p.out_dtype = 1, 1
        p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = 1, 8, 2, 1, 1000, 128
        p.q8 = p.q_scale = p.k8 = p.k_scale = p.v8 = p.v_scale = p.out = 4096
        p.tile_m = 64
        p.o_str[:] = [8 * 128, 128, 128]
        for key, val in kw.items():
            setattr(p, key, val)
        return p
    cases = [(dict(struct_size=4), 3), (dict(D=256), 3), (dict(Hkv=3), 3), (dict(k8=None), 1),
             (dict(q8=4100), 4), (dict(B=-1), 2), (dict(B=0), 0),
             # 64 x 8 groups over 131072 keys: 545 MB of partials > 32 MiB
             (dict(B=64, Hq=8, Hkv=8, S_k=131072), 3)]
    assert lamp.lamp_decode_workspace_bytes(64, 8, 131072, 128) > lamp.LAMP_DECODE_SCRATCH_BYTES
    assert lamp.LAMP_DECODE_SCRATCH_BYTES == 32 << 20
    for kw, st in cases:
        assert f(ctypes.byref(params(**kw)), None) == st, kw
    assert "fixed scratch" in lamp.lamp_last_error()
    assert f(None, None) == 1


def test_library_exports_every_declared_symbol(lamp):
    names = declared_functions()
    assert set(names) >= {"lamp_quantize_blocks", "lamp_build_mask", "lamp_attn_fwd",
                          "lamp_status_string", "lamp_last_error", "lamp_abi_version"}
    assert lamp.exported_symbols(names) == names
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), n


def test_abi_version_and_status_strings(lamp):
    assert lamp.lamp_abi_version() == 3
    for i, n in enumerate(["LAMP_OK", "LAMP_ERR_NULL", "LAMP_ERR_SHAPE", "LAMP_ERR_UNSUPPORTED",
                           "LAMP_ERR_ALIGN", "LAMP_ERR_HIP"]):
        assert lamp.lamp_status_string(i) == n


def _lib(lamp):
    return lamp.lamp._lib


def test_quantize_validation(lamp):
    f = _lib(lamp).lamp_quantize_blocks
    p = ctypes.c_void_p(16)      # aligned non-null dummy; never dereferenced on error paths
    # unsupported head dim
    assert f(p, 1, 1, 1, 64, 96, 0, 0, 96, 64, 2, p, p, None) == 3
    assert "D=96" in lamp.lamp_last_error()
    # bad dtypes
    assert f(p, 2, 1, 1, 64, 128, 0, 0, 128, 64, 2, p, p, None) == 3
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, 64, 1, p, p, None) == 3
    # block_rows out of range
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, 0, 2, p, p, None) == 3
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, 257, 2, p, p, None) == 3
    # negative size / stride
    assert f(p, 1, -1, 1, 64, 128, 0, 0, 128, 64, 2, p, p, None) == 2
    assert f(p, 1, 1, 1, 64, 128, 0, 0, -128, 64, 2, p, p, None) == 2
    # null pointers
    assert f(None, 1, 1, 1, 64, 128, 0, 0, 128, 64, 2, p, p, None) == 1
    # alignment
    assert f(ctypes.c_void_p(18), 1, 1, 1, 64, 128, 0, 0, 128, 64, 2, p, p, None) == 4
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 132, 64, 2, p, p, None) == 4
    # row stride shorter than a row
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 64, 64, 2, p, p, None) == 2
    # empty problem: OK, nothing launched
    assert f(None, 1, 1, 1, 0, 128, 0, 0, 128, 64, 2, None, None, None) == 0


def test_mask_validation(lamp):
    f = _lib(lamp).lamp_build_mask
    p = ctypes.c_void_p(64)
    assert f(1, 1, 256, 256, 64, 64, 1, 1.5, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 1, -0.1, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 1, float("nan"), 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 0, 64, 1, 0.5, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 0, 0.5, 0, p, 1, None) == 2
    # 8192 keys / 64 = 128 groups need 2 words
    assert f(1, 1, 8192, 8192, 128, 64, 1, 0.5, 0, p, 1, None) == 3
    assert f(1, 1, 256, 256, 64, 64, 1, 0.5, 0, None, 1, None) == 1
    assert f(1, 1, 256, 256, 64, 64, 1, 0.5, 0, ctypes.c_void_p(65), 1, None) == 4
    assert f(0, 1, 256, 256, 64, 64, 1, 0.5, 0, None, 1, None) == 0


def test_mask_per_head_validation(lamp):
    f = _lib(lamp).lamp_build_mask_per_head
    p = ctypes.c_void_p(64)
    fr = (ctypes.c_double * 3)(0.1, 0.5, 1.0)
    bad = (ctypes.c_double * 3)(0.1, 1.5, 0.2)
    nan = (ctypes.c_double * 3)(0.1, float("nan"), 0.2)
    big = (ctypes.c_double * 129)(*([0.5] * 129))
    assert f(1, 3, 256, 256, 64, 64, 1, None, 0, p, 1, None) == 1
    assert f(1, 3, 256, 256, 64, 64, 1, bad, 0, p, 1, None) == 2
    assert f(1, 3, 256, 256, 64, 64, 1, nan, 0, p, 1, None) == 2
    assert "frac_16bit[1]" in lamp.lamp_last_error()
    assert f(1, 129, 256, 256, 64, 64, 1, big, 0, p, 1, None) == 3
    assert f(1, 3, 8192, 8192, 128, 64, 1, fr, 0, p, 1, None) == 3     # words_per_row
    assert f(1, 3, 256, 256, 64, 64, 1, fr, 0, None, 1, None) == 1
    assert f(1, 3, 256, 256, 64, 64, 1, fr, 0, ctypes.c_void_p(65), 1, None) == 4
    assert f(0, 3, 256, 256, 64, 64, 1, fr, 0, None, 1, None) == 0


def test_quantize_varlen_validation(lamp):
    f = _lib(lamp).lamp_quantize_blocks_varlen
    p = ctypes.c_void_p(16)
    # misaligned lengths pointer
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, ctypes.c_void_p(18), 64, 2, p, p, None) == 4
    # the dense checks still apply
    assert f(p, 1, 1, 1, 64, 96, 0, 0, 96, None, 64, 2, p, p, None) == 3
    assert f(None, 1, 1, 1, 64, 128, 0, 0, 128, p, 64, 2, p, p, None) == 1
    assert f(None, 1, 1, 1, 0, 128, 0, 0, 128, p, 64, 2, None, None, None) == 0


def test_quantize_v_tiles_validation(lamp):
    f = _lib(lamp).lamp_quantize_v_tiles
    p = ctypes.c_void_p(16)
    assert f(p, 1, 1, 1, 64, 96, 0, 0, 96, None, p, p, None) == 3           # D
    assert f(p, 2, 1, 1, 64, 128, 0, 0, 128, None, p, p, None) == 3         # v_dtype
    assert f(p, 1, -1, 1, 64, 128, 0, 0, 128, None, p, p, None) == 2        # negative size
    assert f(p, 1, 1, 1, 64, 128, 0, 0, -128, None, p, p, None) == 2        # negative stride
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 64, None, p, p, None) == 2          # stride < D
    assert f(None, 1, 1, 1, 64, 128, 0, 0, 128, None, p, p, None) == 1
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, None, p, None, None) == 1
    assert f(ctypes.c_void_p(18), 1, 1, 1, 64, 128, 0, 0, 128, None, p, p, None) == 4
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 132, None, p, p, None) == 4
    assert f(p, 1, 1, 1, 64, 128, 0, 0, 128, ctypes.c_void_p(18), p, p, None) == 4
    assert f(None, 1, 1, 1, 0, 128, 0, 0, 128, None, None, None, None) == 0


def test_mask_template_validation(lamp):
    f = _lib(lamp).lamp_build_mask_template
    p = ctypes.c_void_p(64)
    # negative template parameters
    assert f(1, 1, 256, 256, 64, 64, 1, -1, 2, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 1, 1, -2, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 1, 1, 2, -3, p, 1, None) == 2
    # tiles
    assert f(1, 1, 256, 256, 0, 64, 1, 1, 2, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 64, 0, 1, 2, 0, p, 1, None) == 2
    assert f(1, 1, 256, 256, 64, 1 << 20, 1 << 12, 1, 2, 0, p, 1, None) == 3
    # words, pointers, alignment, empty problem
    assert f(1, 1, 8192, 8192, 128, 64, 1, 1, 2, 0, p, 1, None) == 3
    assert f(1, 1, 256, 256, 64, 64, 1, 1, 2, 0, None, 1, None) == 1
    assert f(1, 1, 256, 256, 64, 64, 1, 1, 2, 0, ctypes.c_void_p(65), 1, None) == 4
    assert f(0, 1, 256, 256, 64, 64, 1, 1, 2, 0, None, 1, None) == 0


def _params(lamp, **kw):
    from mixed_precision_tiled_amd.lamp import lamp_attn_params as P
    p = P()
    p.struct_size = ctypes.sizeof(P)
    p.mode = 0
    p.causal = 1
    p.B, p.Hq, p.Hkv, p.S_q, p.S_k, p.D = 1, 4, 2, 256, 256, 128
    dummy = 4096
    p.q = p.k = p.v = p.q8 = p.k8 = p.q_scale = p.k_scale = p.mask = p.out = dummy
    p.in_dtype, p.code_dtype = 1, 2
    for s in ("q_str", "k_str", "v_str", "o_str"):
        getattr(p, s)[:] = [4 * 256 * 128, 256 * 128, 128]
    p.words_per_row = 1
    p.tile_m, p.tile_n, p.tiles_per_bit = 128, 64, 1
    p.exp8, p.tau, p.sub_rows = 0, 4.0, 32
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), 3),
    (dict(mode=2), 3),
    (dict(D=96), 3),
    (dict(tile_m=32), 3),
    (dict(tile_n=128), 3),
    (dict(Hkv=3), 3),
    (dict(Hkv=0), 3),
    (dict(S_k=200), 3),                          # causal needs S_q <= S_k
    (dict(in_dtype=2), 3),
    (dict(code_dtype=1), 3),
    (dict(mode=1, sub_rows=16), 3),
    (dict(mode=1, tau=float("nan")), 2),
    (dict(sm_scale=float("nan")), 2),
    (dict(tiles_per_bit=0), 2),
    (dict(B=-1), 2),
    (dict(exp8=2), 2),
    (dict(causal=5), 2),
    (dict(S_q=8192, S_k=8192), 3),               # 128 groups do not fit one word
    (dict(q=None), 1),
    (dict(mask=None), 1),
    (dict(out=None), 1),
    (dict(q=4100), 4),
    (dict(code_dtype=3, dbg_qk_acc=4096), 3),    # int32 dump exists on the int8 path only
    (dict(causal=0, S_k=0), 2),
    (dict(seqlens_q=4098), 4),                   # lengths need 4-byte alignment
    (dict(seqlens_k=4097), 4),
    (dict(pv8=2), 2),
    (dict(pv8=1, v8=4096, v_scale=4096), 3),     # 8-bit P V needs exp8
    (dict(pv8=1, exp8=1, mode=1, v8=4096, v_scale=4096), 3),   # and mask routing
    (dict(pv8=1, exp8=1), 1),                    # V codes and scales required
    (dict(pv8=1, exp8=1, v8=4100, v_scale=4096), 4),
    (dict(pv8=1, exp8=1, v8=4096, v_scale=4098), 4),
    (dict(S_q=0, S_k=0), 0),                     # empty: OK, nothing launched
    (dict(B=0), 0),
])
def test_attn_validation(lamp, kw, status):
    p = _params(lamp, **kw)
    st = _lib(lamp).lamp_attn_fwd(ctypes.byref(p), None)
    assert st == status, (kw, st, lamp.lamp_last_error())


def test_attn_validation_strides(lamp):
    p = _params(lamp)
    p.q_str[:] = [4 * 256 * 128, 256 * 128, 100]
    assert _lib(lamp).lamp_attn_fwd(ctypes.byref(p), None) == 2   # row stride < D
    p.q_str[:] = [4 * 256 * 132, 256 * 132, 132]
    assert _lib(lamp).lamp_attn_fwd(ctypes.byref(p), None) == 4   # not a multiple of 8


def test_build_flags():
    build = build_module()
    assert "--offload-arch=gfx950" in build.FLAGS
    i = build.FLAGS.index("-target-feature")
    assert build.FLAGS[i - 1] == "-Xclang" and build.FLAGS[i + 1:i + 3] == ["-Xclang", "-packed-fp32-ops"]


def test_bench_route_counts_match_oracle():
    import numpy as np
    import bench
    from oracle import attention as A
    from oracle import mask as omask
    for causal, S_q, S_k, tm, G, f16 in [(True, 300, 300, 128, 2, 0.3), (False, 200, 333, 64, 1, 0.5),
                                         (True, 512, 512, 64, 3, 0.0), (True, 256, 256, 128, 1, 1.0),
                                         (True, 200, 333, 128, 2, 0.4), (True, 1, 700, 64, 1, 0.5)]:
        rng = np.random.default_rng(S_q)
        q = rng.standard_normal((2, 3, S_q, 8))
        k = rng.standard_normal((2, 1, S_k, 8))
        P = A.make_problem(q, k, k, causal=causal, code="i8", tile_m=tm, tile_n=64,
                           tiles_per_bit=G, frac_16bit=f16, seed=5)
        c = bench.route_counts(P.mask_words, S_q, S_k, tm, 64, G, causal)
        ref = A.route_counts(P)
        assert (c["n8"], c["n16"], c["nvalid"], c["nflag"]) == (ref["n8"], ref["n16"], ref["nvalid"], 0)
    # variable-length batches
    for causal, S_q, S_k, Lq, Lk in [(True, 300, 300, [300, 17, 0], [300, 200, 5]),
                                     (False, 200, 333, [200, 64], [0, 333])]:
        rng = np.random.default_rng(S_k)
        q = rng.standard_normal((len(Lq), 2, S_q, 8))
        k = rng.standard_normal((len(Lq), 1, S_k, 8))
        P = A.make_problem(q, k, k, causal=causal, code="i8", tile_m=128, tile_n=64,
                           tiles_per_bit=2, frac_16bit=0.4, seed=9, seqlens_q=np.array(Lq),
                           seqlens_k=np.array(Lk))
        c = bench.route_counts(P.mask_words, S_q, S_k, 128, 64, 2, causal, seqlens_q=Lq,
                               seqlens_k=Lk)
        ref = A.route_counts(P)
        assert (c["n8"], c["n16"], c["nvalid"]) == (ref["n8"], ref["n16"], ref["nvalid"])
    # flagged-element count: sub-blocks of 32 rows x key tiles
    S = 256
    flags = np.zeros((1, 1, S // 32, 1), np.uint64)
    flags[0, 0, 3, 0] = np.uint64(0b111)          # sub-block 3 (rows 96..127) at key tiles 0, 1, 2
    mw = omask.build_mask(1, 1, S, S, 128, 64, 1, 0.0, 1, 1)
    c = bench.route_counts(mw, S, S, 128, 64, 1, True, flags)
    # tile 0: 32 x 64 valid; tile 1 (keys 64..127): row r sees r - 63 keys;
    # tile 2 (keys 128..191): nothing valid for rows below 128
    assert c["nflag"] == 32 * 64 + sum(r - 63 for r in range(96, 128)) + 0


def test_mfma_probe_library_loads():
    """The measurement harness's sustained-MFMA probe is built beside the
    library and exports its launcher; bad arguments are refused before any
    launch."""
    path = os.path.join(ROOT, "mixed_precision_tiled_amd", "libmfma_probe.so")
    if not os.path.exists(path):
        build_module().build()
    lib = ctypes.CDLL(path)
    f = lib.mfma_probe_launch
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(2, 1, 1, 0, 16, 16, None) == -1     # unknown kind
    assert f(0, 0, 1, 0, 16, 16, None) == -1     # no workgroups
    assert f(0, 1, 1, 0, None, 16, None) == -1   # no sink


def test_exp8_table_validation(lamp):
    # a null table is refused before anything reaches the GPU
    f = _lib(lamp).lamp_exp8_table
    assert f(None, None) == 1
    assert "table" in lamp.lamp_last_error()
