"""Mixed-precision tiled attention prefill for AMD MI355X (gfx950).

The compute lives in ``liblamp.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/lamp.h``); ``lamp`` is a thin ctypes binding with the
same entry-point names.  Importing this package loads the library and fails
loudly if it has not been built.
"""
from .lamp import (  # noqa: F401
    LAMP_BF16, LAMP_E4M3, LAMP_F16, LAMP_I8, LAMP_MODE_ADAPTIVE, LAMP_MODE_MASK, LampError,
    lamp_abi_version, lamp_attn_fwd, lamp_build_mask, lamp_build_mask_per_head,
    lamp_build_mask_template, lamp_last_error,
    lamp_quantize_blocks, lamp_quantize_v_tiles, lamp_decode_fwd, lamp_decode_workspace_bytes,
    lamp_decode_fwd_noalloc, LAMP_DECODE_SCRATCH_BYTES, lamp_exp8_table,
    lamp_status_string, library_path, exported_symbols,
)
