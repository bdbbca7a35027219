"""Acceptance rule for 16-bit outputs (oracle side; test infrastructure only).

|O_gpu - O_ref| <= max(atol, ulp_dtype(O_ref)) + extra_row, element by
element, where atol is 2e-3 for fp16 outputs and 1e-2 for bf16 outputs, and
extra_row is the per-row widening for possible 8-bit rounding flips (zero on
the TileMix path).  One unit in the last place of the output dtype covers the
final rounding of O itself when |O| is large enough that half an ulp exceeds
atol (bf16: |O| >= 2).
"""
import numpy as np

ATOL = {"f16": 2e-3, "bf16": 1e-2}
MANT = {"f16": 10, "bf16": 7}


def ulp(x, dtype):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - MANT[dtype])


def tolerance(O_ref, dtype, extra_row=None):
    tol = np.maximum(ATOL[dtype], ulp(O_ref, dtype))
    if extra_row is not None:
        tol = tol + np.asarray(extra_row)[..., None]
    return tol


def check(O_gpu, O_ref, dtype, extra_row=None, exclude_rows=None):
    """Returns a stats dict; stats['ok'] is the pass/fail decision."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    err = np.abs(O_gpu - O_ref)
    tol = tolerance(O_ref, dtype, extra_row)
    bad = err > tol
    if exclude_rows is not None:
        bad = bad & ~np.asarray(exclude_rows)[..., None]
    finite = np.isfinite(O_gpu).all()
    n_ulp = int(((err > ATOL[dtype]) & ~bad).sum())
    return dict(ok=bool(finite and not bad.any()), max_err=float(err.max()) if err.size else 0.0,
                n_bad=int(bad.sum()), n_ulp_branch=n_ulp, finite=bool(finite))
