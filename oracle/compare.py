"""Acceptance rules for 16-bit outputs (oracle side; test infrastructure only).

|O_gpu - O_ref| <= max(atol, ulp_dtype(O_ref)) + extra, element by element,
where atol is 2e-3 for fp16 outputs and 1e-2 for bf16 outputs, and extra is
the widening for what the weights may move by within the logit error bounds
(on the LampAttention paths: e4m3 rounding flips, e4m3 weights at a running
maximum that may be off, fp32 weights' exponent errors; on the TileMix path:
the exponents' errors, ``attention.tilemix_bounds``).  One unit in the last place of the output dtype
covers the final rounding of O itself when |O| is large enough that half an
ulp exceeds atol (bf16: |O| >= 2).

``check`` applies the rule to one output; ``check_lamp`` applies it to the
branches of a LampAttention emulation (flag decisions within the GPU error
bound of the threshold are evaluated both ways by the oracle, and the GPU's
flags pick the branch).
"""
import numpy as np

ATOL = {"f16": 2e-3, "bf16": 1e-2}
MANT = {"f16": 10, "bf16": 7}


def ulp(x, dtype):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - MANT[dtype])


def tolerance(O_ref, dtype, extra=None):
    """max(atol, ulp(O_ref)) plus the widening extra (per element, or per
    row)."""
    tol = np.maximum(ATOL[dtype], ulp(O_ref, dtype))
    if extra is not None:
        e = np.asarray(extra)
        tol = tol + (e if e.ndim == np.ndim(O_ref) else e[..., None])
    return tol


def check(O_gpu, O_ref, dtype, extra=None, exclude_rows=None):
    """Returns a stats dict; stats['ok'] is the pass/fail decision."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    err = np.abs(O_gpu - O_ref)
    tol = tolerance(O_ref, dtype, extra)
    bad = err > tol
    if exclude_rows is not None:
        bad = bad & ~np.asarray(exclude_rows)[..., None]
    finite = np.isfinite(O_gpu).all()
    n_ulp = int(((err > ATOL[dtype]) & ~bad).sum())
    return dict(ok=bool(finite and not bad.any()), max_err=float(err.max()) if err.size else 0.0,
                n_bad=int(bad.sum()), n_ulp_branch=n_ulp, finite=bool(finite))


def _close(O_gpu, O_ref, dtype, extra):
    err = np.abs(np.asarray(O_gpu, dtype=np.float64) - O_ref)
    tol = np.maximum(ATOL[dtype], ulp(O_ref, dtype)) + extra
    return err, err <= tol


def check_lamp(res, O_gpu, dtype, flags_gpu=None, lse_gpu=None, keep=None):
    """Acceptance of a GPU result against a LampResult of the oracle.

    For each sub-block the oracle holds one branch per outcome of the flag
    decisions that lie within the GPU error bound of the threshold.  The GPU's
    own flags of the sub-block pick the branch with the same flags (none
    matching is a flag mismatch); without GPU flags any branch may match.  The
    rows of the sub-block must then lie within the tolerance (widened by the
    branch's bound on what its weights may move by) of that branch's O, and the LSE
    within the branch's LSE bound.  O_gpu, lse_gpu: rows in the order of the
    oracle's rows; flags_gpu: [n_sb, n_kt] bool in the order of its
    sub-blocks; keep: [R] bool, rows to compare (padding rows of a
    variable-length batch are not).  Returns a stats dict; stats['ok'] is the
    decision."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    if keep is not None:
        O_gpu = np.where(np.asarray(keep)[:, None], O_gpu, 0.0)
    st = dict(ok=True, max_err=0.0, n_bad=0, n_ulp_branch=0, flag_mismatch=0, lse_bad=0,
              n_subblocks=len(res.branches), n_split=int(res.flag_dontcare.sum()),
              n_branches=sum(len(b) for b in res.branches), n_nonprimary=0,
              unresolved=int(res.unresolved.sum()), excluded_rows=0,
              max_extra=float(res.extra_tol.max()) if res.extra_tol.size else 0.0,
              n_elems=0, n_wide=0, finite=bool(np.isfinite(O_gpu).all()))
    if not st["finite"]:
        st["ok"] = False
    for i, (brs, idx) in enumerate(zip(res.branches, res.row_branch)):
        if flags_gpu is not None:
            cand = [j for j, br in enumerate(brs) if (br.flags == flags_gpu[i]).all()]
            if not cand:
                st["flag_mismatch"] += 1
                st["ok"] = False
                continue
        else:
            cand = list(range(len(brs)))
        kp = np.ones(len(idx), dtype=bool) if keep is None else np.asarray(keep)[idx]
        best = None
        for j in cand:
            br = brs[j]
            err, good = _close(O_gpu[idx], br.O, dtype, br.extra_tol)
            err, good = np.where(kp[:, None], err, 0.0), good | ~kp[:, None]
            lse_ok = True
            if lse_gpu is not None:
                lg = np.asarray(lse_gpu, dtype=np.float64)[idx][kp]
                none = np.isneginf(br.lse[kp])
                lr, lt = br.lse[kp], br.lse_tol[kp]
                lse_ok = bool(np.isneginf(lg[none]).all() and np.isfinite(lg[~none]).all() and
                              (np.abs(lg[~none] - lr[~none]) <= lt[~none]).all())
            if good.all() and lse_ok:
                best = (j, err, good, lse_ok)
                break
            if best is None:
                best = (j, err, good, lse_ok)
        j, err, good, lse_ok = best
        if j != 0:
            st["n_nonprimary"] += 1
        # elements whose tolerance the widening takes beyond atol
        st["n_elems"] += int(kp.sum()) * err.shape[1]
        st["n_wide"] += int(((brs[j].extra_tol > ATOL[dtype]) & kp[:, None]).sum())
        st["max_err"] = max(st["max_err"], float(err.max()) if err.size else 0.0)
        st["n_bad"] += int((~good).sum())
        st["n_ulp_branch"] += int(((err > ATOL[dtype]) & good).sum())
        if not lse_ok:
            st["lse_bad"] += 1
        if not good.all() or not lse_ok:
            st["ok"] = False
    if st["unresolved"]:
        st["ok"] = False
    return st
