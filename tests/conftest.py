import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle cases")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line with the LampAttention acceptance counts of the GPU parity
    tests (flag decisions within the error bound evaluated both ways, flag
    mismatches, rows excluded, the widening for what the weights may move by
    within the logit bounds, and how many elements it takes beyond atol)."""
    try:
        from gpu_util import LAMP_REPORT, PATH_REPORT
    except Exception:  # pragma: no cover
        return
    for path, r in sorted(PATH_REPORT.items()):
        terminalreporter.write_line(
            "{} acceptance: elements {} | max |O - oracle| {:.2e} ({}) | elements beyond atol {} | "
            "elements widened beyond atol {} | max widening {:.2e} ({}) | max LSE deviation {:.2e} "
            "({:.2f} of its bound)".format(
                path, r.get("n_elems", 0), r.get("max_err", 0.0), r.get("max_err_test", "-"),
                r.get("n_over_atol", 0), r.get("n_wide", 0), r.get("max_extra", 0.0),
                r.get("max_extra_test", "-"), r.get("max_lse_dev", 0.0), r.get("max_lse_ratio", 0.0)))
    if LAMP_REPORT:
        r = LAMP_REPORT
        terminalreporter.write_line(
            "lamp acceptance: sub-blocks {} | decisions within the error bound (both ways) {} | "
            "non-primary branches picked {} | flag mismatches {} | branch-cap overflows {} | "
            "rows excluded {} | max widening {:.2e} | elements widened beyond atol {} of {} | "
            "max |O - oracle| {:.2e}".format(
                r.get("n_subblocks", 0), r.get("n_split", 0), r.get("n_nonprimary", 0),
                r.get("flag_mismatch", 0), r.get("unresolved", 0), r.get("excluded_rows", 0),
                r.get("max_extra", 0.0), r.get("n_wide", 0), r.get("n_elems", 0),
                r.get("max_err", 0.0)))
        terminalreporter.write_line(
            "lamp largest widening in {}; largest |O - oracle| in {}".format(
                r.get("max_extra_test", "-"), r.get("max_err_test", "-")))
