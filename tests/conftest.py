import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them loudly rather than fail
    # on CPU-only machines when they are selected explicitly.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity margins of the session: max row and state error per checked
    case against its tolerance."""
    try:
        from tests.parity import MARGINS
    except Exception:  # pragma: no cover
        return
    if not MARGINS:
        return
    tr = terminalreporter
    tr.section("parity margins (max relative error: output rows, final states; tolerance)")
    for label, eo, es, tol in MARGINS:
        worst = max(eo, es)
        tr.write_line(f"{label:58s} o {eo:.2e}  state {es:.2e}  tol {tol:.0e}  "
                      f"({worst / tol * 100:5.1f}% of tol)")
