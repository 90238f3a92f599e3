import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # When GPU tests are asked for explicitly (-m gpu) they must run and fail
    # loudly on a machine without a usable GPU, never skip.
    if _gpu_available() or config.getoption("markexpr", "").strip() == "gpu":
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # Full-size parity: every entry of C compared with the oracle; one line
    # per comparison with the worst error ratio found.
    mod = sys.modules.get("gpu_util")
    rows = getattr(mod, "FULL_SIZE_RESULTS", None) if mod is not None else None
    if not rows:
        return
    terminalreporter.write_sep("-", "full-size parity (every entry of C against the oracle)")
    for test, entries, err in rows:
        terminalreporter.write_line(f"{test}: {entries} entries, max error ratio {err:.3e}")
