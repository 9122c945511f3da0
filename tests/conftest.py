import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not _has_gpu():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")


def pytest_runtest_setup(item):
    # Name the case before any GPU work so a fault that ends the box still
    # leaves the test id in the log.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity statistics the GPU cases recorded (plain 1e-3
    relative share of the scores, top-k rows required to match exactly and
    exempted, largest errors), one line per case, also in quiet runs."""
    import json
    try:
        from tests.parity import STATS
    except Exception:
        return
    if not STATS:
        return
    terminalreporter.write_sep("-", "parity statistics")
    for st in STATS:
        terminalreporter.write_line(json.dumps({k: (round(v, 6) if isinstance(v, float) else v)
                                                for k, v in st.items()}))
