import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, takes tens of seconds")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _parity_test_name(request):
    import parity_stats
    parity_stats.CURRENT = request.node.nodeid
    yield


def pytest_terminal_summary(terminalreporter):
    try:
        import parity_stats
    except ImportError:
        return
    if not parity_stats.STATS:
        return
    tr = terminalreporter
    tr.section("fp32 parity against the oracle: worst error / tolerance, plain max relative error")
    worst_r = max(r for r, _ in parity_stats.STATS.values())
    worst_p = max(p for _, p in parity_stats.STATS.values())
    for name, (r, p) in sorted(parity_stats.STATS.items()):
        tr.write_line(f"{r:9.3f}  {p:10.3e}  {name}")
    tr.write_line(f"overall: worst error / tolerance {worst_r:.3f}; plain max relative error {worst_p:.3e} "
                  f"over {len(parity_stats.STATS)} tests")
