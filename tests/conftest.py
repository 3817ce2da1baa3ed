import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload")
    config.addinivalue_line("markers", "device_check_flags: feeds the kernels bad device data "
                            "on purpose (page ids outside the pool, out-of-range indices, NaN)")


@pytest.fixture(autouse=True)
def _device_checks_clean(request):
    """With DSA_DEVICE_CHECKS=1 every GPU test runs on libdsa_checked.so: after
    each test the device check word must be clear, unless the test is marked
    as feeding bad data on purpose (no false positives across the suite)."""
    yield
    if os.environ.get("DSA_DEVICE_CHECKS", "0") in ("", "0") or "gpu" not in request.keywords:
        return
    import torch
    if not torch.cuda.is_available():
        return
    from sparse_attention_02_amd import binding
    flags = binding.dsa_device_check()
    if request.node.get_closest_marker("device_check_flags") is None:
        assert flags == 0, f"device checks flagged 0x{flags:x} in a test with clean inputs"


def pytest_terminal_summary(terminalreporter):
    """The achieved error of every parity check beside its bar (worst case per
    test and quantity), so the margins show in passing runs."""
    mod = sys.modules.get("gpu_common")
    rows = getattr(mod, "MARGINS", None) if mod else None
    if not rows:
        return
    worst = {}
    for test, quantity, achieved, bar in rows:
        key = (test, quantity)
        if key not in worst or achieved > worst[key][0]:
            worst[key] = (achieved, bar)
    terminalreporter.section("parity margins (achieved vs bar)")
    for (test, quantity), (achieved, bar) in sorted(worst.items()):
        terminalreporter.line(f"{achieved:10.3e} / {bar:8.1e}  {quantity:34s} {test}")
