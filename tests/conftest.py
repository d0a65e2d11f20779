import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU run (oracle at large sizes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests fail loudly if it or the GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from spatially_sharded_conv_amd import _lib
    return _lib.load()


def pytest_terminal_summary(terminalreporter):
    """Parity figures the tests recorded (max-abs and rel-L2 against the bar), one line each."""
    from tests._util import PARITY_LOG
    if not PARITY_LOG:
        return
    terminalreporter.section("parity (measured / bar)")
    for what, ma, rl, ba, br in PARITY_LOG:
        bars = f" / {ba:g}, {br:g}" if ba is not None else ""
        terminalreporter.write_line(f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}{bars}")
