import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU in this container")
    import torch
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Print the worst errors of the passing parity checks (row relative error,
    largest absolute error, largest error over its row's max |ref|)."""
    parity = sys.modules.get("parity")
    worst = getattr(parity, "WORST", None)
    if not worst:
        return
    terminalreporter.section("worst parity errors against the oracle")
    for what in sorted(worst):
        terminalreporter.write_line(
            f"{what:<60s} " + "  ".join(f"{k} {v:.3e}" for k, v in sorted(worst[what].items())))
