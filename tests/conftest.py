import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


_CONFIG = None


def pytest_configure(config):
    global _CONFIG
    _CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def progress(*a):
    """Print a progress line past pytest's output capture, so that a long
    GPU test shows it is alive even under -q."""
    cm = _CONFIG.pluginmanager.getplugin("capturemanager") if _CONFIG is not None else None
    if cm is not None:
        with cm.global_and_fixture_disabled():
            print(*a, flush=True)
    else:
        print(*a, flush=True)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
