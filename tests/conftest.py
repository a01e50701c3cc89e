import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # torch first: its bundled HIP runtime must be the process's one (the
    # library's loader does the same; this covers tests that load the
    # library by other routes)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    from tests import helpers
    helpers.CAPMAN = config.pluginmanager.getplugin("capturemanager")
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")
