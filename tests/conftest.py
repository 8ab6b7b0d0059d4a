import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU for the oracle)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once; tests marked gpu use it."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import gated_delta_rule_14_amd as gdn
    gdn.load()          # raises if the HIP library is missing: no fallback
    return gdn


@pytest.fixture(autouse=True)
def _gdn_debug(request, monkeypatch):
    """GPU tests run with GDN_DEBUG set: after every prefill call the binding
    reads the single-pass kernel's synchronisation status word (and, for
    packed input, the check of cu_seqlens) and raises if it is set."""
    if request.node.get_closest_marker("gpu"):
        monkeypatch.setenv("GDN_DEBUG", "1")
