import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly on a machine with a GPU if the library is missing; on a host
    # without a GPU they are skipped (the CPU suite runs with -m "not gpu").
    try:
        import torch

        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def plan_override():
    """Set launch-plan overrides through the library (fql_set_plan_override) for
    one test; every override the test set is removed afterwards."""
    import fp8_quantized_linear_amd as fql

    used = set()

    def set_override(spec, which="nvfp4"):
        fql.set_plan_override(spec, which)
        used.add(which)

    yield set_override
    for which in used:
        fql.set_plan_override(None, which)
