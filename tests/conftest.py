import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.hookimpl(trylast=True)  # after -m has deselected
def pytest_collection_modifyitems(session, config, items):
    """A session that selects GPU tests must have the library loaded and a gfx950 device
    visible: a missing library or GPU fails the session instead of turning every GPU test
    into a skip."""
    if not any(item.get_closest_marker("gpu") for item in items):
        return
    import torch

    import streaming_kv_cache_write_amd as skv
    if not torch.cuda.is_available():
        raise pytest.UsageError("GPU tests selected but no GPU is visible to torch")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    if not arch.startswith("gfx950"):
        raise pytest.UsageError(f"GPU tests need gfx950 (found {arch})")
    print(f"\nGPU tests on {arch} with {skv.LIB_PATH}", flush=True)
