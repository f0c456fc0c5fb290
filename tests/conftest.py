"""Shared pytest setup: the `gpu` marker, import paths, and a build of a
fresh checkout."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity against the CPU oracle")
    import __graft_entry__
    __graft_entry__.ensure_built()       # a fresh checkout is built first


def pytest_runtest_teardown(item, nextitem):
    """After each GPU test, hand the device memory torch has cached back, so
    the full-size tests (60-175 GB each) start from an empty pool."""
    if item.get_closest_marker("gpu") is None:
        return
    import gc
    gc.collect()
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
