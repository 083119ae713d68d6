import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size sampled checks)")


@pytest.fixture(scope="session")
def e4b():
    """The binding, with libe4b.so built in-tree first if it is missing."""
    lib = os.path.join(ROOT, "bit_quantized_mixture_amd", "libe4b.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_e4b_build", os.path.join(ROOT, "bit_quantized_mixture_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import bit_quantized_mixture_amd as m
    return m
