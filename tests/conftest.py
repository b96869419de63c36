import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU-side test")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def _ensure_built():
    """Build the three libraries if a fresh checkout has none (build() is the
    normal route; this only covers a missing .so)."""
    import importlib
    for mod, path in (("workload", "workload/libworkload.so"), ("oracle", "oracle/liboracle.so")):
        if not os.path.exists(os.path.join(ROOT, path)):
            importlib.import_module(mod).build()
    if not os.path.exists(os.path.join(ROOT, "resident_expert_caching_amd", "libmoe_spark.so")):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "resident_expert_caching_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()


_ensure_built()
