import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: exhaustive sweeps; run with IQK_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("IQK_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep; set IQK_SLOW=1 to run")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


def _ensure_built():
    """Build the HIP library in-tree only when nothing is built yet."""
    lib = os.path.join(ROOT, "dequant_iqk_moe_amd", "libiqk.so")
    if not os.path.exists(lib):
        # build.py by path: importing the package itself needs the library
        import importlib.util
        spec = importlib.util.spec_from_file_location("_iqk_build", os.path.join(ROOT, "dequant_iqk_moe_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
