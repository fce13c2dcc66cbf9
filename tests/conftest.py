import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _build_library_if_missing():
    lib = os.path.join(ROOT, "chunked_matmul_reduce_amd", "libmmar.so")
    if os.path.exists(lib):
        return
    path = os.path.join(ROOT, "chunked_matmul_reduce_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_mmar_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: longer CPU test")
    _build_library_if_missing()
