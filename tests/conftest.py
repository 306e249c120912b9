import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X) and the built HIP library")


def _ensure_library():
    """Build libpkv.so if it is missing (never rebuilds an existing one). The build script is
    loaded by path: importing the package itself would try to load the library."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "pkv_build", os.path.join(ROOT, "paged_kv_cache_459_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ensure_built()


_ensure_library()
