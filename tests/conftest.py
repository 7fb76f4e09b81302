import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def build_module():
    """mla_latent_kv_partial_amd/build.py, loaded by path (importing the
    package loads the library that it builds)."""
    spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(ROOT, "mla_latent_kv_partial_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # A fresh checkout has no library yet; hipcc cross-compiles it without a GPU.
    B = build_module()
    if not os.path.exists(B.LIB):
        B.build()
